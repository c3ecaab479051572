// Internal declarations shared by the host library and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gift.h"

namespace gift {

constexpr int kBlock = 128;          // per-block scaling tile (128 x 128)
constexpr int kMaxRank = 64;         // k + p <= 64 for the small dense solvers
constexpr int kProjChunk = 512;      // columns per partial in the projection X U

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Offsets (bytes) of the regions of one layer's device state.
struct StateLayout {
  size_t S_A = 0, A = 0, S_G = 0, G = 0, U = 0, coef = 0, tinv_a = 0, t_a = 0, lg_inv = 0, lg = 0,
         flags = 0, total = 0;
  // fused rank-k path: packed U operands, tagged projection partials and
  // amax words
  size_t ub = 0, ua = 0, xpub = 0, apub = 0;
  // statistics: grow-only flags of the workgroups that share an output tile
  size_t ssync = 0;
};

// Fused rank-k kernel geometry (48 x 768 tiles, 8 waves).
constexpr int kFusedTR = 48, kFusedTC = 768;
// Packed U_k operands per 32-column block and operand order: 2 groups x 2
// f16 pieces x 64 lanes x 16 bytes.
constexpr int kUPackBytes = 2 * 2 * 64 * 16;
// Per-tensor amax words of the fused encode: kAmaxCopies copies of the
// [tiles] array, each on its own 4 KiB page(s), so that no single memory
// channel serves every workgroup's reads.
constexpr int kAmaxCopies = 16;
__host__ __device__ inline int amax_copy_stride(int tiles) { return (tiles + 511) / 512 * 512; }

// Arguments of the fused encode (mode 0) / decode-reduce (mode 1) kernel.
struct FusedArgs {
  int mode, m, d, CG, fmt, scaling, R;
  int lr;                     // 1: rank-k transform; 0: Euclidean (T_A = I)
  unsigned epoch;
  const float* W;
  int64_t ldw;
  const uint4* ub;
  const uint4* ua;
  const float* coef;
  unsigned long long* xpub;   // state: tagged projection partials [tiles][48][32], then sums [row groups][48][32]
  unsigned long long* apub;   // state: [tiles][16] epoch-tagged amax words, then kAmaxCopies x [tiles]
  unsigned* flags;
  const float* amax_in;
  float* amax_out;
  uint8_t* codes;
  float* scales;
  uint8_t* bscales;           // FP4 encode: E4M3 block scale codes [m][d / 16]
  float* tscale;              // FP4 encode: the tensor scale [1]
  float* whitened;
  float* resid;               // error feedback: fp32 [m][d] residual, read and rewritten (NULL: none)
  const uint8_t* qcodes;
  int64_t code_stride;
  const float* qscales;
  int64_t scale_stride;
  const uint8_t* qbscales;    // FP4 decode: block scale codes of replica r at r * bscale_stride
  int64_t bscale_stride;
  const float* qtscales;      // FP4 decode: tensor scales [R]
  float invR;
  float* out;
  int64_t ldo;
};
// Persistent launch of a fused kernel; the caller has checked that the grid
// fits the kernels' occupancy (fused_resident_groups).
hipError_t launch_fused(const FusedArgs& args, int grid, hipStream_t s);
// Workgroups of the fused kernels the current device holds at once (0: unknown).
int fused_resident_groups();
// Grouped launch of several rank-k layers (table: device array of n
// FusedArgs, epochs by value).
constexpr int kMaxGroup = 32;
struct GroupEpochs {
  unsigned v[kMaxGroup];
};
hipError_t launch_group(const FusedArgs* table, int n, const GroupEpochs& ep, int decode, int fmt, int scaling, int R,
                        int grid, hipStream_t s);
// Upper bound on co-resident workgroups that the persistent kernels may
// assume (gift_set_max_resident; 0 = none).
int max_resident_cap();
// Orders a persistent launch on stream s after the previous persistent
// launch of the library on this device, when that one went to another
// stream (see gift_api.hip).
hipError_t order_persistent(hipStream_t s);
hipError_t launch_pack_u(const float* U, int d, void* ub, void* ua, hipStream_t s);

// Refresh products Y = A X (A symmetric d x d): each workgroup takes 256
// columns of A and a range of its rows; the partial sums of the ranges are
// added in a fixed order.  At most 512 workgroups (two per compute unit, the
// fp64 kernel's occupancy), so that they run in one even round.
constexpr int kAqCols = 256;
__host__ __device__ inline int aq_rows_per_split(int d) {
  const int cb = (int)cdiv(d, kAqCols);
  int splits = 512 / cb;   // at most two workgroups per compute unit: one even round
  const int max_splits = (int)cdiv(d, 64);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return (int)cdiv(cdiv(d, splits), 32) * 32;
}
__host__ __device__ inline int aq_splits(int d) { return (int)cdiv(d, aq_rows_per_split(d)); }
// The fp32 products: workgroups of 64 columns, row ranges (multiples of 64
// rows) split so that there are about 768 workgroups (three per compute unit).
__host__ __device__ inline int aq32_rows_per_split(int d) {
  const int cb = (int)cdiv(d, 64);
  int splits = (int)cdiv(768, cb);
  const int max_splits = (int)cdiv(d, 64);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return (int)cdiv(cdiv(d, splits), 64) * 64;
}
__host__ __device__ inline int aq32_splits(int d) { return (int)cdiv(d, aq32_rows_per_split(d)); }
constexpr int kGramRows = 64;   // rows per partial of the l x l Gram products

// Offsets (bytes) inside the per-call workspace.  Regions overlap between
// calls of different kinds (encode / decode / refresh never run at once on
// one workspace).
struct WorkLayout {
  // encode / decode
  size_t tile = 0;      // fp32 [m][d]: whitened tensor (encode) or reduced U (decode)
  size_t tmp = 0;       // fp32 [m][d]: second buffer (two-sided)
  size_t ppart = 0;     // fp64 [nchunk][m][k]: projection partials
  size_t pc = 0;        // fp32 [m][k]: their sum times the coefficients
  size_t amax = 0;      // uint32 [nblk]
  // refresh
  size_t Y = 0, Q = 0, Z = 0;   // fp64 [d][l]
  size_t small = 0;             // fp64 scratch for the l x l solvers
  size_t gpart = 0;             // fp64 [nchunk][l][l]
  size_t apart = 0;             // partials of A X: fp64 [splits][d][l] or fp32 [splits32][d][l]
  size_t chol = 0;              // fp64 [n][n] (Cholesky variants)
  size_t chol2 = 0;             // fp64 [n][n]
  // statistics of a GIFT_LAYER_TRANSIENT_STATS layer: the window sum S,
  // fp32 [n][n] (aliases the areas above: no other call runs meanwhile)
  size_t stats = 0;
  size_t total = 0;
};

struct Dims {
  int m, d, k, l;
};

StateLayout state_layout(const gift_layer_desc& desc);
WorkLayout work_layout(const gift_layer_desc& desc);

// ---- kernel launchers (each returns hipGetLastError() of its launches) ----
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, size_t n, hipStream_t s);

// amax of |x + resid| over a [m][ld] fp32 tensor into uint32 slots (bit
// patterns); resid: NULL or fp32 [m][d] (error feedback).
hipError_t launch_amax(const float* x, int64_t ld, int m, int d, int scaling, const float* resid,
                       uint32_t* slots, hipStream_t s);
// quantise u = x [m][ld] (+ resid) with amax slots (or amax_in) -> codes,
// scales, amax_out; with resid also resid <- u - s dec(code).
hipError_t launch_quantize(const float* x, int64_t ld, int m, int d, int fmt, int scaling,
                           const uint32_t* slots, const float* amax_in, float* amax_out,
                           uint8_t* codes, float* scales, float* resid, uint32_t* flags, hipStream_t s);
// FP4 (E2M1, 16-element row blocks with E4M3 scales, fp32 tensor scale):
// quantise u = x (+ resid) with the tensor amax in slot[0] (or amax_in) ->
// codes [m][d/2], bscales [m][d/16], tscale[0], amax_out[0]; with resid
// also resid <- u - S_b dec(code).  d a multiple of 16.
hipError_t launch_quantize_fp4(const float* x, int64_t ld, int m, int d, const uint32_t* slot, const float* amax_in,
                               float* amax_out, uint8_t* codes, uint8_t* bscales, float* tscale, float* resid,
                               uint32_t* flags, hipStream_t s);
// U = (1/R) sum_r S_{b,r} dec(q_r) of R FP4 payloads -> fp32 [m][ldo]
hipError_t launch_dequant_sum_fp4(const uint8_t* codes, int64_t code_stride, const uint8_t* bscales,
                                  int64_t bscale_stride, const float* tscales, int R, int m, int d, float* out,
                                  int64_t ldo, hipStream_t s);
// Flat gradient buckets (Euclidean codec over many tensors, one launch per
// phase).  Prefix tables in device memory, n + 1 entries each.
struct BucketTable {
  const int64_t* chunk_start;   // first 4096-element chunk of each tensor
  const int64_t* elem_off;      // first element of each tensor in the flat buffer
  const int64_t* scale_off;     // first scale of each tensor
  int n;
  int64_t chunks;
  uint32_t* flags;
};
hipError_t launch_bucket_amax(const BucketTable& t, const float* g, int block512, uint32_t* slots, int cus,
                              hipStream_t s);
hipError_t launch_bucket_quantize(const BucketTable& t, const float* g, int fmt, int block512, const uint32_t* slots,
                                  const float* amax_in, float* amax_out, uint8_t* codes, float* scales, int cus,
                                  hipStream_t s);
hipError_t launch_bucket_dequant_sum(const BucketTable& t, const uint8_t* codes, int64_t code_stride,
                                     const float* scales, int64_t scale_stride, int R, int fmt, int block512,
                                     float* out, int cus, hipStream_t s);

// U = (1/R) sum_r s_r dec(q_r) -> fp32 [m][ldo]
hipError_t launch_dequant_sum(const uint8_t* codes, int64_t code_stride, const float* scales,
                              int64_t scale_stride, int R, int m, int d, int fmt, int scaling,
                              float* out, int64_t ldo, hipStream_t s);

// Low-rank transform pieces: partials of X U, then out = alpha X + (P c) U^T.
hipError_t launch_lr_project(const float* x, int64_t ldx, int m, int d, const float* U, int k,
                             double* ppart, hipStream_t s);
// (ppart is first reduced into pc: fp32 [m][32] workspace)
hipError_t launch_lr_apply(const float* x, int64_t ldx, int m, int d, const float* U, int k,
                           const double* ppart, float* pc, const float* coef, int which, float* out,
                           int64_t ldo, int scaling, uint32_t* amax_slots, hipStream_t s);
// Column scaling out = x * v[j] (diagonal transform), with optional amax.
hipError_t launch_diag_apply(const float* x, int64_t ldx, int m, int d, const float* v, float* out,
                             int64_t ldo, int scaling, uint32_t* amax_slots, hipStream_t s);

// Statistics.
// S += x^T x over T tokens (lower-triangle tiles).  The bf16 matrix-core
// path splits the (tile, stage) work evenly over `cus` resident workgroups;
// the workgroups sharing a tile add into S in a fixed order, handing over
// through `sync` (grow-only, one word per workgroup) at `epoch`.
constexpr int kStatsMaxGroups = 1024;
// overwrite: the call opens a window, so its sums are stored, not added
hipError_t launch_stats(const void* x, int dtype, int64_t T, int64_t ld, int n, float* S, unsigned* sync,
                        unsigned epoch, uint32_t* flags, int cus, bool overwrite, hipStream_t s);
// Workgroups of the matrix-core statistics kernel the current device holds
// at once (0: unknown).
int stats_resident_groups();
hipError_t launch_commit(const float* S, float* A, int n, double inv_count, float beta, int first,
                         hipStream_t s);

// Refresh (rank-k).
hipError_t launch_refresh_lowrank(const float* A, int d, int k, int l, int q, float damping_rel,
                                  const float* omega, float* U, float* coef, const WorkLayout& w,
                                  char* work, uint32_t* flags, hipStream_t s);
hipError_t launch_refresh_diag(const float* A, int d, float damping_rel, float* coef,
                               uint32_t* flags, hipStream_t s);
hipError_t launch_refresh_chol(const float* A, int n, float damping_rel, float* tinv, float* t,
                               int lower_out, double* work_a, double* work_b, uint32_t* flags,
                               hipStream_t s);

// Dense fp32 product with a triangular right/left operand:
//   out = x * M (M [d][d], upper triangular, right side)   side = 0
//   out = M * x (M [m][m], lower triangular, left side)    side = 1
hipError_t launch_trmm(const float* x, int64_t ldx, int m, int d, const float* M, int side,
                       float* out, int64_t ldo, hipStream_t s);

// Profiler: upper / lower boundary hits of one flattened gradient with its
// local per-tensor amax (already in slot).
hipError_t launch_hits(const float* g, int64_t n, int fmt, const uint32_t* slot,
                       unsigned long long* counts, hipStream_t s);
hipError_t launch_amax_out(const uint32_t* slots, float* amax_out, int64_t n, hipStream_t s);
hipError_t launch_amax_flat(const float* g, int64_t n, uint32_t* slot, hipStream_t s);

}  // namespace gift
