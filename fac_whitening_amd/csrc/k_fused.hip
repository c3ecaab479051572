// Fused rank-k encode and decode-reduce: one persistent kernel per direction.
//
// GIFT 阅读笔记, Algorithm 1 (geometry branch): U = W (L_A)^-T, Scale_loc, Q;
// AllReduceSum, Dequantize / N, W^ = U L_A^T; §简化二 Eq. (17) gives the rank-32
// factor, applied here in the form T = U_k diag(c) U_k^T + alpha I:
//     P = X U_k;   X~ = alpha X + (P diag(c)) U_k^T.
//
// Layout of the work (gfx950, wave64):
//  * One workgroup (8 waves) owns a 48 x 768 tile of the gradient and keeps it
//    in registers from the first load to the last store: the tensor is read
//    from HBM once.  A tile is 3 x 24 sub-tiles of 16 rows x 32 columns; wave
//    w owns the 3 column blocks w, w + 8, w + 16 in all 3 row blocks, so each
//    packed U operand a wave loads serves three sub-tiles.
//  * In a sub-tile, lane l holds row l % 16 and columns 4 g .. 4 g + 3 and
//    16 + 4 g .. 16 + 4 g + 3 (g = l / 16).  These eight values are the A
//    operand of the projection MFMA (16x16x32 f16, with U_k's rows permuted
//    the same way) and have the layout of the result (D layout) of the
//    reconstruction MFMA that computes the transposed sub-tile.
//  * Near-fp32 products from f16 MFMA: every row of an operand is scaled
//    by a power of two that puts its largest magnitude in [2^14, 2^15)
//    (U_k, whose entries are at most 1, by 2^14), split into two f16 pieces
//    (x = h + l, h the RNE f16 of x, l that of the residual), and the three
//    products l*h, h*l, h*h are accumulated in fp32; the sums are scaled
//    back exactly (ldexp).  Piece rounding and the dropped l*l term stay
//    below about 3 * 2^-22 of each product; entries far below their row's
//    largest lose relative precision in the f16 subnormal range, but never
//    more than about 2^-40 of that largest entry.
//  * P needs whole rows: the workgroups of one row group (same 48 rows)
//    publish their partial P as epoch-tagged words in the layer state; each
//    sums one slice of the partials in column-group order and publishes the
//    sums (a reduce-scatter), then every workgroup reads the row group's
//    sums.  A reader re-reads a word until it carries the call's tag, so
//    there is no barrier and no writer ever waits for its own stores.
//  * Encode: every workgroup publishes its tile's amax (per tensor, or per
//    128 x 128 block it touches) as 64-bit words tagged with the call's
//    epoch, and reads the words of the workgroups it depends on until all
//    carry the current epoch (an all-gather: no serial chain of atomics).
//  * Error feedback (Algorithm 1): the _ef encode reads the residual R in
//    the sub-tile layout of the registers, quantises W~ + R and rewrites R
//    with what the codes did not carry, in the same pass.
//  * Tags derive from per-direction call counters that only grow, so
//    nothing is reset between calls.  Every wait is bounded; a timeout sets
//    GIFT_FLAG_SPIN_TIMEOUT and the kernel still exits.
#include <type_traits>

#include "fp8_codec.hpp"
#include "gift_internal.hpp"

namespace gift {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ unsigned long long ld_dev64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the 64-bit word carries `epoch` in its upper half; return it.
// A wait that runs out sets the sticky flag and *bad (an LDS word).
__device__ __forceinline__ unsigned long long wait_tag(const unsigned long long* p, unsigned epoch,
                                                       unsigned* flags, int* bad) {
  unsigned long long v = ld_dev64(p);
  int spins = 0;
  while ((unsigned)(v >> 32) != epoch) {
    if (++spins > kSpinLimit) {
      atomicOr(flags, (unsigned)GIFT_FLAG_SPIN_TIMEOUT);
      *bad = 1;
      break;
    }
    v = ld_dev64(p);
  }
  return v;
}

__device__ __forceinline__ uint32_t absbits_f(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// x = h + l + (a residual below 2^-22 |x| in the f16 normal range): h the
// RNE f16 of x, l that of x - h (exact in fp32).
__device__ __forceinline__ void split2(float x, _Float16& h, _Float16& l) {
  h = (_Float16)x;
  l = (_Float16)(x - (float)h);
}

// Scale exponent of a row whose largest magnitude is mx: 2^e mx lies in
// [2^14, 2^15) (e clamped to [-126, 127]; 0 for a zero or non-finite mx,
// whose row then carries its zeros, Inf or NaN through unchanged).
__device__ __forceinline__ int row_exp(float mx) {
  const uint32_t b = __float_as_uint(mx);
  if (mx == 0.0f || (b & 0x7F800000u) == 0x7F800000u) return 0;
  const int ex = (int)((b >> 23) & 0xFF) - 127;   // floor(log2 mx); -127 for subnormal mx
  const int e = 14 - ex;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}
// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes holding
// one row of a sub-tile), with the VALU's row swaps (v_permlane32_swap
// exchanges the two 32-lane halves, v_permlane16_swap neighbouring 16-lane
// rows) instead of the LDS permute path.
__device__ __forceinline__ float rowmax4(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
// 4 x 4 transpose over the lanes of a row: with r[k] of lane l + 16 s
// called M[s][k] (l < 16), afterwards r[k] of lane l + 16 s holds M[k][s].
// Two stages of row swaps on register pairs: the 32-lane halves of (r0, r2)
// and (r1, r3), then the neighbouring 16-lane rows of (r0, r1) and (r2, r3).
__device__ __forceinline__ void quad_transpose(uint32_t (&r)[4]) {
  auto p = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
  auto q = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
  r[0] = p[0]; r[2] = p[1]; r[1] = q[0]; r[3] = q[1];
  p = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
  q = __builtin_amdgcn_permlane16_swap(r[2], r[3], false, false);
  r[0] = p[0]; r[1] = p[1]; r[2] = q[0]; r[3] = q[1];
}
// Maximum over the wave, in every lane: rotations inside each 16-lane row
// (DPP row_ror 8, 4, 2, 1), then the row swaps.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = umax32(p[0], p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return umax32(q[0], q[1]);
}
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }
constexpr int kUExp = 14;   // U_k's pieces are of 2^14 U_k

// Buffer resources: loads outside [0, bytes) return 0 and stores there are
// dropped, so edge tiles need no branches around their memory operations
// (branches would force a full wait on every outstanding load).
typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kOff = (int)0x80000000u;   // an offset past any buffer used here
// Cache policy of the payload streams: the encode's code stores and the
// decode's code loads are non-temporal (each byte is touched once per call;
// kept from the caches' normal replacement they leave the U_k operands and
// exchange words their place: 57.5 -> 52.3 us per unit at 1536 x 6144).  The
// rank-k decode's fp32 stores, whole 1 KB row segments, are non-temporal as
// well (50.3 -> 48.2 us per unit; while they were 64-byte pieces of 16 rows
// it measured slower).  The gradient loads stay normal (non-temporal there
// measured slower).  With error feedback the residual's stores are
// non-temporal too (it is next read a whole step later: 33.9 -> 33.0 us for
// the encode with its residual); its loads stay normal (measured slower).
constexpr int kNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, kRsrcWord3);
}

// Column of sub-tile position (g, j) in the permuted operand order.
__device__ __forceinline__ int perm_col(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// ---------------------------------------------------------------------------
// Packing of U_k into the MFMA operand orders (done once per refresh).
//   ub[cb][half][piece][lane]: projection B operand, lane l = (n, g):
//       slot j -> U[32 cb + perm_col(g, j)][n + 16 half]
//   ua[cb][grp][piece][lane]: reconstruction A operand:
//       slot j -> U[32 cb + 16 grp + n][8 g + j]
// Pieces: the two f16 pieces of 2^14 U (split2).
// ---------------------------------------------------------------------------
__global__ void k_pack_u(const float* __restrict__ U, int d, uint4* __restrict__ ub, uint4* __restrict__ ua) {
  const int ncb = (int)cdiv(d, 32);
  const int t = blockIdx.x * blockDim.x + threadIdx.x;   // (cb, which, half, lane)
  if (t >= ncb * 2 * 2 * 64) return;
  const int lane = t & 63, half = (t >> 6) & 1, which = (t >> 7) & 1, cb = t >> 8;
  const int n = lane & 15, g = lane >> 4;
  _Float16 h[8], l[8];
  for (int j = 0; j < 8; ++j) {
    int col, k;
    if (which == 0) {
      col = 32 * cb + perm_col(g, j);
      k = n + 16 * half;
    } else {
      col = 32 * cb + 16 * half + n;
      k = 8 * g + j;
    }
    const float v = col < d ? U[(int64_t)col * 32 + k] : 0.0f;
    split2(v * pow2f(kUExp), h[j], l[j]);
  }
  uint4* dst = (which == 0 ? ub : ua) + ((int64_t)(cb * 2 + half) * 2) * 64 + lane;
  dst[0] = __builtin_bit_cast(uint4, h);
  dst[64] = __builtin_bit_cast(uint4, l);
}

hipError_t launch_pack_u(const float* U, int d, void* ub, void* ua, hipStream_t s) {
  const int n = (int)cdiv(d, 32) * 256;
  hipLaunchKernelGGL(k_pack_u, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, U, d, static_cast<uint4*>(ub),
                     static_cast<uint4*>(ua));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The fused kernel
// ---------------------------------------------------------------------------

constexpr int TR = kFusedTR, TC = kFusedTC, NSUB = 9;
constexpr int kApub = 16;   // published amax words per workgroup
constexpr int kPipeDepth = 6;   // block-pipelined decode: units in flight per thread

// Decode the 4 codes of one 32-bit word.
template <int FMT>
__device__ __forceinline__ void dec4(uint32_t w, float* v) {
  float2v lo, hi;
  if constexpr (FMT == 0) {
    lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  } else {
    lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  }
  v[0] = lo[0];
  v[1] = lo[1];
  v[2] = hi[0];
  v[3] = hi[1];
}

// Decode the 8 E2M1 codes of one 32-bit word (the low nibble of each byte
// first) by the hardware conversion with a unit scale, which is exact.
__device__ __forceinline__ void dec8_fp4(uint32_t w, float* v) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
}

// Sub-tile i of wave w: column block cb = w + 8 (i / 3), row block rb = i % 3.
#define SUB_RB(i) ((i) % 3)
#define SUB_CB(i) (wave + 8 * ((i) / 3))

// Flat streaming of a tile: 8-element chunks, chunk q of the tile is row
// q / 96, columns 8 (q % 96) .. + 7; thread t owns chunks t + 512 j.
constexpr int kTilePad = TC + 4;            // LDS row stride of the staged tile (floats)
constexpr int kCPT = TR * TC / 8 / 512;     // chunks per thread (9)
constexpr int kMaxRFused = 64;              // replicas whose scales are staged in LDS

typedef int int32x2 __attribute__((ext_vector_type(2)));

// Decode streaming.  A replica's tile (48 x 768 codes = 36 KiB) is read as
// flat bytes f: thread t takes the 16-byte chunks f = 16 (t + 512 j), j < 4
// (the first 32 KiB), and the 8-byte chunk f = 32768 + 8 t (the rest); a
// 16-byte chunk never crosses a row (768 = 48 x 16).  Replicas past R are
// read through an empty buffer resource (no memory traffic, zeros), so every
// load is issued unconditionally and the loads of three replicas stay in
// flight.
constexpr int kDCPT = 4;                    // 16-byte chunks per thread
constexpr int kDTail = 32768;               // first byte of the 8-byte chunks

// One replica of one 16-row block (block-pipelined decode).
struct Unit {
  int32x4 v;    // 16 codes
  int32x2 t;    // 8 codes
};
// The same unit of an FP4 payload: 16 and 8 E2M1 codes and the E4M3 scale
// codes of the blocks they lie in.
struct Unit4 {
  int32x2 v;
  int t;
  uint32_t sa, sb;
};
template <bool B, class T, class F> struct pick_t { using type = T; };
template <class T, class F> struct pick_t<false, T, F> { using type = F; };

struct CodeBuf {
  int32x4 v[kDCPT];
  int32x2 t;
};

template <int FMT>
__device__ __forceinline__ void load_codes(const FusedArgs& a, int R, int r, const int* off, int offt, CodeBuf& dst) {
  const bool in = r < R;
  const auto q = make_rsrc(a.qcodes + (in ? (int64_t)r * a.code_stride : 0), in ? (int64_t)a.m * a.d : 0);
#pragma unroll
  for (int j = 0; j < kDCPT; ++j) dst.v[j] = __builtin_amdgcn_raw_buffer_load_b128(q, off[j], 0, kNT);
  dst.t = __builtin_amdgcn_raw_buffer_load_b64(q, offt, 0, kNT);
}

// hi[j] is false where a chunk's upper 8 codes lie past the row end (d is a
// multiple of 8, not always of 16): they belong to the next row and are
// replaced by zero codes.
// PT: one scale for the whole replica (`sr`), else the chunk's block scale
// from the LDS table `ssc_r`.
template <int FMT, bool PT>
__device__ __forceinline__ void accum_codes(float (*acc)[16], float* acct, const CodeBuf& c, const float* ssc_r,
                                            float sr, const int* sidx, int sidxt, const bool* hi, bool first) {
#pragma unroll
  for (int j = 0; j < kDCPT; ++j) {
    float v[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) dec4<FMT>((w < 2 || hi[j]) ? (uint32_t)c.v[j][w] : 0u, v + 4 * w);
    const float s = PT ? sr : ssc_r[sidx[j]];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[j][k] = first ? s * v[k] : acc[j][k] + s * v[k];
  }
  float v[8];
  dec4<FMT>((uint32_t)c.t[0], v);
  dec4<FMT>((uint32_t)c.t[1], v + 4);
  const float s = PT ? sr : ssc_r[sidxt];
#pragma unroll
  for (int k = 0; k < 8; ++k) acct[k] = first ? s * v[k] : acct[k] + s * v[k];
}

// Projection / reconstruction operands of one wave's three column blocks,
// [column block q][half or group][piece], read through a buffer resource
// so that blocks past the last column read zeros instead of memory.
struct UOps {
  half8 u[3][2][2];
};

__device__ __forceinline__ void load_uops(const uint4* packed, int d, int cbg0, UOps& o) {
  const auto rs = make_rsrc(packed, cdiv(d, 32) * kUPackBytes);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int off = ((((cbg0 + 8 * q) * 2 + h) * 2 + p) * 64 + lane) * 16;
        o.u[q][h][p] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      }
}

// Published projection words: (tag << 32) | float bits.  The tag makes each
// word self-validating, so a producer never waits for its own stores (on
// this architecture that wait would also wait for every load in flight) and
// readers need no separate barrier: they read until every word carries it.
__device__ __forceinline__ unsigned long long tagged(unsigned tag, float v) {
  return ((unsigned long long)tag << 32) | __float_as_uint(v);
}

constexpr int kXW = TR * 32;        // projection words per tile (1536)
constexpr int kFp4Pad = TC / 2 + 16;  // LDS row stride (bytes) of a tile's FP4 codes
// Output staging of the rank-k decode: two 48 x 256 fp32 slabs, row stride
// kStagePad floats; the first over the per-wave partials (8 x 3 x 16 x 33
// floats), the second after the gathered projection (48 x 33 floats).
constexpr int kStagePad = 260;
constexpr int kStageB = 8 * 3 * 16 * 33 + 48 * 33 + 80;
static_assert(TR * kStagePad <= 8 * 3 * 16 * 33, "first output slab over the partials");
static_assert(kStageB % 4 == 0 && kStageB + TR * kStagePad <= TR * kTilePad, "second output slab inside the tile");
constexpr int kXPT = kXW / 512;     // of them per thread (3)

// SC: the scaling (0 per tensor, 1 per block) as a compile-time constant
// (-1: read at run time).  Per tensor, each replica's scale is one
// uniform word read in the replica loop; per block the scales of the tile's
// blocks are staged in LDS first.
// RC > 0: the decode's replica count is a compile-time constant and the
// replica loop is unrolled, so every wait on a load names exactly the loads
// it needs (a runtime trip count rotates the buffers through different
// registers per iteration and the waits become full drains).
//
// Order of the memory operations (loads retire in order, so whatever is
// needed first is issued first): tile data, then the projection operands;
// the projection partials go out with atomic exchanges nobody waits for;
// the reconstruction operands are requested before the partner partials are
// read, so they arrive while the row group finishes its own partials.
// LR: the rank-k transform (false: the Euclidean codec, T_A = I: the same
// tile schedule, amax all-gather and quantiser without the projection,
// exchange and reconstruction).
template <int FMT, bool ENC, int RC, int SC, bool LR, bool EF = false>
__device__ __forceinline__ void fused_body(const FusedArgs& a, const int g, const int G, const unsigned epoch) {
  // The staged tile (fp32, padded rows); after it has been read into
  // registers the same memory holds the per-wave projection partials and the
  // projection of the tile rows, and finally the outgoing tile.
  __shared__ float smem[TR * kTilePad];
  __shared__ float ssc[kMaxRFused][12];   // decode scales of the tile's blocks
  __shared__ uint32_t blk[2][8];          // combined amax of the blocks of this tile
  __shared__ uint32_t wmax[16];
  __shared__ float srs[12];               // reciprocal scales of those blocks
  __shared__ float sss[12];               // and their scales (error feedback)
  __shared__ uint32_t sam[12];            // the amax bits they come from
  // Set when a bounded wait of this workgroup ran out (a partner never
  // published).  Its results are then poisoned, not left silently wrong:
  // the encode publishes a NaN amax (every code 0x7F and a NaN scale follow)
  // and writes 0x7F codes, the decode writes NaN.
  __shared__ int s_bad;
  // cp[rb][wave]: the row block's partials lie in the first 5.5 tile rows
  // (rb 0), the next 5.5 (rb 1), ...
  float (*cp)[8][16][33] = reinterpret_cast<float (*)[8][16][33]>(smem);
  float (*pf)[33] = reinterpret_cast<float (*)[33]>(smem + 8 * 3 * 16 * 33);
  // g: this workgroup's tile, G: the tiles of the layer (the grid of a
  // single-layer launch)
  const int rg = g / a.CG, cgi = g % a.CG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = rg * TR, col0 = cgi * TC;
  const int m = a.m, d = a.d;
  constexpr bool enc = ENC;
  const int nbd = (int)cdiv(d, kBlock);
  const int rb0 = row0 / kBlock, cb0 = col0 / kBlock;
  const int cbg0 = (col0 >> 5) + wave;   // this wave's first 32-column block
  const bool pts = SC >= 0 ? SC == 0 : a.scaling == 0;   // one scale for the whole tensor
  const unsigned tag = (epoch << 1) | (enc ? 0u : 1u);
  if (tid < 16) wmax[tid] = 0u;
  if (tid == 0) s_bad = 0;
  // PIPE: the projection of each 16-row block runs as soon as the block is
  // in (the rank-k encode; the rank-k decode with a compile-time replica
  // count of at most 8 streams the replicas block by block: at 16 the
  // unrolled stream no longer fits the registers, and its unit buffers
  // would go to scratch memory)
  constexpr bool PIPE = LR && (ENC || (RC > 0 && RC <= 8));

  float x[NSUB][8];
  bool live[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) live[q] = col0 + (wave + 8 * q) * 32 < d;
  UOps uo;
  // projection P = X U of row block rb (this wave's partial, 16 rows x 32),
  // in units of 2^(xe[rb] + 14) for row 16 rb + (lane % 16): the row's scale
  // exponent over this wave's three column blocks (the four lanes of a row
  // agree through the two shuffles), U_k's pieces carrying 2^14
  floatx4 pacc[3][2];
  int xe[3];
#pragma unroll
  for (int rb = 0; rb < 3; ++rb)
#pragma unroll
    for (int h = 0; h < 2; ++h) pacc[rb][h] = (floatx4){0.f, 0.f, 0.f, 0.f};
  auto project_rb = [&](int rb) {
    float mx = 0.f;
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (live[q]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(x[q * 3 + rb][j]));
      }
    xe[rb] = row_exp(rowmax4(mx));
    const float sc = pow2f(xe[rb]);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (!live[q]) continue;
      const int i = q * 3 + rb;
      half8 xh, xl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        _Float16 h, l;
        split2(x[i][j] * sc, h, l);
        xh[j] = h;
        xl[j] = l;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const half8* u = uo.u[q][h];
        floatx4 c = pacc[rb][h];
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, u[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, u[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, u[0], c, 0, 0, 0);
        pacc[rb][h] = c;
      }
    }
  };
  // slot e of pacc[rb][h] is row 4 (lane / 16) + e of the block: its scale
  // exponent is that of the lane holding the row
  auto unscaled = [&](int rb, int h, int e) {
    const int er = __shfl(xe[rb], 4 * lg + e, 64);
    return __builtin_ldexpf(pacc[rb][h][e], -(er + kUExp));
  };

  // ---- stream the tile in: the rank-k encode straight into the sub-tile
  // registers, the other kernels flat and coalesced through LDS -------------
  if constexpr (ENC) {
    const auto wr = make_rsrc(a.W, ((int64_t)(m - 1) * a.ldw + d) * 4);
    // the projection operands first: loads complete in order, so the
    // projection of a row block then waits for that block's data only
    if constexpr (LR) load_uops(a.ub, d, cbg0, uo);
    if constexpr (LR) {
      // each lane loads its sub-tiles directly (row 16 rb + lr, columns
      // c .. c + 3 and c + 16 .. c + 19), row block by row block; loads
      // complete in order, so the projection of a row block waits for that
      // block only while the later blocks stream in
#pragma unroll
      for (int rb = 0; rb < 3; ++rb)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const int row = row0 + 16 * rb + lr, c = col0 + 32 * (wave + 8 * q) + 4 * lg;
          const int o = (int)(((int64_t)row * a.ldw + c) * 4);
          const int32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(wr, (row < m && c < d) ? o : kOff, 0, 0);
          const int32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(wr, (row < m && c + 16 < d) ? o + 64 : kOff, 0, 0);
          float* xi = x[q * 3 + rb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xi[e] = __int_as_float(v0[e]);
            xi[4 + e] = __int_as_float(v1[e]);
          }
        }
#pragma unroll
      for (int rb = 0; rb < 3; ++rb) project_rb(rb);
    } else {
      int32x4 v[2 * kCPT];
#pragma unroll
      for (int j = 0; j < 2 * kCPT; ++j) {
        const int q = tid + 512 * j, r = q / 192, c = (q % 192) * 4;
        const bool ok = row0 + r < m && col0 + c < d;
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, ok ? (int)(((int64_t)(row0 + r) * a.ldw + col0 + c) * 4) : kOff,
                                                     0, 0);
      }
#pragma unroll
      for (int j = 0; j < 2 * kCPT; ++j) {
        const int q = tid + 512 * j, r = q / 192, c = (q % 192) * 4;
        *reinterpret_cast<int32x4*>(smem + r * kTilePad + c) = v[j];
      }
    }
  } else if constexpr (PIPE) {
    // Units (row block rb, replica r), rb-major; a unit is the block's
    // 16 x 768 codes of one replica: the 16-byte chunk at byte 16 t and the
    // 8-byte chunk at 8192 + 8 t of thread t (768 = 48 x 16: a 16-byte
    // chunk never crosses a row).  kPipeDepth units in flight (FP8), twice
    // as many of the half-size FP4 units.
    constexpr int NU = 3 * RC;
    constexpr bool PT = SC == 0;
    const int fA = 16 * tid, rA = fA / TC, cA = fA % TC;
    const int fB = 8192 + 8 * tid, rB = fB / TC, cB = fB % TC;
    const bool hiA = col0 + cA + 8 < d;   // the upper 8 codes of chunk A lie inside the row
    // FP8: code offsets (bytes) and the staged-scale entries; FP4 (d a
    // multiple of 16, so chunk A is one whole scale block): code offsets
    // (two codes a byte) and the offsets of the two blocks' scale bytes
    int offA[3], offB[3], sA[3], sB[3];
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) {
      const int ra = row0 + 16 * rb + rA, rbw = row0 + 16 * rb + rB;
      const bool okA = ra < m && col0 + cA < d, okB = rbw < m && col0 + cB < d;
      if constexpr (FMT == 2) {
        offA[rb] = okA ? (ra * d + col0 + cA) >> 1 : kOff;
        offB[rb] = okB ? (rbw * d + col0 + cB) >> 1 : kOff;
        sA[rb] = okA ? ra * (d / kFp4Block) + (col0 + cA) / kFp4Block : kOff;
        sB[rb] = okB ? rbw * (d / kFp4Block) + (col0 + cB) / kFp4Block : kOff;
      } else {
        offA[rb] = okA ? ra * d + col0 + cA : kOff;
        offB[rb] = okB ? rbw * d + col0 + cB : kOff;
        sA[rb] = (PT || !okA) ? 0 : (ra / kBlock - rb0) * 6 + (col0 + cA) / kBlock - cb0;
        sB[rb] = (PT || !okB) ? 0 : (rbw / kBlock - rb0) * 6 + (col0 + cB) / kBlock - cb0;
      }
    }
    if constexpr (!PT) {
      // the last wave stages the block scales before its code stream starts
      if (wave == 7) {
        const int nbm = (int)cdiv(m, kBlock);
        for (int t = lane; t < RC * 12; t += 64) {
          const int r = t / 12, e = t % 12, br = rb0 + e / 6, bc = cb0 + e % 6;
          ssc[r][e] = (br < nbm && bc < nbd) ? a.qscales[(int64_t)r * a.scale_stride + br * nbd + bc] : 0.f;
        }
      }
    }
    // the projection operands first (loads complete in order)
    load_uops(a.ub, d, cbg0, uo);
    using UnitT = typename pick_t<FMT == 2, Unit4, Unit>::type;
    // FP4 units are half the bytes: twice as many in flight
    constexpr int PD = FMT == 2 ? 2 * kPipeDepth : kPipeDepth;
    UnitT buf[PD];
    auto issue = [&](int u, UnitT& U) {
      const int rb = u / RC, r = u % RC;
      const bool in = u < NU;
      if constexpr (FMT == 2) {
        const auto q = make_rsrc(a.qcodes + (in ? (int64_t)r * a.code_stride : 0), in ? (int64_t)m * d / 2 : 0);
        const auto qs = make_rsrc(a.qbscales + (in ? (int64_t)r * a.bscale_stride : 0),
                                  in ? (int64_t)m * d / kFp4Block : 0);
        U.v = __builtin_amdgcn_raw_buffer_load_b64(q, in ? offA[rb < 3 ? rb : 2] : kOff, 0, kNT);
        U.t = __builtin_amdgcn_raw_buffer_load_b32(q, in ? offB[rb < 3 ? rb : 2] : kOff, 0, kNT);
        U.sa = __builtin_amdgcn_raw_buffer_load_b8(qs, in ? sA[rb < 3 ? rb : 2] : kOff, 0, 0);
        U.sb = __builtin_amdgcn_raw_buffer_load_b8(qs, in ? sB[rb < 3 ? rb : 2] : kOff, 0, 0);
      } else {
        const auto q = make_rsrc(a.qcodes + (in ? (int64_t)r * a.code_stride : 0), in ? (int64_t)m * d : 0);
        U.v = __builtin_amdgcn_raw_buffer_load_b128(q, in ? offA[rb < 3 ? rb : 2] : kOff, 0, kNT);
        U.t = __builtin_amdgcn_raw_buffer_load_b64(q, in ? offB[rb < 3 ? rb : 2] : kOff, 0, kNT);
      }
    };
#pragma unroll
    for (int u = 0; u < PD; ++u) issue(u, buf[u]);
    if constexpr (!PT) __syncthreads();   // the staged scales are visible
    float accA[16], accB[8];
    const float ir = a.invR;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int rb = u / RC, r = u % RC;
      UnitT& U = buf[u % PD];
      {
        float sa, sb, va[16], vb[8];
        if constexpr (FMT == 2) {
          // S_b = fp32(dec(sc_b) g_r); the E2M1 codes converted exactly by
          // the hardware (unit scale), the low nibble the even column
          const float gr = a.qtscales[r];
          sa = dec_e4m3(U.sa) * gr;
          sb = dec_e4m3(U.sb) * gr;
          dec8_fp4((uint32_t)U.v[0], va);
          dec8_fp4((uint32_t)U.v[1], va + 8);
          dec8_fp4((uint32_t)U.t, vb);
        } else {
          sa = PT ? a.qscales[(int64_t)r * a.scale_stride] : ssc[r][sA[rb]];
          sb = PT ? sa : ssc[r][sB[rb]];
#pragma unroll
          for (int w = 0; w < 4; ++w) dec4<FMT>((w < 2 || hiA) ? (uint32_t)U.v[w] : 0u, va + 4 * w);
          dec4<FMT>((uint32_t)U.t[0], vb);
          dec4<FMT>((uint32_t)U.t[1], vb + 4);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) accA[k] = r == 0 ? sa * va[k] : accA[k] + sa * va[k];
#pragma unroll
        for (int k = 0; k < 8; ++k) accB[k] = r == 0 ? sb * vb[k] : accB[k] + sb * vb[k];
      }
      issue(u + PD, U);   // past the last unit: an empty buffer resource, no memory traffic
      if (r == RC - 1) {
        // the block's mean into its rows of the tile, then its projection
        float* da = smem + (16 * rb + rA) * kTilePad + cA;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<float4*>(da + 4 * w) =
              make_float4(accA[4 * w] * ir, accA[4 * w + 1] * ir, accA[4 * w + 2] * ir, accA[4 * w + 3] * ir);
        float* db = smem + (16 * rb + rB) * kTilePad + cB;
        *reinterpret_cast<float4*>(db) = make_float4(accB[0] * ir, accB[1] * ir, accB[2] * ir, accB[3] * ir);
        *reinterpret_cast<float4*>(db + 4) = make_float4(accB[4] * ir, accB[5] * ir, accB[6] * ir, accB[7] * ir);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const float* src = smem + (rb * 16 + lr) * kTilePad + (wave + 8 * q) * 32 + 4 * lg;
          const float4 v0 = *reinterpret_cast<const float4*>(src);
          const float4 v1 = *reinterpret_cast<const float4*>(src + 16);
          float* xi = x[q * 3 + rb];
          xi[0] = v0.x; xi[1] = v0.y; xi[2] = v0.z; xi[3] = v0.w;
          xi[4] = v1.x; xi[5] = v1.y; xi[6] = v1.z; xi[7] = v1.w;
        }
        project_rb(rb);
        // partials into LDS: block b's lie in tile rows 5.5 b .. 5.5 b + 5.5,
        // which are free once every block before the one being read is read:
        // blocks 0 and 1 after block 1's barrier, block 2 after the last
        if (rb == 1) {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int e = 0; e < 4; ++e) cp[b][wave][4 * lg + e][lr + 16 * h] = unscaled(b, h, e);
        }
      }
    }
  } else {
    const int R = RC > 0 ? RC : a.R;
    int off[kDCPT], sidx[kDCPT];
    bool hi[kDCPT];
#pragma unroll
    for (int j = 0; j < kDCPT; ++j) {
      const int f = 16 * (tid + 512 * j), r = f / TC, c = f % TC;
      const bool ok = row0 + r < m && col0 + c < d;
      off[j] = ok ? (row0 + r) * d + col0 + c : kOff;
      hi[j] = col0 + c + 8 < d;
      sidx[j] = (pts || !ok) ? 0 : ((row0 + r) / kBlock - rb0) * 6 + (col0 + c) / kBlock - cb0;
    }
    const int ft = kDTail + 8 * tid, rt = ft / TC, ct = ft % TC;
    const bool okt = row0 + rt < m && col0 + ct < d;
    const int offt = okt ? (row0 + rt) * d + col0 + ct : kOff;
    const int sidxt = (pts || !okt) ? 0 : ((row0 + rt) / kBlock - rb0) * 6 + (col0 + ct) / kBlock - cb0;
    float acc[kDCPT][16], acct[8];
    CodeBuf b0, b1, b2;
    constexpr bool PT = SC == 0;
    // the projection operands go out right behind the last replica's codes
    auto load = [&](int r, CodeBuf& b) {
      load_codes<FMT>(a, R, r, off, offt, b);
      if (LR && RC > 0 && r == R - 1) load_uops(a.ub, d, cbg0, uo);
    };
    if constexpr (PT) {
      load(0, b0);
      load(1, b1);
    } else {
      // The last wave stages the block scales in LDS before it starts its
      // code stream; the other waves start theirs at once.  (A scale load
      // issued behind the code loads would wait for all of them: loads
      // retire in order.)
      if (wave == 7) {
        const int nbm = (int)cdiv(m, kBlock);
        for (int t = lane; t < R * 12; t += 64) {
          const int r = t / 12, e = t % 12, br = rb0 + e / 6, bc = cb0 + e % 6;
          ssc[r][e] = (br < nbm && bc < nbd) ? a.qscales[(int64_t)r * a.scale_stride + br * nbd + bc] : 0.f;
        }
      }
      load(0, b0);
      load(1, b1);
      __syncthreads();
    }
    // per-tensor scale of replica r: a uniform word (scalar load)
    auto rscale = [&](int r) -> float { return PT ? a.qscales[(int64_t)r * a.scale_stride] : 0.f; };
    auto three = [&](int r) -> bool {   // replicas r .. r + 2; false once past R
      load(r + 2, b2);
      accum_codes<FMT, PT>(acc, acct, b0, ssc[r], rscale(r), sidx, sidxt, hi, r == 0);
      if (r + 1 >= R) return false;
      load(r + 3, b0);
      accum_codes<FMT, PT>(acc, acct, b1, ssc[r + 1], rscale(r + 1), sidx, sidxt, hi, false);
      if (r + 2 >= R) return false;
      load(r + 4, b1);
      accum_codes<FMT, PT>(acc, acct, b2, ssc[r + 2], rscale(r + 2), sidx, sidxt, hi, false);
      return true;
    };
    if constexpr (RC > 0) {
#pragma unroll
      for (int r = 0; r < RC; r += 3)
        if (!three(r)) break;
    } else {
      for (int r = 0; r < R; r += 3)
        if (!three(r)) break;
      if constexpr (LR) load_uops(a.ub, d, cbg0, uo);
    }
    const float ir = a.invR;
#pragma unroll
    for (int j = 0; j < kDCPT; ++j) {
      const int f = 16 * (tid + 512 * j), r = f / TC, c = f % TC;
      float* dst = smem + r * kTilePad + c;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        *reinterpret_cast<float4*>(dst + 4 * w) = make_float4(acc[j][4 * w] * ir, acc[j][4 * w + 1] * ir,
                                                              acc[j][4 * w + 2] * ir, acc[j][4 * w + 3] * ir);
    }
    {
      float* dst = smem + rt * kTilePad + ct;
      *reinterpret_cast<float4*>(dst) = make_float4(acct[0] * ir, acct[1] * ir, acct[2] * ir, acct[3] * ir);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(acct[4] * ir, acct[5] * ir, acct[6] * ir, acct[7] * ir);
    }
  }
  if constexpr (!PIPE) {
  __syncthreads();
  if constexpr (!LR && !ENC) {
    // Euclidean decode: the staged tile is the output
    const auto orr = make_rsrc(a.out, ((int64_t)(m - 1) * a.ldo + d) * 4);
#pragma unroll
    for (int j = 0; j < 2 * kCPT; ++j) {
      const int q = tid + 512 * j, r = q / 192, c = (q % 192) * 4;
      const bool ok = row0 + r < m && col0 + c < d;
      const int32x4 v = *reinterpret_cast<const int32x4*>(smem + r * kTilePad + c);
      __builtin_amdgcn_raw_buffer_store_b128(v, orr, ok ? (int)(((int64_t)(row0 + r) * a.ldo + col0 + c) * 4) : kOff,
                                             0, 0);
    }
    return;
  }
  // each lane takes its sub-tile layout out of the staged tile
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    const float* src = smem + (SUB_RB(i) * 16 + lr) * kTilePad + SUB_CB(i) * 32 + 4 * lg;
    const float4 v0 = *reinterpret_cast<const float4*>(src);
    const float4 v1 = *reinterpret_cast<const float4*>(src + 16);
    x[i][0] = v0.x; x[i][1] = v0.y; x[i][2] = v0.z; x[i][3] = v0.w;
    x[i][4] = v1.x; x[i][5] = v1.y; x[i][6] = v1.z; x[i][7] = v1.w;
  }
  }   // staging of everything but the rank-k encode
  __syncthreads();   // every sub-tile read is done: the tile memory is free

  if constexpr (LR) {
  if constexpr (!PIPE) {
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) project_rb(rb);
  }
  // (the block-pipelined decode has written blocks 0 and 1 already)
#pragma unroll
  for (int rb = (PIPE && !ENC) ? 2 : 0; rb < 3; ++rb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) cp[rb][wave][4 * lg + e][lr + 16 * h] = unscaled(rb, h, e);
  __syncthreads();
  // sum the 8 waves (fixed order) and publish this tile's partial: word
  // e = 32 row + k of the tile, one atomic exchange each (it takes effect at
  // the device's coherence point; nobody waits for it)
  unsigned long long* xg = a.xpub + (int64_t)g * kXW;
#pragma unroll
  for (int j = 0; j < kXPT; ++j) {
    const int e = tid + 512 * j, r = e >> 5, k = e & 31;
    float s = cp[r >> 4][0][r & 15][k];
#pragma unroll
    for (int w = 1; w < 8; ++w) s += cp[r >> 4][w][r & 15][k];
    __hip_atomic_exchange(xg + e, tagged(tag, s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the reconstruction operands, before the partner words
  load_uops(a.ua, d, cbg0, uo);
  // Reduce-scatter, then all-gather, inside the row group: workgroup cgi
  // sums the slice [cgi S, cgi S + S) of the 48 x 32 words over the CG
  // partials (in column-group order) and publishes the sums; every workgroup
  // then reads the row group's sums.  Each word is read until it carries this
  // call's tag.  (Each workgroup reading every partial would move CG times
  // the data through the device-scope path on every polling round.)
  {
    const int cg = a.CG;
    const unsigned long long* rowpub = a.xpub + (int64_t)rg * cg * kXW;
    unsigned long long* sums = a.xpub + (int64_t)G * kXW + (int64_t)rg * kXW;
    const int S = (kXW + cg - 1) / cg;
    for (int t = tid; t < S; t += 512) {   // one pass unless CG < 3
      const int e = cgi * S + t;
      if (e >= kXW) break;
      float s = 0.f;
      for (int h0 = 0; h0 < cg; h0 += 16) {
        unsigned long long w[16];
        int spins = 0;
        for (;;) {
          // all loads first, then the tests (a test inside the load's
          // branch would wait for each load in turn); partners past the
          // row group are not read
#pragma unroll
          for (int h = 0; h < 16; ++h)
            if (h0 + h < cg) w[h] = ld_dev64(rowpub + (int64_t)(h0 + h) * kXW + e);
          bool ok = true;
#pragma unroll
          for (int h = 0; h < 16; ++h) ok = ok && (h0 + h >= cg || (unsigned)(w[h] >> 32) == tag);
          if (ok) break;
          if (++spins > kSpinLimit) {
            atomicOr(a.flags, (unsigned)GIFT_FLAG_SPIN_TIMEOUT);
            s_bad = 1;
            break;
          }
        }
#pragma unroll
        for (int h = 0; h < 16; ++h) {
          const float v = __uint_as_float((uint32_t)w[h]);
          if (h0 + h == 0)
            s = v;
          else if (h0 + h < cg)
            s += v;
        }
      }
      __hip_atomic_exchange(sums + e, tagged(tag, s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const float* cvec = a.coef + (enc ? 0 : 32);
    unsigned long long w[kXPT];
    int spins = 0;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < kXPT; ++j) {
        w[j] = ld_dev64(sums + tid + 512 * j);
        ok = ok && (unsigned)(w[j] >> 32) == tag;
      }
      if (ok) break;
      if (++spins > kSpinLimit) {
        atomicOr(a.flags, (unsigned)GIFT_FLAG_SPIN_TIMEOUT);
        s_bad = 1;
        break;
      }
    }
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int e = tid + 512 * j;
      pf[e >> 5][e & 31] = __uint_as_float((uint32_t)w[j]) * cvec[e & 31];
    }
  }
  __syncthreads();

  // ---- reconstruction X~ = alpha X + (P c) U^T ------------------------------
  {
    const bool bad = s_bad != 0;   // uniform: every wait of the exchange is before the barrier
    const float alpha = a.coef[64 + (enc ? 0 : 1)];
    // P c of row 16 rb + (lane % 16), 8 rank entries per lane: scaled by the
    // row's exponent (over its 32 entries, which the four lanes of the row
    // hold) and split into two f16 pieces
    half8 ph[3], pl[3];
    int pe[3];
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) {
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(pf[rb * 16 + lr][8 * lg + j]));
      pe[rb] = row_exp(rowmax4(mx));
      const float sc = pow2f(pe[rb]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        _Float16 h, l;
        split2(pf[rb * 16 + lr][8 * lg + j] * sc, h, l);
        ph[rb][j] = h;
        pl[rb][j] = l;
      }
    }
    // the three sub-tiles of column block q (this wave's columns
    // col0 + 32 (wave + 8 q) ..) made final in the registers
    auto recon_q = [&](int q) {
      if (!live[q]) return;
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        const half8 uh = uo.u[q][grp][0], ul = uo.u[q][grp][1];
#pragma unroll
        for (int rb = 0; rb < 3; ++rb) {
          const int i = q * 3 + rb;
          floatx4 c = (floatx4){0.f, 0.f, 0.f, 0.f};
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ul, ph[rb], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(uh, pl[rb], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(uh, ph[rb], c, 0, 0, 0);
          // slot e is the lane's own row: alpha x + the product scaled back
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[i][4 * grp + e] = __builtin_fmaf(alpha, x[i][4 * grp + e], __builtin_ldexpf(c[e], -(pe[rb] + kUExp)));
        }
      }
    };
    if constexpr (ENC) {
#pragma unroll
      for (int q = 0; q < 3; ++q) recon_q(q);
    } else {
      // Decode: the output leaves through LDS so that every store
      // instruction of a wave writes 1 KB of one row (256 columns) instead
      // of 64 bytes of 16 rows.  Column block q of all 8 waves is the 48 x
      // 256 slab at columns col0 + 256 q; slabs alternate between two
      // buffers (the partials' area and the space after the gathered
      // projection), and the products of the next slab run while the
      // previous one is stored.
      float* stg[2] = {smem, smem + kStageB};
      auto stage = [&](int q) {
        float* b = stg[q & 1];
#pragma unroll
        for (int rb = 0; rb < 3; ++rb) {
          const int i = q * 3 + rb;
          float* dst = b + (16 * rb + lr) * kStagePad + 32 * wave + 4 * lg;
          if (bad) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = __builtin_nanf("");
          }
          *reinterpret_cast<float4*>(dst) = make_float4(x[i][0], x[i][1], x[i][2], x[i][3]);
          *reinterpret_cast<float4*>(dst + 16) = make_float4(x[i][4], x[i][5], x[i][6], x[i][7]);
        }
      };
      const auto orr = make_rsrc(a.out, ((int64_t)(m - 1) * a.ldo + d) * 4);
      auto drain = [&](int q) {
        const float* b = stg[q & 1];
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          const int f = tid + 512 * j, r = f >> 6, c = (f & 63) * 4;
          const int32x4 v = *reinterpret_cast<const int32x4*>(b + r * kStagePad + c);
          const int row = row0 + r, col = col0 + 256 * q + c;
          __builtin_amdgcn_raw_buffer_store_b128(
              v, orr, (row < m && col < d) ? (int)(((int64_t)row * a.ldo + col) * 4) : kOff, 0, kNT);
        }
      };
      recon_q(0);
      stage(0);
      __syncthreads();
      recon_q(1);
      drain(0);
      stage(1);
      __syncthreads();
      recon_q(2);
      drain(1);
      stage(2);
      __syncthreads();
      drain(2);
    }
  }

  }   // LR

  if constexpr (LR && !ENC) return;   // the decode stored its sub-tiles above

  if (!enc) {
    // ---- decode: store W^ --------------------------------------------------
    __syncthreads();   // everyone is done with pf (aliased by the tile)
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      float* dst = smem + (SUB_RB(i) * 16 + lr) * kTilePad + SUB_CB(i) * 32 + 4 * lg;
      *reinterpret_cast<float4*>(dst) = make_float4(x[i][0], x[i][1], x[i][2], x[i][3]);
      *reinterpret_cast<float4*>(dst + 16) = make_float4(x[i][4], x[i][5], x[i][6], x[i][7]);
    }
    __syncthreads();
    const auto orr = make_rsrc(a.out, ((int64_t)(m - 1) * a.ldo + d) * 4);
#pragma unroll
    for (int j = 0; j < 2 * kCPT; ++j) {
      const int q = tid + 512 * j, r = q / 192, c = (q % 192) * 4;
      const bool ok = row0 + r < m && col0 + c < d;
      const int32x4 v = *reinterpret_cast<const int32x4*>(smem + r * kTilePad + c);
      __builtin_amdgcn_raw_buffer_store_b128(v, orr, ok ? (int)(((int64_t)(row0 + r) * a.ldo + col0 + c) * 4) : kOff,
                                             0, 0);
    }
    return;
  }

  // ---- encode: inspection copy, error feedback, amax, scale, quantise -------
  // The residual R (error feedback, Algorithm 1) is read in the sub-tile
  // layout of x: sub-tile i of this lane holds row row0 + 16 SUB_RB(i) + lr,
  // columns c .. c + 3 and c + 16 .. c + 19, c = col0 + 32 SUB_CB(i) + 4 lg.
  const auto rr = make_rsrc(a.resid, EF ? (int64_t)m * d * 4 : 0);
  int32x4 rv[NSUB][2];
  if constexpr (EF) {
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      const int row = row0 + SUB_RB(i) * 16 + lr, c = col0 + SUB_CB(i) * 32 + 4 * lg;
      const int o = (row * d + c) * 4;
      rv[i][0] = __builtin_amdgcn_raw_buffer_load_b128(rr, (row < m && c < d) ? o : kOff, 0, 0);
      rv[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rr, (row < m && c + 16 < d) ? o + 64 : kOff, 0, 0);
    }
  }
  if (a.whitened) {
    const auto wh = make_rsrc(a.whitened, (int64_t)m * d * 4);
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      const int row = row0 + SUB_RB(i) * 16 + lr, c = col0 + SUB_CB(i) * 32 + 4 * lg;
      const int o = (row * d + c) * 4;
      const int32x4 v0 = {__float_as_int(x[i][0]), __float_as_int(x[i][1]), __float_as_int(x[i][2]), __float_as_int(x[i][3])};
      const int32x4 v1 = {__float_as_int(x[i][4]), __float_as_int(x[i][5]), __float_as_int(x[i][6]), __float_as_int(x[i][7])};
      __builtin_amdgcn_raw_buffer_store_b128(v0, wh, (row < m && c < d) ? o : kOff, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(v1, wh, (row < m && c + 16 < d) ? o + 64 : kOff, 0, 0);
    }
  }
  if constexpr (EF) {
    // U~ = fp32(W~ + R); entries outside the tensor read zeros
#pragma unroll
    for (int i = 0; i < NSUB; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] += __int_as_float(rv[i][j >> 2][j & 3]);
  }
  // |x| bit patterns order like |x| (NaN above +Inf): the lane maximum of
  // each sub-tile.  Dead column blocks hold zeros.
  uint32_t lmax[NSUB];
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = absbits_f(x[i][j]);
      v = v > b ? v : b;
    }
    lmax[i] = v;
  }
  // Blocks this tile touches: rows row0 .. row0 + 47 lie in at most two
  // 128-row blocks (rb0, rb0 + 1); columns col0 .. col0 + 767 in the six
  // 128-column blocks cb0 .. cb0 + 5 (col0 is a multiple of 768).  Local
  // amax of this tile per block entry (2 x 6), or per tensor (entry 0).
  if (pts) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < NSUB; ++i) v = v > lmax[i] ? v : lmax[i];
    v = wave_umax(v);
    if (lane == 0) wmax[8 + wave] = v;
    __syncthreads();
    if (tid == 0) {
      uint32_t t = wmax[8];
#pragma unroll
      for (int w = 1; w < 8; ++w) t = t > wmax[8 + w] ? t : wmax[8 + w];
      wmax[0] = t;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      const uint32_t v = wave_umax(lmax[i]);
      if (lane == 0 && live[i / 3] && v != 0u) {
        const int e = ((row0 + SUB_RB(i) * 16) / kBlock - rb0) * 6 + (col0 + SUB_CB(i) * 32) / kBlock - cb0;
        atomicMax(&wmax[e], v);
      }
    }
  }
  if (tid < 16) blk[tid >> 3][tid & 7] = 0u;
  __syncthreads();
  if (s_bad) {   // uniform here: a partner of the exchange never published
    if (tid < 16) wmax[tid] = 0x7FC00000u;   // NaN bits order above every |x|
    __syncthreads();
  }
  const bool need_sync = a.amax_in == nullptr || a.amax_out != nullptr;
  if (need_sync) {
    unsigned long long* pub = a.apub;
    const unsigned long long etag = (unsigned long long)epoch << 32;
    // the tag makes each word self-validating: no ordering with other data
    // is needed.  The words are published with atomic exchanges, which take
    // effect at the device's coherence point at once.
    if (pts) {
      // per tensor: one word per workgroup, written into kAmaxCopies copies
      // of a compact array (lane c of wave 0 writes copy c); workgroup g
      // reads copy g % kAmaxCopies with one wave, a few coalesced loads per
      // round
      const int cstride = amax_copy_stride(G);
      unsigned long long* pt = pub + (int64_t)G * kApub + (int64_t)(g % kAmaxCopies) * cstride;
      if (wave == 0) {
        if (lane < kAmaxCopies) atomicExch(pub + (int64_t)G * kApub + (int64_t)lane * cstride + g, etag | wmax[0]);
        uint32_t v = 0;
        for (int base = 0; base < G; base += 256) {
          unsigned long long w[4];
          int spins = 0;
          for (;;) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int h = base + lane + 64 * j;
              w[j] = h < G ? ld_dev64(pt + h) : etag;
            }
            bool ok = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) ok = ok && (unsigned)(w[j] >> 32) == epoch;
            if (__all(ok)) break;
            if (++spins > kSpinLimit) {
              if (lane == 0) {
                atomicOr(a.flags, (unsigned)GIFT_FLAG_SPIN_TIMEOUT);
                s_bad = 1;
              }
              break;
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) v = v > (uint32_t)w[j] ? v : (uint32_t)w[j];
        }
        v = wave_umax(v);
        if (lane == 0) blk[0][0] = v;
      }
    } else {
      if (tid < kApub) atomicExch(pub + (int64_t)g * kApub + tid, etag | wmax[tid]);
      // the tiles of this column group whose rows meet blocks rb0, rb0 + 1
      const int r_lo = (rb0 * kBlock) / TR;
      const int r_hi = min((int)cdiv(m, TR) - 1, ((rb0 + 2) * kBlock - 1) / TR);
      const int nr = r_hi - r_lo + 1;
      for (int t = tid; t < nr * 12; t += 512) {
        const int rr = r_lo + t / 12, e = t % 12;
        const int h = rr * a.CG + cgi;
        const unsigned long long w = wait_tag(pub + (int64_t)h * kApub + e, epoch, a.flags, &s_bad);
        const int brow = (rr * TR) / kBlock + e / 6;   // global block row of that entry
        const int slot_r = brow - rb0;
        if (slot_r >= 0 && slot_r < 2 && (uint32_t)w) atomicMax(&blk[slot_r][e % 6], (uint32_t)w);
      }
    }
    __syncthreads();
  }
  // scale pair of every block entry of this tile (entry 0 per tensor);
  // the workgroup holding a block's top-left sub-tile writes its scale and
  // local amax
  const float fmax = fp8_fmax(FMT);
  if constexpr (FMT == 2) {
    // FP4: the tensor scale g = fp32(amax_T / 2688) from the tensor amax
    // (local, or the shared one); the block scales follow per 16 elements
    if (tid == 0) {
      const uint32_t local = blk[0][0];
      const bool bad = s_bad != 0;
      const uint32_t am = bad ? 0x7FC00000u : (a.amax_in ? absbits_f(a.amax_in[0]) : local);
      sss[0] = fp4_tscale(am);
      if (g == 0) {
        if (a.tscale) a.tscale[0] = sss[0];
        if (a.amax_out) a.amax_out[0] = bad ? __builtin_nanf("") : __uint_as_float(local);
        if (am >= 0x7F800000u) atomicOr(a.flags, (unsigned)GIFT_FLAG_NONFINITE);
      }
    }
  } else if (tid < 12 && (!pts || tid == 0)) {
    const int br = rb0 + tid / 6, bc = cb0 + tid % 6;
    // blocks rb0 and cb0 .. cb0 + 5 always meet the tile; rb0 + 1 may not
    const bool inside = br * kBlock < m && bc * kBlock < d && br * kBlock < row0 + TR;
    srs[tid] = 0.0f;
    sss[tid] = 0.0f;
    sam[tid] = 0u;
    if (inside) {
      const int slot = pts ? 0 : br * nbd + bc;
      const uint32_t local = blk[tid / 6][tid % 6];
      const uint32_t am = a.amax_in ? absbits_f(a.amax_in[slot]) : local;
      float r, sc;
      scale_pair(am, fmax, r, sc);
      srs[tid] = r;
      sss[tid] = sc;
      sam[tid] = am;
      const bool leader = pts ? g == 0 : (br * kBlock >= row0 && bc * kBlock >= col0);
      if (leader) {
        const bool bad = s_bad != 0;
        if (a.scales) a.scales[slot] = bad ? __builtin_nanf("") : sc;
        if (a.amax_out) a.amax_out[slot] = bad ? __builtin_nanf("") : __uint_as_float(local);
        if (am >= 0x7F800000u) atomicOr(a.flags, (unsigned)GIFT_FLAG_NONFINITE);
      }
    }
  }
  __syncthreads();   // the tile memory now receives the codes
  if (!a.codes) return;
  const bool bad = s_bad != 0;
  // hardware conversion of 8 finite values (clamped to the format's range:
  // saturating RNE)
  auto hw8 = [&](const float* xi, float r, uint32_t& q0, uint32_t& q1) {
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = __builtin_amdgcn_fmed3f(xi[j] * r, fmax, -fmax);
    if constexpr (FMT == 0) {
      q0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      q0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)q0, true);
      q1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      q1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)q1, true);
    } else {
      q0 = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
      q0 = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], (int)q0, true);
      q1 = __builtin_amdgcn_cvt_pk_bf8_f32(y[4], y[5], 0, false);
      q1 = __builtin_amdgcn_cvt_pk_bf8_f32(y[6], y[7], (int)q1, true);
    }
  };
  // the codes into the tile memory; with error feedback the new residual
  // fp32(U~ - s dec(q)), the difference rounded once
  auto emit = [&](int i, uint32_t q0, uint32_t q1, float sc) {
    const int rbl = SUB_RB(i), cbl = SUB_CB(i);
    uint8_t* cs = reinterpret_cast<uint8_t*>(smem) + (rbl * 16 + lr) * (TC + 16) + cbl * 32 + 4 * lg;
    *reinterpret_cast<uint32_t*>(cs) = q0;
    *reinterpret_cast<uint32_t*>(cs + 16) = q1;
    if constexpr (EF) {
      float dv[8];
      dec4<FMT>(q0, dv);
      dec4<FMT>(q1, dv + 4);
      int32x4 o0, o1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o0[j] = __float_as_int(__builtin_fmaf(-sc, dv[j], x[i][j]));
        o1[j] = __float_as_int(__builtin_fmaf(-sc, dv[4 + j], x[i][4 + j]));
      }
      const int row = row0 + rbl * 16 + lr, c = col0 + cbl * 32 + 4 * lg;
      const int o = (row * d + c) * 4;
      __builtin_amdgcn_raw_buffer_store_b128(o0, rr, (row < m && c < d) ? o : kOff, 0, kNT);
      __builtin_amdgcn_raw_buffer_store_b128(o1, rr, (row < m && c + 16 < d) ? o + 64 : kOff, 0, kNT);
    }
  };
  if constexpr (FMT == 2) {
    // FP4: a sub-tile row's 32 columns are two 16-element blocks (block
    // j = 2 i + h of sub-tile i), each held by the four lanes of the row,
    // columns 4 lg .. 4 lg + 3 of it.  Blocks go in groups of four: each
    // lane forms its partial amax over |x| bits (NaN on top) of the four,
    // a transpose over the row's lanes hands lane lg the four partials of
    // the group's block lg, and that lane alone forms the block amax, sig =
    // fp32(amax_b / 6g), the E4M3 block scale (which it stores) and r_b =
    // fp32(1 / S_b), NaN for a NaN block scale.  A transpose of the r_b,
    // replicated, gives every lane of the row the group's four.  The E2M1
    // codes come from the hardware conversion at unit scale, which rounds
    // as the encoder does (to nearest, ties to the even code, saturating at
    // 6, both signs of zero kept) for every non-NaN input; where a product
    // x r_b can be NaN in the wave (a non-finite x, an infinite or NaN r_b)
    // NaN products are set to +0 first, the encoder's code for NaN and
    // the zero codes of a NaN block scale.  Four codes per lane and block
    // go into the tile memory (rows of 384 bytes, the even column in the
    // low nibble).  With error feedback the S_b are spread the same way
    // and the new residual fp32(U~ - S_b dec(q)) is formed from the codes
    // (the difference rounded once) and stored.
    const float gt = sss[0];
    const int bpr = d / kFp4Block;
    constexpr int NG = (2 * NSUB + 3) / 4;
    float rbs[NG][4], sbs[EF ? NG : 1][4];
    bool risky = false;
#pragma unroll
    for (int g4 = 0; g4 < NG; ++g4) {
      uint32_t r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = 4 * g4 + k;
        uint32_t mb = 0;
        if (j < 2 * NSUB) {
#pragma unroll
          for (int e = 0; e < 4; ++e) mb = umax32(mb, absbits_f(x[j >> 1][4 * (j & 1) + e]));
        }
        r[k] = mb;
      }
      quad_transpose(r);
      const uint32_t mb = umax32(umax32(r[0], r[1]), umax32(r[2], r[3]));
      float sig;
      if (gt != gt) sig = __builtin_nanf("");
      else if (gt == 0.0f) sig = 0.0f;
      else sig = (float)((double)__uint_as_float(mb) / (6.0 * (double)gt));
      const uint32_t sc = enc_e4m3(sig);
      const float S = dec_e4m3(sc) * gt;
      const float rb_ = S != S ? S : (S > 0.0f ? 1.0f / S : 0.0f);
      risky = risky || mb >= 0x7F800000u || !(__builtin_fabsf(rb_) < __builtin_inff());
      const int j = 4 * g4 + lg, i = j >> 1;
      const int row = row0 + (i % 3) * 16 + lr, col = col0 + (wave + 8 * (i / 3)) * 32 + 16 * (j & 1);
      if (j < 2 * NSUB && row < m && col < d) {
        a.bscales[(int64_t)row * bpr + col / kFp4Block] = (uint8_t)sc;
        if (S != S && gt == gt) atomicOr(a.flags, (unsigned)GIFT_FLAG_NONFINITE);
      }
      uint32_t bq[4] = {__float_as_uint(rb_), __float_as_uint(rb_), __float_as_uint(rb_), __float_as_uint(rb_)};
      quad_transpose(bq);
#pragma unroll
      for (int k = 0; k < 4; ++k) rbs[g4][k] = __uint_as_float(bq[k]);
      if constexpr (EF) {
        uint32_t bs[4] = {__float_as_uint(S), __float_as_uint(S), __float_as_uint(S), __float_as_uint(S)};
        quad_transpose(bs);
#pragma unroll
        for (int k = 0; k < 4; ++k) sbs[g4][k] = __uint_as_float(bs[k]);
      }
    }
    auto codes = [&](auto fix) {
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
        if (!live[i / 3]) continue;
        const int rbl = SUB_RB(i), cbl = SUB_CB(i);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * i + h;
          const float rb_ = rbs[j >> 2][j & 3];
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = x[i][4 * h + e] * rb_;
            y[e] = (!decltype(fix)::value || t == t) ? t : 0.0f;
          }
          uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
          const int cb = cbl * 32 + 16 * h;   // the block's first column in the tile
          *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(smem) + (rbl * 16 + lr) * kFp4Pad + (cb >> 1) +
                                       2 * lg) = (uint16_t)w;
          if constexpr (EF) {
            const float sb = sbs[j >> 2][j & 3];
            const auto d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
            const auto d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
            const float dv[4] = {d0[0], d0[1], d1[0], d1[1]};
            int32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __float_as_int(__builtin_fmaf(-sb, dv[e], x[i][4 * h + e]));
            const int row = row0 + rbl * 16 + lr, c = col0 + cb + 4 * lg;
            __builtin_amdgcn_raw_buffer_store_b128(o, rr, (row < m && c < d) ? (row * d + c) * 4 : kOff, 0, kNT);
          }
        }
      }
    };
    if (__any(risky)) codes(std::true_type{});
    else codes(std::false_type{});
  } else {
  // Per tensor with a finite amax and no non-finite element in the wave's
  // sub-tiles (the usual case, one uniform test): one scale pair for every
  // sub-tile and no per-sub-tile branches.
  bool nonfin = false;
#pragma unroll
  for (int i = 0; i < NSUB; ++i) nonfin = nonfin || lmax[i] >= 0x7F800000u;
  if (pts && !bad && sam[0] < 0x7F800000u && !__any(nonfin)) {
    const float r = srs[0], sc = sss[0];
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      if (!live[i / 3]) continue;
      uint32_t q0, q1;
      hw8(x[i], r, q0, q1);
      emit(i, q0, q1, sc);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      if (!live[i / 3]) continue;
      const int rbl = SUB_RB(i), cbl = SUB_CB(i);
      const int e = pts ? 0 : ((row0 + rbl * 16) / kBlock - rb0) * 6 + (col0 + cbl * 32) / kBlock - cb0;
      const float r = srs[e];
      const uint32_t am = sam[e];
      uint32_t q0, q1;
      if (am >= 0x7F800000u || bad) {
        q0 = q1 = 0x7F7F7F7Fu;
      } else if (lmax[i] >= 0x7F800000u) {
        // a non-finite element under a finite shared amax: exact integer path
        uint32_t e8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e8[j] = enc_fp8<FMT>(x[i][j] * r);
        q0 = e8[0] | (e8[1] << 8) | (e8[2] << 16) | (e8[3] << 24);
        q1 = e8[4] | (e8[5] << 8) | (e8[6] << 16) | (e8[7] << 24);
      } else {
        hw8(x[i], r, q0, q1);
      }
      emit(i, q0, q1, sss[e]);
    }
  }
  }   // FP8
  __syncthreads();
  if constexpr (FMT == 2) {
    // FP4 codes: 48 rows of 384 bytes, in 8-byte pieces (16 columns each)
    const auto cr = make_rsrc(a.codes, (int64_t)m * (d / 2));
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int q = tid + 512 * j;
      if (q >= TR * (TC / 16)) break;
      const int r = q / (TC / 16), c16 = q % (TC / 16);
      const bool ok = row0 + r < m && col0 + 16 * c16 < d;
      const int32x2 v = *reinterpret_cast<const int32x2*>(reinterpret_cast<const uint8_t*>(smem) + r * kFp4Pad + 8 * c16);
      __builtin_amdgcn_raw_buffer_store_b64(v, cr, ok ? ((row0 + r) * d + col0) / 2 + 8 * c16 : kOff, 0, kNT);
    }
    return;
  }
  const auto cr = make_rsrc(a.codes, (int64_t)m * d);
#pragma unroll
  for (int j = 0; j < kCPT; ++j) {
    const int q = tid + 512 * j, r = q / 96, c = (q % 96) * 8;
    const bool ok = row0 + r < m && col0 + c < d;
    const int32x2 v = *reinterpret_cast<const int32x2*>(reinterpret_cast<const uint8_t*>(smem) + r * (TC + 16) + c);
    __builtin_amdgcn_raw_buffer_store_b64(v, cr, ok ? (row0 + r) * d + col0 + c : kOff, 0, kNT);
  }
}

// One kernel per direction, transform and format (distinct names in
// traces); the encode also with error feedback (_ef), the decode per
// replica count 4, 8, 16 (0: any count up to 64) and scaling.
template <int FMT, int SC>
__global__ void __launch_bounds__(512) k_rank_encode(FusedArgs a) {
  fused_body<FMT, true, 0, SC, true>(a, blockIdx.x, gridDim.x, a.epoch);
}
template <int FMT, int SC>
__global__ void __launch_bounds__(512) k_rank_encode_ef(FusedArgs a) {
  fused_body<FMT, true, 0, SC, true, true>(a, blockIdx.x, gridDim.x, a.epoch);
}
template <int FMT, int RC, int SC>
__global__ void __launch_bounds__(512) k_rank_decode(FusedArgs a) {
  fused_body<FMT, false, RC, SC, true>(a, blockIdx.x, gridDim.x, a.epoch);
}
template <int FMT, int SC>
__global__ void __launch_bounds__(512) k_euclid_encode(FusedArgs a) {
  fused_body<FMT, true, 0, SC, false>(a, blockIdx.x, gridDim.x, a.epoch);
}
template <int FMT, int SC>
__global__ void __launch_bounds__(512) k_euclid_encode_ef(FusedArgs a) {
  fused_body<FMT, true, 0, SC, false, true>(a, blockIdx.x, gridDim.x, a.epoch);
}
template <int FMT, int RC, int SC>
__global__ void __launch_bounds__(512) k_euclid_decode(FusedArgs a) {
  fused_body<FMT, false, RC, SC, false>(a, blockIdx.x, gridDim.x, a.epoch);
}

// Grouped launch: several rank-k layers one after another in one persistent
// launch (one per phase).  Workgroup g takes tile g of each layer in turn
// (layers with fewer tiles skip it) and moves on as soon as its part of a
// layer is done, so the tail of one layer overlaps the loads of the next in
// other workgroups.  Each layer's exchange words and amax words live in its
// own state, tagged with its own call epoch (passed by value).
template <int FMT, bool ENC, int RC, int SC>
__global__ void __launch_bounds__(512) k_rank_group(const FusedArgs* __restrict__ table, int n, GroupEpochs ep) {
  for (int L = 0; L < n; ++L) {
    const FusedArgs& a = table[L];
    const int tiles = (int)cdiv(a.m, TR) * a.CG;
    if ((int)blockIdx.x < tiles) fused_body<FMT, ENC, RC, SC, true>(a, blockIdx.x, tiles, ep.v[L]);
    __syncthreads();   // the LDS of this layer is free before the next one
  }
}

// Persistent launches.  The workgroups of these kernels wait on words that
// other workgroups of the same launch publish, so every workgroup of the grid
// must be resident at once: the host takes this route only when the grid
// fits the kernels' occupancy (fused_resident_groups) and orders its
// persistent launches device-wide, so two of them never share the device.
// (A cooperative launch would have the runtime guarantee co-residency, but
// it measured about 18 us more per launch than the 25-35 us kernels.)
template <typename K>
static hipError_t persistent_launch(K kernel, int grid, const FusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int FMT, int SC, bool LR>
static hipError_t launch_decode(const FusedArgs& a, int grid, hipStream_t s) {
  if constexpr (LR) {
    switch (a.R) {
      case 4: return persistent_launch(k_rank_decode<FMT, 4, SC>, grid, a, s);
      case 8: return persistent_launch(k_rank_decode<FMT, 8, SC>, grid, a, s);
      case 16: return persistent_launch(k_rank_decode<FMT, 16, SC>, grid, a, s);
      default: return persistent_launch(k_rank_decode<FMT, 0, SC>, grid, a, s);
    }
  } else {
    switch (a.R) {
      case 4: return persistent_launch(k_euclid_decode<FMT, 4, SC>, grid, a, s);
      case 8: return persistent_launch(k_euclid_decode<FMT, 8, SC>, grid, a, s);
      case 16: return persistent_launch(k_euclid_decode<FMT, 16, SC>, grid, a, s);
      default: return persistent_launch(k_euclid_decode<FMT, 0, SC>, grid, a, s);
    }
  }
}

template <int FMT, bool LR>
static hipError_t launch_decode(const FusedArgs& a, int grid, hipStream_t s) {
  return a.scaling == 0 ? launch_decode<FMT, 0, LR>(a, grid, s) : launch_decode<FMT, 1, LR>(a, grid, s);
}

template <int SC>
static hipError_t launch_encode(const FusedArgs& a, int grid, hipStream_t s) {
  // kernel by transform, error feedback and format
  const int which = (a.lr ? 4 : 0) + (a.resid ? 2 : 0) + (a.fmt == 0 ? 0 : 1);
  switch (which) {
    case 0: return persistent_launch(k_euclid_encode<0, SC>, grid, a, s);
    case 1: return persistent_launch(k_euclid_encode<1, SC>, grid, a, s);
    case 2: return persistent_launch(k_euclid_encode_ef<0, SC>, grid, a, s);
    case 3: return persistent_launch(k_euclid_encode_ef<1, SC>, grid, a, s);
    case 4: return persistent_launch(k_rank_encode<0, SC>, grid, a, s);
    case 5: return persistent_launch(k_rank_encode<1, SC>, grid, a, s);
    case 6: return persistent_launch(k_rank_encode_ef<0, SC>, grid, a, s);
    default: return persistent_launch(k_rank_encode_ef<1, SC>, grid, a, s);
  }
}

hipError_t launch_fused(const FusedArgs& a, int grid, hipStream_t s) {
  hipError_t e;
  if (a.fmt == 2) {
    // FP4 (tensor amax, 16-element block scales): the encode, with or
    // without error feedback; the rank-k decode at 4 or 8 replicas
    if (a.mode == 0) {
      if (a.resid)
        e = a.lr ? persistent_launch(k_rank_encode_ef<2, 0>, grid, a, s)
                 : persistent_launch(k_euclid_encode_ef<2, 0>, grid, a, s);
      else
        e = a.lr ? persistent_launch(k_rank_encode<2, 0>, grid, a, s)
                 : persistent_launch(k_euclid_encode<2, 0>, grid, a, s);
    } else {
      if (!a.lr || (a.R != 4 && a.R != 8)) return hipErrorInvalidValue;
      e = a.R == 4 ? persistent_launch(k_rank_decode<2, 4, 0>, grid, a, s)
                   : persistent_launch(k_rank_decode<2, 8, 0>, grid, a, s);
    }
  } else if (a.mode == 0) {
    e = a.scaling == 0 ? launch_encode<0>(a, grid, s) : launch_encode<1>(a, grid, s);
  } else if (a.fmt == 0) {
    e = a.lr ? launch_decode<0, true>(a, grid, s) : launch_decode<0, false>(a, grid, s);
  } else {
    e = a.lr ? launch_decode<1, true>(a, grid, s) : launch_decode<1, false>(a, grid, s);
  }
  return e;
}

template <int FMT, int SC>
static void launch_group_decode(const FusedArgs* table, int n, const GroupEpochs& ep, int R, int grid,
                                hipStream_t s) {
  const dim3 gd((unsigned)grid), bd(512);
  switch (R) {
    case 4: hipLaunchKernelGGL((k_rank_group<FMT, false, 4, SC>), gd, bd, 0, s, table, n, ep); break;
    case 8: hipLaunchKernelGGL((k_rank_group<FMT, false, 8, SC>), gd, bd, 0, s, table, n, ep); break;
    case 16: hipLaunchKernelGGL((k_rank_group<FMT, false, 16, SC>), gd, bd, 0, s, table, n, ep); break;
    default: hipLaunchKernelGGL((k_rank_group<FMT, false, 0, SC>), gd, bd, 0, s, table, n, ep); break;
  }
}

hipError_t launch_group(const FusedArgs* table, int n, const GroupEpochs& ep, int decode, int fmt, int scaling, int R,
                        int grid, hipStream_t s) {
  const dim3 gd((unsigned)grid), bd(512);
  if (!decode) {
    if (fmt == 0) {
      if (scaling == 0) hipLaunchKernelGGL((k_rank_group<0, true, 0, 0>), gd, bd, 0, s, table, n, ep);
      else hipLaunchKernelGGL((k_rank_group<0, true, 0, 1>), gd, bd, 0, s, table, n, ep);
    } else {
      if (scaling == 0) hipLaunchKernelGGL((k_rank_group<1, true, 0, 0>), gd, bd, 0, s, table, n, ep);
      else hipLaunchKernelGGL((k_rank_group<1, true, 0, 1>), gd, bd, 0, s, table, n, ep);
    }
  } else if (fmt == 0) {
    if (scaling == 0) launch_group_decode<0, 0>(table, n, ep, R, grid, s);
    else launch_group_decode<0, 1>(table, n, ep, R, grid, s);
  } else {
    if (scaling == 0) launch_group_decode<1, 0>(table, n, ep, R, grid, s);
    else launch_group_decode<1, 1>(table, n, ep, R, grid, s);
  }
  return hipGetLastError();
}

// Workgroups of the fused kernels that the current device can hold at once:
// the smallest occupancy of any variant, single-layer and grouped (one query
// per kernel), times the compute units; 0 if a query fails.
int fused_resident_groups() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev]) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  const void* kernels[] = {
#define GIFT_ENC(S)                                                                                       \
  reinterpret_cast<const void*>(k_rank_encode<0, S>), reinterpret_cast<const void*>(k_rank_encode<1, S>),      \
      reinterpret_cast<const void*>(k_rank_encode_ef<0, S>), reinterpret_cast<const void*>(k_rank_encode_ef<1, S>), \
      reinterpret_cast<const void*>(k_euclid_encode<0, S>), reinterpret_cast<const void*>(k_euclid_encode<1, S>),  \
      reinterpret_cast<const void*>(k_euclid_encode_ef<0, S>), reinterpret_cast<const void*>(k_euclid_encode_ef<1, S>)
      GIFT_ENC(0), GIFT_ENC(1),
#undef GIFT_ENC
#define GIFT_DEC(F, S)                                                                                      \
  reinterpret_cast<const void*>(k_rank_decode<F, 4, S>), reinterpret_cast<const void*>(k_rank_decode<F, 8, S>), \
      reinterpret_cast<const void*>(k_rank_decode<F, 16, S>), reinterpret_cast<const void*>(k_rank_decode<F, 0, S>), \
      reinterpret_cast<const void*>(k_euclid_decode<F, 4, S>), reinterpret_cast<const void*>(k_euclid_decode<F, 8, S>), \
      reinterpret_cast<const void*>(k_euclid_decode<F, 16, S>), reinterpret_cast<const void*>(k_euclid_decode<F, 0, S>)
      GIFT_DEC(0, 0), GIFT_DEC(0, 1), GIFT_DEC(1, 0), GIFT_DEC(1, 1),
#undef GIFT_DEC
  // the grouped launches of the same bodies
#define GIFT_GRP(F, S)                                                                                         \
  reinterpret_cast<const void*>(k_rank_group<F, true, 0, S>), reinterpret_cast<const void*>(k_rank_group<F, false, 4, S>), \
      reinterpret_cast<const void*>(k_rank_group<F, false, 8, S>),                                                \
      reinterpret_cast<const void*>(k_rank_group<F, false, 16, S>), reinterpret_cast<const void*>(k_rank_group<F, false, 0, S>)
      GIFT_GRP(0, 0), GIFT_GRP(0, 1), GIFT_GRP(1, 0), GIFT_GRP(1, 1),
#undef GIFT_GRP
      // the FP4 payload
      reinterpret_cast<const void*>(k_rank_encode<2, 0>), reinterpret_cast<const void*>(k_euclid_encode<2, 0>),
      reinterpret_cast<const void*>(k_rank_encode_ef<2, 0>), reinterpret_cast<const void*>(k_euclid_encode_ef<2, 0>),
      reinterpret_cast<const void*>(k_rank_decode<2, 4, 0>), reinterpret_cast<const void*>(k_rank_decode<2, 8, 0>)
  };
  int per_cu = 1 << 30;
  for (const void* k : kernels) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 512, 0) != hipSuccess) return 0;
    per_cu = n < per_cu ? n : per_cu;
  }
  cache[dev] = per_cu * cus;
  return cache[dev];
}

}  // namespace gift
