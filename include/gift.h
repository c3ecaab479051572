/*
 * gift.h -- C ABI of libgift, an MI355X (gfx950) library for the
 * data-parallel hot path of GIFT: geometry-aware FP8 encode / decode of one
 * layer's weight gradient.
 *
 * Sources (cited by page title and equation / section):
 *   [Note] "GIFT 阅读笔记:量化用的坐标系,比量化器本身更重要" (zhongzhuzhou.org)
 *   [Abs]  "GIFT: Geometry-Informed Low-precision Gradient Communication for
 *          LLM Pretraining" (shd-paper.top abstract page)
 *
 * Conventions for every call:
 *   - Device pointers ("d_") are allocated and owned by the caller; the
 *     library never allocates or frees device memory.  Host pointers ("h_")
 *     are read or written during the call only.
 *   - Matrices are row-major.  A leading dimension ("ld") is in elements and
 *     must be >= the row length and a multiple of 4 (fp32) or 8 (bf16);
 *     device pointers must be 16-byte aligned.  d_in must be a multiple of 8.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns without waiting, except where noted.
 *   - All argument checks happen before anything is enqueued: on any error
 *     return nothing has been enqueued.  A HIP launch failure returns
 *     GIFT_ERR_HIP; gift_last_hip_error() then gives the hipError_t.
 *   - Non-finite data is not reported synchronously: the affected scale is
 *     written as NaN, its codes as 0x7F, decode propagates NaN, and the
 *     layer's sticky device flag GIFT_FLAG_NONFINITE is set
 *     (gift_layer_flags()).
 *   - Handles are not thread-safe; distinct handles are independent.
 *     Calls that share a workspace buffer must be ordered on one stream.
 */
#ifndef GIFT_H
#define GIFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gift_status;
typedef void* gift_stream_t;                 /* a hipStream_t */
typedef struct gift_layer* gift_layer_t;       /* opaque host handle */
typedef struct gift_profiler* gift_profiler_t; /* opaque host handle */
typedef struct gift_bucket* gift_bucket_t;     /* opaque host handle */

enum {
  GIFT_OK = 0,
  GIFT_ERR_INVALID_ARG = 1, /* bad pointer, shape, stride, alignment or enum */
  GIFT_ERR_WORKSPACE = 2,   /* state or workspace buffer smaller than required */
  GIFT_ERR_NOT_READY = 3,   /* encode/decode of a non-Euclidean layer before its first refresh,
                               or a refresh before any statistics were committed */
  GIFT_ERR_NUMERICAL = 4,   /* reserved for host-detected numerical failure */
  GIFT_ERR_UNSUPPORTED = 5, /* valid but not implemented combination */
  GIFT_ERR_HIP = 6          /* a HIP runtime call failed */
};

/* Change of coordinates applied before quantisation ([Note] Algorithm 1). */
enum gift_transform {
  GIFT_EUCLID = 0,          /* none: the Euclidean FP8 baseline ([Note] Algorithm 1, the Euclidean branch) */
  GIFT_DIAG = 1,            /* T_A = diag((A_ii + lam)^-1/2) ([Note] §简化二, Table II "diagonal") */
  GIFT_LOWRANK = 2,         /* T_A = U diag((Lt)^-1/2 - rho^-1/2) U^T + rho^-1/2 I, rank k
                               ([Note] §简化二, Eq. (17); the form is this library's reading) */
  GIFT_CHOL_INPUT = 3,      /* T_A = L_A^-T, A + lam I = L_A L_A^T ([Note] Eq. (7), (16)) */
  GIFT_CHOL_TWOSIDED = 4    /* W~ = L_G^-1 W L_A^-T ([Note] Eq. (11)); map back Eq. (14) */
};

/* FP8 ([Note] §前置知识); E2M1 = FP4 ([Abs] NVFP4), only through the _fp4 calls */
enum gift_format { GIFT_E4M3 = 0, GIFT_E5M2 = 1, GIFT_E2M1 = 2 };
/* BLOCK16: the FP4 payload's 16-element row blocks (gift_payload_bytes only);
 * BLOCK512: 512 consecutive elements of a tensor (gift_bucket_* only) */
enum gift_scaling {
  GIFT_SCALE_TENSOR = 0,
  GIFT_SCALE_BLOCK128 = 1,
  GIFT_SCALE_BLOCK16 = 2,
  GIFT_SCALE_BLOCK512 = 3
};
enum gift_dtype { GIFT_BF16 = 0, GIFT_FP32 = 1 };
enum gift_side { GIFT_SIDE_A = 0, GIFT_SIDE_G = 1 };      /* input / output statistics */
enum { GIFT_FLAG_NONFINITE = 1u, GIFT_FLAG_SPIN_TIMEOUT = 2u };

/* Description of one layer.  d_out x d_in is the shape of W_g. */
typedef struct gift_layer_desc {
  int32_t d_out;       /* m, rows of W_g                                   */
  int32_t d_in;        /* d, columns of W_g; multiple of 8                 */
  int32_t transform;   /* enum gift_transform                              */
  int32_t rank;        /* k for GIFT_LOWRANK (32 on the pages), 1..d_in    */
  int32_t oversample;  /* p: the test matrix has l = min(k + p, d) columns */
  int32_t power_iters; /* q: re-orthonormalised products after Y = A Omega */
  float ema_decay;     /* beta in [0, 1): A <- beta A + (1 - beta) A_batch  */
  float damping_rel;   /* lam = damping_rel * tr(A) / d (also for G)       */
  int32_t flags;       /* GIFT_LAYER_* bits, 0 for none                    */
} gift_layer_desc;

/* Layer flags.
 * GIFT_LAYER_TRANSIENT_STATS: every statistics window is accumulated and
 *   committed in one gift_accumulate_stats call (commit nonzero, nothing
 *   pending).  The window's running sum S then lives in the caller's
 *   workspace for the duration of that call, and the state holds only the
 *   committed A (and G): d_in^2 (+ d_out^2) fp32 less per layer, which is
 *   what lets many layers share one workspace.  Any other statistics call
 *   on such a layer returns GIFT_ERR_INVALID_ARG. */
enum { GIFT_LAYER_TRANSIENT_STATS = 1 };

/* ---------------------------------------------------------------------------
 * Layer state.
 * gift_layer_state_bytes: bytes of the caller-owned device state buffer for
 * this layer (the window sums S_A [and S_G] unless GIFT_LAYER_TRANSIENT_STATS,
 * the committed A [and G], the factor, flags) and the largest workspace any
 * call on this layer needs.  Both are multiples of 256.
 * gift_layer_create: binds `d_state` (>= state_bytes, 256-byte aligned) to a
 * new host handle; enqueues the zeroing of the state on `stream`.
 * The state is plain device memory: copying it (and the handle's host
 * counters, see gift_layer_get_counters/gift_layer_set_counters) is a
 * checkpoint.
 * ------------------------------------------------------------------------- */
gift_status gift_layer_state_bytes(const gift_layer_desc* desc, size_t* state_bytes,
                                   size_t* workspace_bytes);
gift_status gift_layer_create(const gift_layer_desc* desc, void* d_state, size_t state_bytes,
                              gift_stream_t stream, gift_layer_t* out);
gift_status gift_layer_destroy(gift_layer_t layer);
/* Host-side counters: [0] tokens pending in the A window, [1] tokens pending
 * in the G window, [2] commits of A, [3] commits of G, [4] refreshes,
 * [5] / [6] call epochs of the fused rank-k encode / decode (the tags of
 * their exchange words), [7] barrier epoch of the statistics accumulation
 * ([5]..[7] must travel with a copy of the state: the words they tag in the
 * state only grow). */
gift_status gift_layer_get_counters(gift_layer_t layer, int64_t h_counters[8]);
gift_status gift_layer_set_counters(gift_layer_t layer, const int64_t h_counters[8]);
/* Reads the sticky device flags (GIFT_FLAG_*).  Synchronises `stream`. */
gift_status gift_layer_flags(gift_layer_t layer, gift_stream_t stream, uint32_t* h_flags);
/* Device addresses inside the state buffer, for inspection and for
 * stage-isolated tests.  Any pointer argument may be NULL.
 *   A, G:       fp32 [d][d] / [m][m] committed statistics (EMA)
 *   U:          fp32 [d][k] rank-k basis (GIFT_LOWRANK)
 *   coef:       fp32 [2k + 4]: c_enc[k], c_dec[k], rho^-1/2, rho^1/2, lam, rho
 *               (GIFT_LOWRANK); fp32 [2d]: (A_ii+lam)^-1/2, (A_ii+lam)^1/2 (GIFT_DIAG)
 *   tinv_a:     fp32 [d][d] T_A (= L_A^-T, upper triangular) (Cholesky variants)
 *   t_a:        fp32 [d][d] T_A^-1 (= L_A^T, upper triangular)
 *   lg_inv, lg: fp32 [m][m] L_G^-1 and L_G (lower triangular) (two-sided)   */
gift_status gift_layer_buffers(gift_layer_t layer, float** A, float** G, float** U, float** coef,
                               float** tinv_a, float** t_a, float** lg_inv, float** lg);
/* Marks a factor written directly into the state (through gift_layer_buffers)
 * as valid, so encode/decode accept the layer without a refresh; for
 * GIFT_LOWRANK it enqueues the repacking of U into the kernel operand
 * order on `stream`. */
gift_status gift_layer_mark_ready(gift_layer_t layer, gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Statistics.  [Note] §前置知识 Eq. (4): A = E[a a^T] over the layer's input
 * activations a (d_in), G = E[delta delta^T] over output gradients (d_out).
 *
 * gift_accumulate_stats: S_side += x^T x for x = d_x [T][ld] (dtype bf16 or
 * fp32, the first n columns used, n = d_in for side A, d_out for side G),
 * and adds T to the side's pending-token count; the first call of a window
 * (nothing pending) stores x^T x instead.  If `commit` is nonzero the
 * window is then committed in the same call (see gift_commit_stats).
 * T may be 0 (no-op unless commit).  d_work / work_bytes: the layer's
 * workspace (>= its workspace_bytes); read only for layers created with
 * GIFT_LAYER_TRANSIENT_STATS, where S lives there for the call (commit must
 * be nonzero, T > 0 and nothing pending), otherwise it may be NULL.
 * gift_commit_stats: A_batch = S / count; A = A_batch on the first commit,
 * else A = beta A + (1 - beta) A_batch; count = 0 (S keeps its contents
 * until the next window's first call replaces them).  GIFT_ERR_NOT_READY
 * if no tokens are pending; GIFT_ERR_INVALID_ARG on a
 * GIFT_LAYER_TRANSIENT_STATS layer (its windows commit inside
 * gift_accumulate_stats).
 * ------------------------------------------------------------------------- */
gift_status gift_accumulate_stats(gift_layer_t layer, int32_t side, const void* d_x, int32_t dtype,
                                  int64_t T, int64_t ld, int32_t commit, void* d_work, size_t work_bytes,
                                  gift_stream_t stream);
gift_status gift_commit_stats(gift_layer_t layer, int32_t side, gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Factor refresh ([Note] §简化二 Eq. (17); refreshed every K steps, Algorithm 1
 * preamble).  From the committed A (and G):
 *   GIFT_DIAG:     the two diagonal vectors.
 *   GIFT_LOWRANK:  randomized subspace iteration with the caller's test matrix
 *                  d_omega (fp32 [d_in][l], l = min(rank + oversample, d_in),
 *                  row-major): Y = A Omega, q times {Q = orth(Y), Y = A Q},
 *                  Q = orth(Y), Rayleigh-Ritz B = Q^T A Q = V Theta V^T,
 *                  U = Q V[:, :k]; Lt = max(Theta_k, 0) + lam,
 *                  rho = max((tr A - sum Theta_k)/(d - k), 0) + lam.
 *   GIFT_CHOL_*:   L_A = chol(A + lam I) in fp64, T_A = L_A^-T and L_A^T
 *                  stored in fp32; two-sided also L_G^-1 and L_G.
 * d_omega may be NULL for the other transforms.  GIFT_ERR_NOT_READY if A
 * (or G) was never committed.  A non-positive pivot sets
 * GIFT_FLAG_NONFINITE and leaves a NaN factor.
 * ------------------------------------------------------------------------- */
gift_status gift_refresh_factors(gift_layer_t layer, const float* d_omega, void* d_work,
                                 size_t work_bytes, gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Encode one replica's gradient ([Note] Algorithm 1, the geometry branch without
 * error feedback (see gift_encode_ef); the Euclidean branch's scale and quantise):
 *   W~ = W T_A (two-sided: L_G^-1 W T_A), amax per tensor or per 128x128
 *   tile (edge tiles: their valid region), r = fp32(FMAX / amax),
 *   code = FP8(fp32(w~ * r)) with round-to-nearest-even (ties to the even
 *   code), saturation at +-FMAX (also for +-Inf), NaN -> 0x7F; scale
 *   s = fp32(amax / FMAX).  amax = 0 gives r = s = 0.
 * d_W:          fp32 [d_out][ldw]
 * d_amax_in:    NULL (use the local amax) or fp32 [nblk] shared amax, e.g. the
 *               max over replicas (the AllReduceMax of Algorithm 1)
 * d_amax_out:   NULL or fp32 [nblk]: the local amax of W~
 * d_codes:      uint8 [d_out][d_in]; NULL = only compute d_amax_out
 * d_scales:     fp32 [nblk]; nblk = 1 (tensor) or ceil(m/128) * ceil(d/128),
 *               row-major over tiles
 * d_whitened:   NULL or fp32 [d_out][d_in]: receives W~ (inspection)
 * d_work:       workspace of >= the layer's workspace_bytes
 * ------------------------------------------------------------------------- */
gift_status gift_encode(gift_layer_t layer, const float* d_W, int64_t ldw, int32_t fmt,
                        int32_t scaling, const float* d_amax_in, float* d_amax_out,
                        uint8_t* d_codes, float* d_scales, float* d_whitened, void* d_work,
                        size_t work_bytes, gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Encode with error feedback ([Note] Algorithm 1, the geometry branch with its error-feedback steps: the
 * residual of the previous step is added in the whitened coordinates):
 *   U~ = fp32(W~ + R), amax, scale and codes of U~ exactly as gift_encode
 *   computes them for W~, then R <- fp32(U~ - s dec(code)) (the difference
 *   rounded once).
 * d_resid:      fp32 [d_out][d_in] (leading dimension d_in), caller-owned,
 *               one per worker (replica); zero it before the first step.
 *               Read, and rewritten when d_codes is given; an amax-only call
 *               (d_codes NULL: d_amax_out receives the amax of U~, e.g. for
 *               the AllReduceMax of a shared scale) leaves it unchanged.
 *               Must not overlap d_W, d_whitened, d_codes or d_scales.
 * d_whitened:   receives W~ (without the residual).
 * Other arguments, errors and the NULL-resid case as gift_encode
 * (d_resid NULL: GIFT_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------- */
gift_status gift_encode_ef(gift_layer_t layer, const float* d_W, int64_t ldw, int32_t fmt,
                           int32_t scaling, const float* d_amax_in, float* d_amax_out,
                           uint8_t* d_codes, float* d_scales, float* d_whitened, float* d_resid,
                           void* d_work, size_t work_bytes, gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Decode-reduce R replica payloads ([Note] Eq. (1) and Algorithm 1, the
 * geometry branch's AllReduceSum, Dequantize / N and map back; the payloads
 * of R workers held in one GPU's memory):
 *   U = (1/R) sum_{r=0..R-1} s_r dec(q_r) (fp32, r in increasing order),
 *   W^ = U T_A^-1 (two-sided: L_G U L_A^T), written as fp32.
 * d_codes:      replica r at d_codes + r * code_stride (bytes), [d_out][d_in]
 * d_scales:     replica r at d_scales + r * scale_stride (elements), [nblk]
 * d_out:        fp32 [d_out][ldo]
 * ------------------------------------------------------------------------- */
gift_status gift_decode_reduce(gift_layer_t layer, const uint8_t* d_codes, int64_t code_stride,
                               const float* d_scales, int64_t scale_stride, int32_t R,
                               int32_t fmt, int32_t scaling, float* d_out, int64_t ldo,
                               void* d_work, size_t work_bytes, gift_stream_t stream);

/* Payload size of one replica: d_out * d_in code bytes + 4 * nblk scale
 * bytes (FP8); d_out * d_in / 2 + d_out * d_in / 16 + 4 (GIFT_SCALE_BLOCK16,
 * the FP4 payload). */
size_t gift_payload_bytes(int32_t d_out, int32_t d_in, int32_t scaling);

/* ---------------------------------------------------------------------------
 * FP4 payload ([Abs]: NVFP4 named as a low-precision communication format;
 * [Note] summary: the coordinate change carries over to FP4.  The pages
 * leave the layout open; this library's reading):
 *   elements E2M1 (OCP 4-bit float: values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6},
 *   round to nearest, ties to the even code, saturating, NaN -> +0),
 *   blocks of 16 consecutive elements of a row, each with an E4M3 scale,
 *   one fp32 scale per tensor:
 *     g     = fp32(amax_T / (6 * 448)),  sig_b = fp32(amax_b / (6 g)),
 *     sc_b  = E4M3(sig_b),  S_b = fp32(dec(sc_b) * g),
 *     code  = E2M1(fp32(x * fp32(1 / S_b)))  (x * 0 when S_b = 0),
 *   value S_b * dec(code).  A non-finite amax_T sets g = NaN, every block
 *   scale 0x7F (NaN), codes 0 and GIFT_FLAG_NONFINITE.
 * Requires d_in % 16 == 0.  Routes: the rank-k and Euclidean encodes (with
 * or without d_resid) run as one persistent launch where the layer's route
 * allows it (gift_layer_route), and so does the rank-k decode of 4 or 8
 * replicas; everything else takes the multi-kernel route.  Codes, scales
 * and amax are the same on both routes; decoded tensors agree to within
 * fp32 rounding.
 *
 * gift_encode_fp4: W~ as gift_encode (with d_resid: U~ = W~ + R and
 * R <- fp32(U~ - S_b dec(code)), as gift_encode_ef).
 * d_amax_in:    NULL or fp32 [1]: shared amax_T (the AllReduceMax)
 * d_amax_out:   NULL or fp32 [1]: local amax_T (of U~ with d_resid)
 * d_codes:      uint8 [d_out][d_in / 2], column 2j in the low nibble;
 *               NULL = only compute d_amax_out (d_resid unchanged)
 * d_bscales:    uint8 [d_out][d_in / 16] E4M3 block scale codes
 * d_tscale:     fp32 [1]: g
 * d_whitened, d_resid, d_work: as gift_encode / gift_encode_ef (d_resid may
 *               be NULL).
 * gift_decode_reduce_fp4: U = (1/R) sum_r S_{b,r} dec(q_r) (fp32, r in
 * increasing order), then W^ as gift_decode_reduce.  Replica r at
 * d_codes + r * code_stride (bytes), d_bscales + r * bscale_stride (bytes),
 * d_tscales[r].
 * ------------------------------------------------------------------------- */
gift_status gift_encode_fp4(gift_layer_t layer, const float* d_W, int64_t ldw, const float* d_amax_in,
                            float* d_amax_out, uint8_t* d_codes, uint8_t* d_bscales, float* d_tscale,
                            float* d_whitened, float* d_resid, void* d_work, size_t work_bytes,
                            gift_stream_t stream);
gift_status gift_decode_reduce_fp4(gift_layer_t layer, const uint8_t* d_codes, int64_t code_stride,
                                   const uint8_t* d_bscales, int64_t bscale_stride,
                                   const float* d_tscales, int32_t R, float* d_out, int64_t ldo,
                                   void* d_work, size_t work_bytes, gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Flat gradient buckets: the Euclidean FP8 path of every layer outside the
 * selected set ([Note] Algorithm 1, the Euclidean branch) over a whole buffer of
 * tensors, one launch per phase.
 *
 * A bucket describes n tensors of h_numel[i] fp32 elements (each a multiple
 * of 4, >= 4) lying one after another in one flat buffer (tensor i starts at
 * element sum_{j<i} numel_j; 16-byte aligned buffers).  Codes use the same
 * offsets (1 byte per element).  Scales are numbered tensor by tensor:
 *   GIFT_SCALE_TENSOR:   one per tensor;
 *   GIFT_SCALE_BLOCK512: one per 512 consecutive elements of a tensor
 *                        (blocks restart at every tensor; the last block of
 *                        a tensor may be shorter): the per-block Euclidean
 *                        baseline of [Note] (experiment setup, block 512).
 * The quantiser is gift_encode's (R4 of the scale, RNE saturating codes,
 * NaN scale and 0x7F codes for a non-finite amax, GIFT_FLAG_NONFINITE in the
 * bucket's flag word).
 *
 * gift_bucket_create: d_table = caller-owned device memory of
 *   gift_bucket_table_bytes(n) bytes, 256-byte aligned (the offset tables
 *   and the flag word); the call copies the tables and synchronises stream.
 * gift_bucket_sizes: total elements, number of scales, and the workspace
 *   bytes gift_bucket_encode needs for a local amax.
 * gift_bucket_amax: d_amax_out fp32 [nscales] = the amax of every scale
 *   block (for the AllReduceMax of Algorithm 1's Euclidean branch).
 * gift_bucket_encode: codes uint8 [numel] and scales fp32 [nscales] with the
 *   shared amax d_amax_in (NULL: the local one, computed first into d_work);
 *   d_amax_out NULL or fp32 [nscales] receives the local amax.
 * gift_bucket_decode_reduce: U = (1/R) sum_r s_r dec(q_r) (fp32, r in
 *   increasing order) into d_out fp32 [numel]; replica r at
 *   d_codes + r * code_stride (bytes) and d_scales + r * scale_stride.
 * ------------------------------------------------------------------------- */
size_t gift_bucket_table_bytes(int32_t n);
gift_status gift_bucket_create(int32_t n, const int64_t* h_numel, int32_t scaling, void* d_table,
                               size_t table_bytes, gift_stream_t stream, gift_bucket_t* out);
gift_status gift_bucket_destroy(gift_bucket_t bucket);
gift_status gift_bucket_sizes(gift_bucket_t bucket, int64_t* h_numel, int64_t* h_nscales,
                              size_t* h_workspace_bytes);
gift_status gift_bucket_flags(gift_bucket_t bucket, gift_stream_t stream, uint32_t* h_flags);
gift_status gift_bucket_amax(gift_bucket_t bucket, const float* d_grad, float* d_amax_out,
                             gift_stream_t stream);
gift_status gift_bucket_encode(gift_bucket_t bucket, const float* d_grad, int32_t fmt,
                               const float* d_amax_in, float* d_amax_out, uint8_t* d_codes,
                               float* d_scales, void* d_work, size_t work_bytes, gift_stream_t stream);
/* gift_bucket_encode_static: gift_bucket_encode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * It allocates nothing: the local amax slots live in a scratch array of
 * 1 MiB compiled into the library (one per device, held until the process
 * ends), so a bucket may have at most 262144 scales when the local amax is
 * needed (d_amax_in NULL or d_amax_out given); more gives GIFT_ERR_WORKSPACE
 * with nothing enqueued.  Codes and scales equal gift_bucket_encode's.
 * Every call on a device shares that device's array (the slots are cleared
 * at the start of each call): calls that overlap in time on one device,
 * from different streams or threads, race and must not be issued. */
gift_status gift_bucket_encode_static(gift_bucket_t bucket, const float* d_grad, int32_t fmt,
                                      const float* d_amax_in, float* d_amax_out, uint8_t* d_codes,
                                      float* d_scales, gift_stream_t stream);
gift_status gift_bucket_decode_reduce(gift_bucket_t bucket, const uint8_t* d_codes, int64_t code_stride,
                                      const float* d_scales, int64_t scale_stride, int32_t R,
                                      int32_t fmt, float* d_out, gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Grouped rank-k layers ([Note] Algorithm 1: every step encodes, reduces and
 * maps back each selected layer; §实验设置: 13 fc2 layers take the rank-32
 * path): the encodes of several GIFT_LOWRANK layers in one launch, and their
 * decode-reduces in one launch, on the single-launch kernels (every layer
 * must take the fused route: gift_layer_route gives 1 for its ld's).  Each
 * layer is the same computation as gift_encode / gift_decode_reduce with
 * the local amax (results bit-identical to those calls); a workgroup moves
 * to its tile of the next layer as soon as its part of a layer is done.
 *
 * A group binds fixed buffers, given per layer in gift_group_item:
 *   d_W, ldw:            fp32 [d_out][ldw] gradient to encode
 *   d_codes, d_scales:   this worker's payload (written by the encode)
 *   d_rcodes, code_stride, d_rscales, scale_stride: the R payloads to decode
 *                        (replica r at + r * stride, as gift_decode_reduce)
 *   d_out, ldo:          fp32 [d_out][ldo] decoded mean
 * gift_group_create: n <= 32 distinct layers, one format / scaling / R for
 * all; d_table = caller-owned device memory of gift_group_table_bytes(n)
 * bytes, 256-byte aligned; the call copies the launch table into it and
 * synchronises `stream`.  GIFT_ERR_UNSUPPORTED if a layer cannot take the
 * fused route.  The layers may be refreshed later; encode / decode return
 * GIFT_ERR_NOT_READY while any of them has no factor.  Calls on a group and
 * on its layers must be ordered on one stream.
 * ------------------------------------------------------------------------- */
typedef struct gift_group* gift_group_t;
typedef struct gift_group_item {
  gift_layer_t layer;
  const float* d_W;
  int64_t ldw;
  uint8_t* d_codes;
  float* d_scales;
  const uint8_t* d_rcodes;
  int64_t code_stride;
  const float* d_rscales;
  int64_t scale_stride;
  float* d_out;
  int64_t ldo;
} gift_group_item;
size_t gift_group_table_bytes(int32_t n);
gift_status gift_group_create(int32_t n, const gift_group_item* items, int32_t R, int32_t fmt, int32_t scaling,
                              void* d_table, size_t table_bytes, gift_stream_t stream, gift_group_t* out);
gift_status gift_group_destroy(gift_group_t group);
gift_status gift_group_encode(gift_group_t group, gift_stream_t stream);
gift_status gift_group_decode_reduce(gift_group_t group, gift_stream_t stream);

/* Scale-sync schedule ([Note] Algorithm 1, its scale-sync step): the geometry-aware
 * layers quantise with their local scale and, on a scale-sync step, with the
 * scale shared across workers (the AllReduceMax of the local amaxes: an
 * amax-only gift_encode / gift_encode_ef per replica, then the call with
 * d_amax_in).  Returns 1 when `step` (0-based) is a sync step of a schedule
 * that syncs every `period` steps starting at step 0, else 0; period <= 0
 * never syncs (the local-scale default the pages prefer). */
int32_t gift_scale_sync_due(int64_t step, int32_t period);

/* ---------------------------------------------------------------------------
 * FP8 boundary-hit profiler ([Note] §简化三, Fig. 3): over the first steps of
 * Euclidean training, count per layer how many FP8 codes hit the upper
 * boundary (|code| = the largest finite code) or the lower one (a nonzero
 * gradient element encoded as +-0), with each layer's local scale; rank the
 * layers by the mean hit rate and keep those before the sharp drop.
 *
 * gift_profiler_create: d_counts = caller-owned uint64 [n_layers][2]
 * (upper, lower); zeroing is enqueued on `stream`.
 * gift_profile_step: one step over n_layers fp32 gradients (device pointers
 * given in the host array h_grads, h_numel elements each, contiguous).
 * d_work: >= gift_profiler_workspace_bytes(n_layers, scaling, max numel).
 * gift_select_layers: synchronises `stream`, reads the counts, writes
 * h_scores[n_layers] = (upper + lower) / (numel * steps), h_order[n_layers]
 * (descending score, ties to the lower index), and the selection: the first
 * i* layers of h_order where i* maximises s_i / s_{i+1} over
 * 1 <= i <= min(n_layers - 1, max_select) (s_{i+1} = 0 < s_i counts as
 * infinite, 0/0 as 1, ties to the smallest i).
 * ------------------------------------------------------------------------- */
gift_status gift_profiler_create(int32_t n_layers, int32_t fmt, int32_t scaling, uint64_t* d_counts,
                                 gift_stream_t stream, gift_profiler_t* out);
gift_status gift_profiler_destroy(gift_profiler_t prof);
size_t gift_profiler_workspace_bytes(int32_t n_layers, int32_t scaling, int64_t max_numel);
gift_status gift_profile_step(gift_profiler_t prof, int32_t n_layers, const float* const* h_grads,
                              const int64_t* h_numel, void* d_work, size_t work_bytes,
                              gift_stream_t stream);
gift_status gift_select_layers(gift_profiler_t prof, int32_t max_select, double* h_scores,
                               int32_t* h_order, int32_t* h_selected, int32_t* h_n_selected,
                               gift_stream_t stream);

/* ---------------------------------------------------------------------------
 * Diagnostics.
 * ------------------------------------------------------------------------- */
const char* gift_status_string(gift_status s);
int32_t gift_last_hip_error(void);
/* Process-wide choice of the GIFT_LOWRANK and GIFT_EUCLID kernels: nonzero
 * (the default) uses the single-launch persistent kernels whenever every
 * 48 x 768 tile of the gradient can be resident on the device at once and
 * each buffer they address spans less than 2 GiB; zero always uses the
 * multi-kernel path (project, apply, amax, quantise / dequantise-sum,
 * project, apply).  Both give results within the same tolerances; the
 * persistent kernels keep the tile in registers and read the gradient
 * once.  Returns the previous setting.
 *
 * Persistent kernels (the fused encode / decode and the matrix-core
 * statistics kernel): their workgroups wait on words that other workgroups
 * of the same launch publish, so the whole grid must be resident at once.
 *   - The fused route is taken only when the grid fits the device (the
 *     kernels' occupancy times the compute units, or the bound set by
 *     gift_set_max_resident); otherwise the multi-kernel path runs (same
 *     results).  The statistics grid never exceeds that bound.
 *   - The library orders its persistent launches device-wide: a persistent
 *     call on a stream other than the previous one's first waits for that
 *     stream (an event recorded on it at the time of the call; nothing is
 *     added while one stream carries every call; streams under graph
 *     capture are not ordered).  Two libgift persistent kernels therefore
 *     never share the device.  Kernels of other software that also wait on
 *     their own workgroups must not run beside them.
 *   - Every wait is bounded.  A wait that runs out sets
 *     GIFT_FLAG_SPIN_TIMEOUT (read with gift_layer_flags) and poisons the
 *     result instead of leaving it silently wrong: the encode then gives a
 *     NaN amax / scale and 0x7F codes, the decode NaN, the statistics NaN
 *     in A (and so a NaN factor and GIFT_FLAG_NONFINITE at refresh).
 * Calls on one layer must be ordered on one stream (the persistent kernels
 * exchange epoch-tagged words through the layer state). */
int32_t gift_set_fused(int32_t enable);
/* Process-wide upper bound on the workgroups that a persistent launch may
 * count on being resident at once (0, the default: the device's own limit,
 * from the occupancy of the kernels times the compute units).  For callers
 * that keep part of the device busy with work of their own, and for tests
 * of the route choice.  The fused encode / decode are taken only when all
 * their tiles fit under the bound; the statistics kernel shrinks its grid to
 * it.  Returns the previous value. */
int32_t gift_set_max_resident(int32_t max_groups);
/* Which route gift_encode (op = 0, rows of W at leading dimension ld) or
 * gift_decode_reduce (op = 1, output leading dimension ld, R replicas)
 * would take for this layer under the current settings: *h_fused = 1 for
 * the single-launch persistent kernels, 0 for the multi-kernel path. */
gift_status gift_layer_route(gift_layer_t layer, int32_t op, int64_t ld, int32_t R, int32_t* h_fused);

#ifdef __cplusplus
}
#endif
#endif /* GIFT_H */
