// Host side of libgift: argument checks, state / workspace layout, and the
// order in which each C-ABI call enqueues its kernels.  Nothing here touches
// data on the host; every step of the path runs in the kernels.
//
// GIFT 阅读笔记, Algorithm 1: per step and layer, the Euclidean branch
// (Scale -> AllReduceMax -> Q -> AllReduceSum -> Dequantize / N) or the
// geometry branch (W L_A^-T -> Scale_loc -> Q -> AllReduceSum -> Dequantize
// / N -> L_A^T).  On one GPU the collectives become: a shared amax passed in
// by the caller (AllReduceMax) and a decode that reduces R payloads held in
// device memory (AllReduceSum).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "gift_internal.hpp"

struct gift_layer {
  gift_layer_desc desc;
  gift::StateLayout sl;
  gift::WorkLayout wl;
  char* state;
  // tokens A, tokens G, commits A, commits G, refreshes, fused encode and
  // decode barrier epochs (the device counters in the state only grow)
  int64_t counters[8];
  bool ready;
};

struct gift_bucket {
  int32_t n = 0, scaling = 0;
  int64_t numel = 0, nscales = 0;
  std::vector<int64_t> host;   // chunk_start, elem_off, scale_off (n + 1 each), the source of the table copy
  gift::BucketTable t{};
};

struct gift_group {
  int32_t n = 0, R = 0, fmt = 0, scaling = 0, grid = 0;
  std::vector<gift_layer_t> layers;
  gift::FusedArgs* table = nullptr;   // device: n encode entries, then n decode entries
};

struct gift_profiler {
  int32_t n_layers, fmt, scaling;
  uint64_t* counts;
  int64_t steps;
  std::vector<int64_t> numel;
};

namespace {

thread_local int32_t g_last_hip = 0;

gift_status hip_fail(hipError_t e) {
  g_last_hip = (int32_t)e;
  return GIFT_ERR_HIP;
}

#define GIFT_HIP(expr)                                  \
  do {                                                  \
    hipError_t _e = (expr);                             \
    if (_e != hipSuccess) return hip_fail(_e);          \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int lp_of(int l) { return l <= 48 ? 48 : 64; }

int l_of(const gift_layer_desc& d) { return std::min(d.rank + d.oversample, d.d_in); }

bool desc_ok(const gift_layer_desc* d) {
  if (!d) return false;
  if (d->d_out < 1 || d->d_in < 8 || d->d_in % 8 != 0) return false;
  if (d->transform < GIFT_EUCLID || d->transform > GIFT_CHOL_TWOSIDED) return false;
  if (!(d->ema_decay >= 0.0f && d->ema_decay < 1.0f)) return false;
  if (!(d->damping_rel >= 0.0f) || !std::isfinite(d->damping_rel)) return false;
  if (d->flags & ~(int32_t)GIFT_LAYER_TRANSIENT_STATS) return false;   // unknown flag bits
  if (d->transform == GIFT_LOWRANK) {
    if (d->rank < 1 || d->rank > 32 || d->rank > d->d_in) return false;
    if (d->oversample < 0 || d->power_iters < 0 || d->power_iters > 64) return false;
    if (l_of(*d) > gift::kMaxRank || l_of(*d) < d->rank) return false;
  }
  return true;
}

int64_t nblk(int m, int d, int scaling) {
  return scaling == GIFT_SCALE_TENSOR ? 1 : gift::cdiv(m, gift::kBlock) * gift::cdiv(d, gift::kBlock);
}

int g_fused_enabled = 1;

// Scratch of gift_bucket_encode_static: the amax slots of one bucket, in a
// file-scope device array (each device that runs the library holds its own
// copy until the process ends).  Host code never passes the array's name to
// a kernel: it takes the device address once per device with
// hipGetSymbolAddress and uses that.
constexpr size_t kStaticScratchBytes = (size_t)1 << 20;   // 262144 amax slots
static __device__ __align__(256) uint32_t scratch[kStaticScratchBytes / 4];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on each device); nullptr and the HIP error on failure.
void* scratch_address(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Workgroups of the fused rank-k kernels for this shape.
int fused_groups(const gift_layer_desc& g) { return (int)gift::cdiv(g.d_out, gift::kFusedTR); }
int fused_cg(const gift_layer_desc& g) { return (int)gift::cdiv(g.d_in, gift::kFusedTC); }

// Compute units of the current device (cached per device id).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

int g_max_resident = 0;   // gift_set_max_resident (0: the device's own limit)

// Workgroups the persistent kernels may count on being resident at once.
int resident_limit(int device_limit) {
  if (device_limit <= 0) return 0;
  return g_max_resident > 0 && g_max_resident < device_limit ? g_max_resident : device_limit;
}

// Buffer resources of the fused kernels address up to 2 GiB from a base
// with 32-bit offsets (an offset of 2^31 marks a dropped access), so every
// span they touch must stay below 2^31 bytes.
bool span_ok(int m, int d, int64_t ld) {
  const int64_t lim = (int64_t)1 << 31;
  return ((int64_t)(m - 1) * ld + d) * 4 < lim && (int64_t)m * d * 4 < lim;
}

// The fused path keeps every tile resident (its workgroups wait on one
// another), so it is taken when all tiles fit on the device at once (the
// occupancy of the fused kernels times the compute units, or the cap set by
// gift_set_max_resident) and the buffers fit the 32-bit offsets.  The
// Euclidean codec takes the same kernels without the transform.
bool fused_ok(const gift_layer_desc& g, int64_t ld) {
  if (!g_fused_enabled || (g.transform != GIFT_LOWRANK && g.transform != GIFT_EUCLID)) return false;
  if (!span_ok(g.d_out, g.d_in, ld)) return false;
  const int64_t tiles = (int64_t)fused_groups(g) * fused_cg(g);
  const int cap = resident_limit(gift::fused_resident_groups());
  return cap > 0 && tiles <= cap;
}

}  // namespace

namespace gift {

int max_resident_cap() { return g_max_resident; }

// Device-wide order of the persistent launches.  Two persistent kernels
// that shared the device could each hold part of it while waiting for their
// own workgroups that have no room to start.  Launches on one stream are
// ordered by the stream; when a persistent launch comes on a different
// stream than the previous one on this device, the new stream first waits
// for the old one (an event recorded on it now, after everything it was
// given).  Nothing is added while one stream carries every call.  Streams
// under graph capture are left alone.
namespace {
struct PersistentOrder {
  std::mutex mu;
  hipStream_t last[64] = {};
  bool used[64] = {};
  hipEvent_t ev[64] = {};
};
PersistentOrder g_order;

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}
}  // namespace

hipError_t order_persistent(hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_order.mu);
  if (g_order.used[dev] && g_order.last[dev] != s && !capturing(s)) {
    hipStream_t prev = g_order.last[dev];
    if (!g_order.ev[dev]) {
      e = hipEventCreateWithFlags(&g_order.ev[dev], hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    if (!capturing(prev) && hipEventRecord(g_order.ev[dev], prev) == hipSuccess) {
      e = hipStreamWaitEvent(s, g_order.ev[dev], 0);
      if (e != hipSuccess) return e;
    } else {
      // the previous stream is no longer valid (destroyed) or is being
      // captured: order against everything on the device instead
      (void)hipGetLastError();
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return e;
    }
  }
  g_order.last[dev] = s;
  g_order.used[dev] = true;
  return hipSuccess;
}

StateLayout state_layout(const gift_layer_desc& g) {
  StateLayout s;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t d = (size_t)g.d_in, m = (size_t)g.d_out;
  const bool stats_a = g.transform != GIFT_EUCLID;
  const bool stats_g = g.transform == GIFT_CHOL_TWOSIDED;
  const bool keep_s = (g.flags & GIFT_LAYER_TRANSIENT_STATS) == 0;   // window sums in the state
  s.flags = take(256);
  if (stats_a) {
    if (keep_s) s.S_A = take(d * d * 4);
    s.A = take(d * d * 4);
    s.ssync = take(kStatsMaxGroups * 4);   // statistics: one grow-only flag per workgroup
  }
  if (stats_g) {
    if (keep_s) s.S_G = take(m * m * 4);
    s.G = take(m * m * 4);
  }
  if (g.transform == GIFT_LOWRANK) {
    s.U = take(d * 32 * 4);
    s.coef = take(68 * 4);
    const size_t ncb = (size_t)cdiv((int64_t)d, 32);
    s.ub = take(ncb * kUPackBytes);
    s.ua = take(ncb * kUPackBytes);
    // tagged projection partials [tiles][48 x 32], then the row-group sums
    // [row groups][48 x 32]
    s.xpub = take((size_t)fused_groups(g) * (fused_cg(g) + 1) * kFusedTR * 32 * 8);
  }
  if (g.transform == GIFT_LOWRANK || g.transform == GIFT_EUCLID) {
    const size_t tiles = (size_t)fused_groups(g) * fused_cg(g);   // [tiles][16] + the per-tensor copies
    s.apub = take((tiles * 16 + (size_t)kAmaxCopies * amax_copy_stride((int)tiles)) * 8);
  }
  if (g.transform == GIFT_DIAG) s.coef = take(2 * d * 4);
  if (g.transform == GIFT_CHOL_INPUT || g.transform == GIFT_CHOL_TWOSIDED) {
    s.tinv_a = take(d * d * 4);
    s.t_a = take(d * d * 4);
  }
  if (stats_g) {
    s.lg_inv = take(m * m * 4);
    s.lg = take(m * m * 4);
  }
  s.total = off;
  return s;
}

WorkLayout work_layout(const gift_layer_desc& g) {
  WorkLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t d = (size_t)g.d_in, m = (size_t)g.d_out;
  w.amax = take((size_t)nblk((int)m, (int)d, GIFT_SCALE_BLOCK128) * 4);
  if (g.transform != GIFT_EUCLID) w.tile = take(m * d * 4);
  if (g.transform == GIFT_CHOL_TWOSIDED) w.tmp = take(m * d * 4);
  if (g.transform == GIFT_LOWRANK) {
    w.ppart = take((size_t)cdiv((int64_t)d, kProjChunk) * m * 32 * 8);
    w.pc = take(m * 32 * 4);
    const size_t lp = (size_t)lp_of(l_of(g));
    w.Y = take(d * lp * 8);
    w.Q = take(d * lp * 8);
    w.Z = take(d * lp * 8);
    w.small = take((64 + 64 * 64 + 64) * 8);
    w.gpart = take(((size_t)cdiv((int64_t)d, kGramRows) + 1) * lp * lp * 8);   // partials + their sum
    w.apart = take(std::max((size_t)aq_splits((int)d) * d * lp * 8, (size_t)aq32_splits((int)d) * d * lp * 4));
  }
  if (g.transform == GIFT_CHOL_INPUT || g.transform == GIFT_CHOL_TWOSIDED) {
    const size_t n = g.transform == GIFT_CHOL_TWOSIDED ? std::max(d, m) : d;
    w.chol = take(n * n * 8);
    w.chol2 = take(n * n * 8 + 256);   // + the damping scalar
  }
  w.total = std::max<size_t>(off, 256);
  if ((g.flags & GIFT_LAYER_TRANSIENT_STATS) && g.transform != GIFT_EUCLID) {
    const size_t n = g.transform == GIFT_CHOL_TWOSIDED ? std::max(d, m) : d;
    w.stats = 0;
    w.total = std::max(w.total, align256(n * n * 4));
  }
  return w;
}

}  // namespace gift

using gift::cdiv;

extern "C" {

const char* gift_status_string(gift_status s) {
  switch (s) {
    case GIFT_OK: return "ok";
    case GIFT_ERR_INVALID_ARG: return "invalid argument";
    case GIFT_ERR_WORKSPACE: return "state or workspace buffer too small";
    case GIFT_ERR_NOT_READY: return "not ready (no committed statistics or no factor yet)";
    case GIFT_ERR_NUMERICAL: return "numerical failure";
    case GIFT_ERR_UNSUPPORTED: return "unsupported combination";
    case GIFT_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t gift_last_hip_error(void) { return g_last_hip; }

int32_t gift_set_fused(int32_t enable) {
  const int32_t old = g_fused_enabled;
  g_fused_enabled = enable ? 1 : 0;
  return old;
}

int32_t gift_set_max_resident(int32_t max_groups) {
  const int32_t old = g_max_resident;
  g_max_resident = max_groups > 0 ? max_groups : 0;
  return old;
}

gift_status gift_layer_route(gift_layer_t L, int32_t op, int64_t ld, int32_t R, int32_t* h_fused) {
  if (!L || !h_fused || (op != 0 && op != 1) || ld < L->desc.d_in) return GIFT_ERR_INVALID_ARG;
  bool f = fused_ok(L->desc, ld);
  if (op == 1) f = f && R >= 1 && R <= 64;
  *h_fused = f ? 1 : 0;
  return GIFT_OK;
}

size_t gift_payload_bytes(int32_t d_out, int32_t d_in, int32_t scaling) {
  if (d_out < 0 || d_in < 0) return 0;
  if (scaling == GIFT_SCALE_BLOCK16)   // FP4: half a byte per code, one E4M3 byte per 16, the tensor scale
    return (size_t)d_out * (size_t)d_in / 2 + (size_t)d_out * (size_t)d_in / 16 + 4;
  return (size_t)d_out * (size_t)d_in + 4 * (size_t)nblk(d_out, d_in, scaling);
}

gift_status gift_layer_state_bytes(const gift_layer_desc* desc, size_t* state_bytes, size_t* workspace_bytes) {
  if (!desc_ok(desc)) return GIFT_ERR_INVALID_ARG;
  if (state_bytes) *state_bytes = gift::state_layout(*desc).total;
  if (workspace_bytes) *workspace_bytes = gift::work_layout(*desc).total;
  return GIFT_OK;
}

gift_status gift_layer_create(const gift_layer_desc* desc, void* d_state, size_t state_bytes, gift_stream_t stream,
                              gift_layer_t* out) {
  if (!desc_ok(desc) || !out || !d_state || (reinterpret_cast<uintptr_t>(d_state) & 255u)) return GIFT_ERR_INVALID_ARG;
  gift::StateLayout sl = gift::state_layout(*desc);
  if (state_bytes < sl.total) return GIFT_ERR_WORKSPACE;
  gift_layer* L = new (std::nothrow) gift_layer;
  if (!L) return GIFT_ERR_INVALID_ARG;
  L->desc = *desc;
  L->sl = sl;
  L->wl = gift::work_layout(*desc);
  L->state = static_cast<char*>(d_state);
  std::memset(L->counters, 0, sizeof(L->counters));
  L->ready = desc->transform == GIFT_EUCLID;
  hipError_t e = gift::launch_fill_u32(reinterpret_cast<uint32_t*>(d_state), 0u, sl.total / 4,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    delete L;
    return hip_fail(e);
  }
  *out = L;
  return GIFT_OK;
}

gift_status gift_layer_destroy(gift_layer_t layer) {
  delete layer;
  return GIFT_OK;
}

gift_status gift_layer_get_counters(gift_layer_t L, int64_t h[8]) {
  if (!L || !h) return GIFT_ERR_INVALID_ARG;
  std::memcpy(h, L->counters, sizeof(L->counters));
  return GIFT_OK;
}

gift_status gift_layer_set_counters(gift_layer_t L, const int64_t h[8]) {
  if (!L || !h) return GIFT_ERR_INVALID_ARG;
  for (int i = 0; i < 8; ++i)
    if (h[i] < 0) return GIFT_ERR_INVALID_ARG;
  std::memcpy(L->counters, h, sizeof(L->counters));
  L->ready = L->desc.transform == GIFT_EUCLID || h[4] > 0;
  return GIFT_OK;
}

gift_status gift_layer_flags(gift_layer_t L, gift_stream_t stream, uint32_t* h_flags) {
  if (!L || !h_flags) return GIFT_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GIFT_HIP(hipMemcpyAsync(h_flags, L->state + L->sl.flags, 4, hipMemcpyDeviceToHost, s));
  GIFT_HIP(hipStreamSynchronize(s));
  return GIFT_OK;
}

gift_status gift_layer_buffers(gift_layer_t L, float** A, float** G, float** U, float** coef, float** tinv_a,
                               float** t_a, float** lg_inv, float** lg) {
  if (!L) return GIFT_ERR_INVALID_ARG;
  const gift_layer_desc& g = L->desc;
  auto at = [&](size_t off, bool present) -> float* {
    return present ? reinterpret_cast<float*>(L->state + off) : nullptr;
  };
  const bool chol = g.transform == GIFT_CHOL_INPUT || g.transform == GIFT_CHOL_TWOSIDED;
  if (A) *A = at(L->sl.A, g.transform != GIFT_EUCLID);
  if (G) *G = at(L->sl.G, g.transform == GIFT_CHOL_TWOSIDED);
  if (U) *U = at(L->sl.U, g.transform == GIFT_LOWRANK);
  if (coef) *coef = at(L->sl.coef, g.transform == GIFT_LOWRANK || g.transform == GIFT_DIAG);
  if (tinv_a) *tinv_a = at(L->sl.tinv_a, chol);
  if (t_a) *t_a = at(L->sl.t_a, chol);
  if (lg_inv) *lg_inv = at(L->sl.lg_inv, g.transform == GIFT_CHOL_TWOSIDED);
  if (lg) *lg = at(L->sl.lg, g.transform == GIFT_CHOL_TWOSIDED);
  return GIFT_OK;
}

gift_status gift_layer_mark_ready(gift_layer_t L, gift_stream_t stream) {
  if (!L) return GIFT_ERR_INVALID_ARG;
  if (L->desc.transform == GIFT_LOWRANK)
    GIFT_HIP(gift::launch_pack_u(reinterpret_cast<const float*>(L->state + L->sl.U), L->desc.d_in, L->state + L->sl.ub,
                                 L->state + L->sl.ua, static_cast<hipStream_t>(stream)));
  L->ready = true;
  return GIFT_OK;
}

// ---------------------------------------------------------------------------
// Statistics
// ---------------------------------------------------------------------------

// A (or G) from the window sum S (in the state or, for a transient-statistics
// layer, in the workspace).
static gift_status commit_window(gift_layer_t L, int32_t side, const float* S, gift_stream_t stream) {
  const gift_layer_desc& g = L->desc;
  int64_t& tokens = L->counters[side];
  int64_t& commits = L->counters[2 + side];
  if (tokens <= 0) return GIFT_ERR_NOT_READY;
  const int n = side == GIFT_SIDE_A ? g.d_in : g.d_out;
  float* A = reinterpret_cast<float*>(L->state + (side == GIFT_SIDE_A ? L->sl.A : L->sl.G));
  GIFT_HIP(gift::launch_commit(S, A, n, 1.0 / (double)tokens, g.ema_decay, commits == 0 ? 1 : 0,
                               static_cast<hipStream_t>(stream)));
  tokens = 0;
  ++commits;
  return GIFT_OK;
}

gift_status gift_commit_stats(gift_layer_t L, int32_t side, gift_stream_t stream) {
  if (!L || (side != GIFT_SIDE_A && side != GIFT_SIDE_G)) return GIFT_ERR_INVALID_ARG;
  const gift_layer_desc& g = L->desc;
  if (g.transform == GIFT_EUCLID) return GIFT_ERR_INVALID_ARG;
  if (side == GIFT_SIDE_G && g.transform != GIFT_CHOL_TWOSIDED) return GIFT_ERR_INVALID_ARG;
  if (g.flags & GIFT_LAYER_TRANSIENT_STATS) return GIFT_ERR_INVALID_ARG;   // commits inside accumulate
  return commit_window(L, side, reinterpret_cast<const float*>(L->state + (side == GIFT_SIDE_A ? L->sl.S_A : L->sl.S_G)),
                       stream);
}

gift_status gift_accumulate_stats(gift_layer_t L, int32_t side, const void* d_x, int32_t dtype, int64_t T,
                                  int64_t ld, int32_t commit, void* d_work, size_t work_bytes, gift_stream_t stream) {
  if (!L || (side != GIFT_SIDE_A && side != GIFT_SIDE_G)) return GIFT_ERR_INVALID_ARG;
  const gift_layer_desc& g = L->desc;
  if (g.transform == GIFT_EUCLID) return GIFT_ERR_INVALID_ARG;
  if (side == GIFT_SIDE_G && g.transform != GIFT_CHOL_TWOSIDED) return GIFT_ERR_INVALID_ARG;
  if (dtype != GIFT_BF16 && dtype != GIFT_FP32) return GIFT_ERR_INVALID_ARG;
  const int n = side == GIFT_SIDE_A ? g.d_in : g.d_out;
  if (T < 0) return GIFT_ERR_INVALID_ARG;
  if (T > 0) {
    if (!d_x || !aligned16(d_x) || ld < n) return GIFT_ERR_INVALID_ARG;
    if (ld % (dtype == GIFT_BF16 ? 8 : 4) != 0) return GIFT_ERR_INVALID_ARG;
  }
  const bool transient = (g.flags & GIFT_LAYER_TRANSIENT_STATS) != 0;
  const bool opens = L->counters[side] == 0;   // the first call of a window stores its sums
  float* S;
  if (transient) {
    // one call per window: accumulate into the workspace and commit
    if (!commit || !opens || T == 0) return GIFT_ERR_INVALID_ARG;
    if (!d_work || (reinterpret_cast<uintptr_t>(d_work) & 255u)) return GIFT_ERR_INVALID_ARG;
    if (work_bytes < L->wl.total) return GIFT_ERR_WORKSPACE;
    S = reinterpret_cast<float*>(static_cast<char*>(d_work) + L->wl.stats);
  } else {
    S = reinterpret_cast<float*>(L->state + (side == GIFT_SIDE_A ? L->sl.S_A : L->sl.S_G));
  }
  if (commit && L->counters[side] + T <= 0) return GIFT_ERR_NOT_READY;
  if (T > 0) {
    unsigned* ssync = reinterpret_cast<unsigned*>(L->state + L->sl.ssync);
    uint32_t* flags = reinterpret_cast<uint32_t*>(L->state + L->sl.flags);
    const unsigned epoch = (unsigned)(++L->counters[7]);
    GIFT_HIP(gift::launch_stats(d_x, dtype, T, ld, n, S, ssync, epoch, flags, device_cus(), opens,
                                static_cast<hipStream_t>(stream)));
  }
  L->counters[side] += T;
  if (commit) return commit_window(L, side, S, stream);
  return GIFT_OK;
}

// ---------------------------------------------------------------------------
// Refresh
// ---------------------------------------------------------------------------

gift_status gift_refresh_factors(gift_layer_t L, const float* d_omega, void* d_work, size_t work_bytes,
                                 gift_stream_t stream) {
  if (!L) return GIFT_ERR_INVALID_ARG;
  const gift_layer_desc& g = L->desc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.transform == GIFT_EUCLID) return GIFT_OK;
  if (L->counters[2] == 0) return GIFT_ERR_NOT_READY;
  if (g.transform == GIFT_CHOL_TWOSIDED && L->counters[3] == 0) return GIFT_ERR_NOT_READY;
  if (work_bytes < L->wl.total) return GIFT_ERR_WORKSPACE;
  if (!d_work || (reinterpret_cast<uintptr_t>(d_work) & 255u)) return GIFT_ERR_INVALID_ARG;
  char* work = static_cast<char*>(d_work);
  uint32_t* flags = reinterpret_cast<uint32_t*>(L->state + L->sl.flags);
  const float* A = reinterpret_cast<const float*>(L->state + L->sl.A);
  switch (g.transform) {
    case GIFT_DIAG:
      GIFT_HIP(gift::launch_refresh_diag(A, g.d_in, g.damping_rel, reinterpret_cast<float*>(L->state + L->sl.coef),
                                         flags, s));
      break;
    case GIFT_LOWRANK: {
      if (!d_omega || !aligned16(d_omega)) return GIFT_ERR_INVALID_ARG;
      GIFT_HIP(gift::launch_refresh_lowrank(A, g.d_in, g.rank, l_of(g), g.power_iters, g.damping_rel, d_omega,
                                            reinterpret_cast<float*>(L->state + L->sl.U),
                                            reinterpret_cast<float*>(L->state + L->sl.coef), L->wl, work, flags, s));
      GIFT_HIP(gift::launch_pack_u(reinterpret_cast<const float*>(L->state + L->sl.U), g.d_in, L->state + L->sl.ub,
                                   L->state + L->sl.ua, s));
      break;
    }
    case GIFT_CHOL_INPUT:
    case GIFT_CHOL_TWOSIDED: {
      double* wa = reinterpret_cast<double*>(work + L->wl.chol);
      double* wb = reinterpret_cast<double*>(work + L->wl.chol2);
      GIFT_HIP(gift::launch_refresh_chol(A, g.d_in, g.damping_rel, reinterpret_cast<float*>(L->state + L->sl.tinv_a),
                                         reinterpret_cast<float*>(L->state + L->sl.t_a), 0, wa, wb, flags, s));
      if (g.transform == GIFT_CHOL_TWOSIDED) {
        const float* Gm = reinterpret_cast<const float*>(L->state + L->sl.G);
        GIFT_HIP(gift::launch_refresh_chol(Gm, g.d_out, g.damping_rel,
                                           reinterpret_cast<float*>(L->state + L->sl.lg_inv),
                                           reinterpret_cast<float*>(L->state + L->sl.lg), 1, wa, wb, flags, s));
      }
      break;
    }
    default:
      return GIFT_ERR_INVALID_ARG;
  }
  L->ready = true;
  ++L->counters[4];
  return GIFT_OK;
}

// ---------------------------------------------------------------------------
// Encode / decode
// ---------------------------------------------------------------------------

// Multi-kernel map back of the reduced whitened tensor Ub (fp32 [m][d] in
// the workspace) to d_out: W^ = Ub T_A^-1 (two-sided: L_G Ub L_A^T).
static gift_status unwhiten_multi(gift_layer_t L, const float* Ub, float* d_out, int64_t ldo, char* work,
                                  hipStream_t s) {
  const gift_layer_desc& g = L->desc;
  const int m = g.d_out, d = g.d_in;
  switch (g.transform) {
    case GIFT_DIAG:
      GIFT_HIP(gift::launch_diag_apply(Ub, d, m, d, reinterpret_cast<const float*>(L->state + L->sl.coef) + d, d_out,
                                       ldo, GIFT_SCALE_TENSOR, nullptr, s));
      break;
    case GIFT_LOWRANK: {
      double* ppart = reinterpret_cast<double*>(work + L->wl.ppart);
      const float* U = reinterpret_cast<const float*>(L->state + L->sl.U);
      const float* coef = reinterpret_cast<const float*>(L->state + L->sl.coef);
      GIFT_HIP(gift::launch_lr_project(Ub, d, m, d, U, g.rank, ppart, s));
      GIFT_HIP(gift::launch_lr_apply(Ub, d, m, d, U, g.rank, ppart, reinterpret_cast<float*>(work + L->wl.pc), coef, 1,
                                     d_out, ldo, GIFT_SCALE_TENSOR, nullptr,
                                     s));
      break;
    }
    case GIFT_CHOL_INPUT:
      GIFT_HIP(gift::launch_trmm(Ub, d, m, d, reinterpret_cast<const float*>(L->state + L->sl.t_a), 0, d_out, ldo, s));
      break;
    case GIFT_CHOL_TWOSIDED: {
      float* tmp = reinterpret_cast<float*>(work + L->wl.tmp);
      GIFT_HIP(gift::launch_trmm(Ub, d, m, d, reinterpret_cast<const float*>(L->state + L->sl.t_a), 0, tmp, d, s));
      GIFT_HIP(gift::launch_trmm(tmp, d, m, d, reinterpret_cast<const float*>(L->state + L->sl.lg), 1, d_out, ldo, s));
      break;
    }
    default:
      return GIFT_ERR_INVALID_ARG;
  }
  return GIFT_OK;
}

// Encode with an optional error-feedback residual (d_resid: NULL or fp32
// [m][d], read, and rewritten when codes are produced).
static gift_status encode_impl(gift_layer_t L, const float* d_W, int64_t ldw, int32_t fmt, int32_t scaling,
                               const float* d_amax_in, float* d_amax_out, uint8_t* d_codes, float* d_scales,
                               uint8_t* d_bscales, float* d_tscale, float* d_whitened, float* d_resid, void* d_work,
                               size_t work_bytes, gift_stream_t stream) {
  if (!L) return GIFT_ERR_INVALID_ARG;
  const gift_layer_desc& g = L->desc;
  const int m = g.d_out, d = g.d_in;
  const bool fp4 = fmt == GIFT_E2M1;
  if (fp4) {
    if (scaling != GIFT_SCALE_BLOCK16 || d % 16 != 0) return GIFT_ERR_INVALID_ARG;
    if (d_codes && (!aligned16(d_codes) || !d_bscales || !d_tscale)) return GIFT_ERR_INVALID_ARG;
  } else {
    if (fmt != GIFT_E4M3 && fmt != GIFT_E5M2) return GIFT_ERR_INVALID_ARG;
    if (scaling != GIFT_SCALE_TENSOR && scaling != GIFT_SCALE_BLOCK128) return GIFT_ERR_INVALID_ARG;
    if (d_codes && (!aligned16(d_codes) || !d_scales)) return GIFT_ERR_INVALID_ARG;
  }
  if (!d_W || !aligned16(d_W) || ldw < d || ldw % 4 != 0) return GIFT_ERR_INVALID_ARG;
  if (!d_codes && !d_amax_out) return GIFT_ERR_INVALID_ARG;
  if (d_whitened && !aligned16(d_whitened)) return GIFT_ERR_INVALID_ARG;
  if (d_resid && !aligned16(d_resid)) return GIFT_ERR_INVALID_ARG;
  if (!d_work || (reinterpret_cast<uintptr_t>(d_work) & 255u)) return GIFT_ERR_INVALID_ARG;
  if (work_bytes < L->wl.total) return GIFT_ERR_WORKSPACE;
  if (!L->ready) return GIFT_ERR_NOT_READY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* work = static_cast<char*>(d_work);
  uint32_t* slots = reinterpret_cast<uint32_t*>(work + L->wl.amax);
  uint32_t* flags = reinterpret_cast<uint32_t*>(L->state + L->sl.flags);
  // FP4 takes the amax per tensor; its block amax is taken by the quantiser
  const int amax_scaling = fp4 ? GIFT_SCALE_TENSOR : scaling;
  const int64_t nb = nblk(m, d, amax_scaling);
  // the fused kernels take FP8 and FP4 (FP4: rank-k and Euclidean
  // transforms)
  const bool fused_fp4 = fp4 && (g.transform == GIFT_LOWRANK || g.transform == GIFT_EUCLID);
  if (fused_ok(g, ldw) && (!fp4 || fused_fp4)) {
    gift::FusedArgs a{};
    a.mode = 0;
    a.m = m;
    a.d = d;
    a.CG = fused_cg(g);
    a.fmt = fmt;
    a.scaling = fp4 ? GIFT_SCALE_TENSOR : scaling;   // FP4: the tensor amax (block scales in the quantiser)

    a.epoch = (unsigned)(++L->counters[5]);
    a.W = d_W;
    a.ldw = ldw;
    a.lr = g.transform == GIFT_LOWRANK;
    if (a.lr) {
      a.ub = reinterpret_cast<const uint4*>(L->state + L->sl.ub);
      a.ua = reinterpret_cast<const uint4*>(L->state + L->sl.ua);
      a.coef = reinterpret_cast<const float*>(L->state + L->sl.coef);
      a.xpub = reinterpret_cast<unsigned long long*>(L->state + L->sl.xpub);
    }

    a.apub = reinterpret_cast<unsigned long long*>(L->state + L->sl.apub);
    a.flags = flags;
    a.amax_in = d_amax_in;
    a.amax_out = d_amax_out;
    a.codes = d_codes;
    a.scales = d_scales;
    a.bscales = d_bscales;
    a.tscale = d_tscale;
    a.whitened = d_whitened;
    a.resid = d_resid;
    const int grid = fused_groups(g) * a.CG;
    hipError_t e = gift::order_persistent(s);
    if (e != hipSuccess) {
      --L->counters[5];
      return hip_fail(e);
    }
    e = gift::launch_fused(a, grid, s);
    if (e == hipSuccess) return GIFT_OK;
    --L->counters[5];
    // the runtime could not make the grid co-resident: nothing ran, take
    // the multi-kernel route
    if (e != hipErrorCooperativeLaunchTooLarge) return hip_fail(e);
    (void)hipGetLastError();
  }
  GIFT_HIP(gift::launch_fill_u32(slots, 0u, (size_t)nb, s));
  const float* X = d_W;
  int64_t ldx = ldw;
  float* out = d_whitened ? d_whitened : reinterpret_cast<float*>(work + L->wl.tile);
  // with error feedback the amax is that of W~ + R: the whitening epilogues
  // then skip theirs and one amax pass over both follows
  uint32_t* wslots = d_resid ? nullptr : slots;
  switch (g.transform) {
    case GIFT_EUCLID:
      GIFT_HIP(gift::launch_amax(d_W, ldw, m, d, amax_scaling, d_resid, slots, s));
      if (d_whitened) GIFT_HIP(hipMemcpy2DAsync(d_whitened, (size_t)d * 4, d_W, (size_t)ldw * 4, (size_t)d * 4, m,
                                                hipMemcpyDeviceToDevice, s));
      break;
    case GIFT_DIAG:
      GIFT_HIP(gift::launch_diag_apply(d_W, ldw, m, d, reinterpret_cast<const float*>(L->state + L->sl.coef), out, d,
                                       amax_scaling, wslots, s));
      X = out;
      ldx = d;
      if (d_resid) GIFT_HIP(gift::launch_amax(X, ldx, m, d, amax_scaling, d_resid, slots, s));
      break;
    case GIFT_LOWRANK: {
      double* ppart = reinterpret_cast<double*>(work + L->wl.ppart);
      const float* U = reinterpret_cast<const float*>(L->state + L->sl.U);
      const float* coef = reinterpret_cast<const float*>(L->state + L->sl.coef);
      GIFT_HIP(gift::launch_lr_project(d_W, ldw, m, d, U, g.rank, ppart, s));
      GIFT_HIP(gift::launch_lr_apply(d_W, ldw, m, d, U, g.rank, ppart, reinterpret_cast<float*>(work + L->wl.pc), coef,
                                     0, out, d, amax_scaling, wslots, s));
      X = out;
      ldx = d;
      if (d_resid) GIFT_HIP(gift::launch_amax(X, ldx, m, d, amax_scaling, d_resid, slots, s));
      break;
    }
    case GIFT_CHOL_INPUT:
    case GIFT_CHOL_TWOSIDED: {
      const float* src = d_W;
      int64_t lds = ldw;
      if (g.transform == GIFT_CHOL_TWOSIDED) {
        float* tmp = reinterpret_cast<float*>(work + L->wl.tmp);
        GIFT_HIP(gift::launch_trmm(d_W, ldw, m, d, reinterpret_cast<const float*>(L->state + L->sl.lg_inv), 1, tmp, d,
                                   s));
        src = tmp;
        lds = d;
      }
      GIFT_HIP(gift::launch_trmm(src, lds, m, d, reinterpret_cast<const float*>(L->state + L->sl.tinv_a), 0, out, d,
                                 s));
      GIFT_HIP(gift::launch_amax(out, d, m, d, amax_scaling, d_resid, slots, s));
      X = out;
      ldx = d;
      break;
    }
    default:
      return GIFT_ERR_INVALID_ARG;
  }
  if (d_codes && fp4) {
    GIFT_HIP(gift::launch_quantize_fp4(X, ldx, m, d, slots, d_amax_in, d_amax_out, d_codes, d_bscales, d_tscale,
                                       d_resid, flags, s));
  } else if (d_codes) {
    GIFT_HIP(gift::launch_quantize(X, ldx, m, d, fmt, scaling, slots, d_amax_in, d_amax_out, d_codes, d_scales,
                                   d_resid, flags, s));
  } else {
    GIFT_HIP(gift::launch_amax_out(slots, d_amax_out, nb, s));   // amax only
  }
  return GIFT_OK;
}

gift_status gift_encode(gift_layer_t L, const float* d_W, int64_t ldw, int32_t fmt, int32_t scaling,
                        const float* d_amax_in, float* d_amax_out, uint8_t* d_codes, float* d_scales,
                        float* d_whitened, void* d_work, size_t work_bytes, gift_stream_t stream) {
  if (fmt == GIFT_E2M1) return GIFT_ERR_INVALID_ARG;   // gift_encode_fp4
  return encode_impl(L, d_W, ldw, fmt, scaling, d_amax_in, d_amax_out, d_codes, d_scales, nullptr, nullptr,
                     d_whitened, nullptr, d_work, work_bytes, stream);
}

gift_status gift_encode_ef(gift_layer_t L, const float* d_W, int64_t ldw, int32_t fmt, int32_t scaling,
                           const float* d_amax_in, float* d_amax_out, uint8_t* d_codes, float* d_scales,
                           float* d_whitened, float* d_resid, void* d_work, size_t work_bytes,
                           gift_stream_t stream) {
  if (!d_resid || fmt == GIFT_E2M1) return GIFT_ERR_INVALID_ARG;
  return encode_impl(L, d_W, ldw, fmt, scaling, d_amax_in, d_amax_out, d_codes, d_scales, nullptr, nullptr,
                     d_whitened, d_resid, d_work, work_bytes, stream);
}

gift_status gift_encode_fp4(gift_layer_t L, const float* d_W, int64_t ldw, const float* d_amax_in,
                            float* d_amax_out, uint8_t* d_codes, uint8_t* d_bscales, float* d_tscale,
                            float* d_whitened, float* d_resid, void* d_work, size_t work_bytes,
                            gift_stream_t stream) {
  return encode_impl(L, d_W, ldw, GIFT_E2M1, GIFT_SCALE_BLOCK16, d_amax_in, d_amax_out, d_codes, nullptr, d_bscales,
                     d_tscale, d_whitened, d_resid, d_work, work_bytes, stream);
}

gift_status gift_decode_reduce(gift_layer_t L, const uint8_t* d_codes, int64_t code_stride, const float* d_scales,
                               int64_t scale_stride, int32_t R, int32_t fmt, int32_t scaling, float* d_out,
                               int64_t ldo, void* d_work, size_t work_bytes, gift_stream_t stream) {
  if (!L) return GIFT_ERR_INVALID_ARG;
  const gift_layer_desc& g = L->desc;
  const int m = g.d_out, d = g.d_in;
  if (fmt != GIFT_E4M3 && fmt != GIFT_E5M2) return GIFT_ERR_INVALID_ARG;
  if (scaling != GIFT_SCALE_TENSOR && scaling != GIFT_SCALE_BLOCK128) return GIFT_ERR_INVALID_ARG;
  if (R < 1 || !d_codes || !d_scales || !d_out) return GIFT_ERR_INVALID_ARG;
  if (!aligned16(d_codes) || !aligned16(d_out) || ldo < d || ldo % 4 != 0) return GIFT_ERR_INVALID_ARG;
  if (R > 1 && (code_stride < (int64_t)m * d || code_stride % 16 != 0)) return GIFT_ERR_INVALID_ARG;
  const int64_t nb = nblk(m, d, scaling);
  if (R > 1 && scale_stride < nb) return GIFT_ERR_INVALID_ARG;
  if (!d_work || (reinterpret_cast<uintptr_t>(d_work) & 255u)) return GIFT_ERR_INVALID_ARG;
  if (work_bytes < L->wl.total) return GIFT_ERR_WORKSPACE;
  if (!L->ready) return GIFT_ERR_NOT_READY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* work = static_cast<char*>(d_work);
  if (fused_ok(g, ldo) && R <= 64) {   // the kernel stages up to 64 replicas' scales
    gift::FusedArgs a{};
    a.mode = 1;
    a.m = m;
    a.d = d;
    a.CG = fused_cg(g);
    a.fmt = fmt;
    a.scaling = scaling;
    a.R = R;
    a.epoch = (unsigned)(++L->counters[6]);
    a.lr = g.transform == GIFT_LOWRANK;
    if (a.lr) {
      a.ub = reinterpret_cast<const uint4*>(L->state + L->sl.ub);
      a.ua = reinterpret_cast<const uint4*>(L->state + L->sl.ua);
      a.coef = reinterpret_cast<const float*>(L->state + L->sl.coef);
      a.xpub = reinterpret_cast<unsigned long long*>(L->state + L->sl.xpub);
    }

    a.flags = reinterpret_cast<uint32_t*>(L->state + L->sl.flags);
    a.qcodes = d_codes;
    a.code_stride = code_stride;
    a.qscales = d_scales;
    a.scale_stride = scale_stride;
    a.invR = 1.0f / (float)R;
    a.out = d_out;
    a.ldo = ldo;
    const int grid = fused_groups(g) * a.CG;
    hipError_t e = gift::order_persistent(s);
    if (e != hipSuccess) {
      --L->counters[6];
      return hip_fail(e);
    }
    e = gift::launch_fused(a, grid, s);
    if (e == hipSuccess) return GIFT_OK;
    --L->counters[6];
    if (e != hipErrorCooperativeLaunchTooLarge) return hip_fail(e);
    (void)hipGetLastError();   // not co-resident: nothing ran; multi-kernel route
  }
  if (g.transform == GIFT_EUCLID) {
    GIFT_HIP(gift::launch_dequant_sum(d_codes, code_stride, d_scales, scale_stride, R, m, d, fmt, scaling, d_out, ldo,
                                      s));
    return GIFT_OK;
  }
  float* Ub = reinterpret_cast<float*>(work + L->wl.tile);
  GIFT_HIP(gift::launch_dequant_sum(d_codes, code_stride, d_scales, scale_stride, R, m, d, fmt, scaling, Ub, d, s));
  return unwhiten_multi(L, Ub, d_out, ldo, work, s);
}

gift_status gift_decode_reduce_fp4(gift_layer_t L, const uint8_t* d_codes, int64_t code_stride,
                                   const uint8_t* d_bscales, int64_t bscale_stride, const float* d_tscales, int32_t R,
                                   float* d_out, int64_t ldo, void* d_work, size_t work_bytes, gift_stream_t stream) {
  if (!L) return GIFT_ERR_INVALID_ARG;
  const gift_layer_desc& g = L->desc;
  const int m = g.d_out, d = g.d_in;
  if (d % 16 != 0) return GIFT_ERR_INVALID_ARG;
  if (R < 1 || !d_codes || !d_bscales || !d_tscales || !d_out) return GIFT_ERR_INVALID_ARG;
  if (!aligned16(d_codes) || !aligned16(d_out) || ldo < d || ldo % 4 != 0) return GIFT_ERR_INVALID_ARG;
  if (R > 1 && (code_stride < (int64_t)m * d / 2 || code_stride % 16 != 0)) return GIFT_ERR_INVALID_ARG;
  if (R > 1 && bscale_stride < (int64_t)m * d / 16) return GIFT_ERR_INVALID_ARG;
  if (!d_work || (reinterpret_cast<uintptr_t>(d_work) & 255u)) return GIFT_ERR_INVALID_ARG;
  if (work_bytes < L->wl.total) return GIFT_ERR_WORKSPACE;
  if (!L->ready) return GIFT_ERR_NOT_READY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* work = static_cast<char*>(d_work);
  // the fused rank-k decode streams 4 or 8 replicas' FP4 payloads
  if (g.transform == GIFT_LOWRANK && (R == 4 || R == 8) && fused_ok(g, ldo)) {
    gift::FusedArgs a{};
    a.mode = 1;
    a.m = m;
    a.d = d;
    a.CG = fused_cg(g);
    a.fmt = GIFT_E2M1;
    a.scaling = GIFT_SCALE_TENSOR;
    a.R = R;
    a.epoch = (unsigned)(++L->counters[6]);
    a.lr = 1;
    a.ub = reinterpret_cast<const uint4*>(L->state + L->sl.ub);
    a.ua = reinterpret_cast<const uint4*>(L->state + L->sl.ua);
    a.coef = reinterpret_cast<const float*>(L->state + L->sl.coef);
    a.xpub = reinterpret_cast<unsigned long long*>(L->state + L->sl.xpub);
    a.flags = reinterpret_cast<uint32_t*>(L->state + L->sl.flags);
    a.qcodes = d_codes;
    a.code_stride = R > 1 ? code_stride : (int64_t)m * d / 2;
    a.qbscales = d_bscales;
    a.bscale_stride = R > 1 ? bscale_stride : (int64_t)m * d / 16;
    a.qtscales = d_tscales;
    a.invR = 1.0f / (float)R;
    a.out = d_out;
    a.ldo = ldo;
    const int grid = fused_groups(g) * a.CG;
    hipError_t e = gift::order_persistent(s);
    if (e != hipSuccess) {
      --L->counters[6];
      return hip_fail(e);
    }
    e = gift::launch_fused(a, grid, s);
    if (e == hipSuccess) return GIFT_OK;
    --L->counters[6];
    return hip_fail(e);
  }
  if (g.transform == GIFT_EUCLID) {
    GIFT_HIP(gift::launch_dequant_sum_fp4(d_codes, code_stride, d_bscales, bscale_stride, d_tscales, R, m, d, d_out,
                                          ldo, s));
    return GIFT_OK;
  }
  float* Ub = reinterpret_cast<float*>(work + L->wl.tile);
  GIFT_HIP(gift::launch_dequant_sum_fp4(d_codes, code_stride, d_bscales, bscale_stride, d_tscales, R, m, d, Ub, d,
                                        s));
  return unwhiten_multi(L, Ub, d_out, ldo, work, s);
}

// ---------------------------------------------------------------------------
// Grouped rank-k layers (one launch per phase)
// ---------------------------------------------------------------------------

size_t gift_group_table_bytes(int32_t n) {
  if (n < 1 || n > gift::kMaxGroup) return 0;
  return gift::align256((size_t)2 * n * sizeof(gift::FusedArgs));
}

gift_status gift_group_create(int32_t n, const gift_group_item* items, int32_t R, int32_t fmt, int32_t scaling,
                              void* d_table, size_t table_bytes, gift_stream_t stream, gift_group_t* out) {
  if (n < 1 || n > gift::kMaxGroup || !items || !out || !d_table || (reinterpret_cast<uintptr_t>(d_table) & 255u))
    return GIFT_ERR_INVALID_ARG;
  if (fmt != GIFT_E4M3 && fmt != GIFT_E5M2) return GIFT_ERR_INVALID_ARG;
  if (scaling != GIFT_SCALE_TENSOR && scaling != GIFT_SCALE_BLOCK128) return GIFT_ERR_INVALID_ARG;
  if (R < 1 || R > 64) return GIFT_ERR_INVALID_ARG;
  if (table_bytes < gift_group_table_bytes(n)) return GIFT_ERR_WORKSPACE;
  std::vector<gift::FusedArgs> host((size_t)2 * n);
  int grid = 0;
  for (int i = 0; i < n; ++i) {
    const gift_group_item& it = items[i];
    gift_layer_t L = it.layer;
    if (!L || L->desc.transform != GIFT_LOWRANK) return GIFT_ERR_INVALID_ARG;
    const gift_layer_desc& g = L->desc;
    const int m = g.d_out, d = g.d_in;
    const int64_t nb = nblk(m, d, scaling);
    if (!it.d_W || !aligned16(it.d_W) || it.ldw < d || it.ldw % 4 != 0) return GIFT_ERR_INVALID_ARG;
    if (!it.d_codes || !aligned16(it.d_codes) || !it.d_scales) return GIFT_ERR_INVALID_ARG;
    if (!it.d_rcodes || !aligned16(it.d_rcodes) || !it.d_rscales || !it.d_out || !aligned16(it.d_out))
      return GIFT_ERR_INVALID_ARG;
    if (it.ldo < d || it.ldo % 4 != 0) return GIFT_ERR_INVALID_ARG;
    if (R > 1 && (it.code_stride < (int64_t)m * d || it.code_stride % 16 != 0 || it.scale_stride < nb))
      return GIFT_ERR_INVALID_ARG;
    // every layer of the group runs on the fused kernels
    if (!fused_ok(g, it.ldw) || !fused_ok(g, it.ldo)) return GIFT_ERR_UNSUPPORTED;
    for (int j = 0; j < i; ++j)
      if (items[j].layer == L) return GIFT_ERR_INVALID_ARG;   // one entry per layer (one epoch per call)
    gift::FusedArgs& e = host[(size_t)i];
    e.mode = 0;
    e.m = m;
    e.d = d;
    e.CG = fused_cg(g);
    e.fmt = fmt;
    e.scaling = scaling;
    e.lr = 1;
    e.W = it.d_W;
    e.ldw = it.ldw;
    e.ub = reinterpret_cast<const uint4*>(L->state + L->sl.ub);
    e.ua = reinterpret_cast<const uint4*>(L->state + L->sl.ua);
    e.coef = reinterpret_cast<const float*>(L->state + L->sl.coef);
    e.xpub = reinterpret_cast<unsigned long long*>(L->state + L->sl.xpub);
    e.apub = reinterpret_cast<unsigned long long*>(L->state + L->sl.apub);
    e.flags = reinterpret_cast<uint32_t*>(L->state + L->sl.flags);
    e.codes = it.d_codes;
    e.scales = it.d_scales;
    gift::FusedArgs& dd = host[(size_t)(n + i)];
    dd = e;
    dd.mode = 1;
    dd.W = nullptr;
    dd.codes = nullptr;
    dd.scales = nullptr;
    dd.R = R;
    dd.qcodes = it.d_rcodes;
    dd.code_stride = R > 1 ? it.code_stride : (int64_t)m * d;
    dd.qscales = it.d_rscales;
    dd.scale_stride = R > 1 ? it.scale_stride : nb;
    dd.invR = 1.0f / (float)R;
    dd.out = it.d_out;
    dd.ldo = it.ldo;
    grid = std::max(grid, fused_groups(g) * e.CG);
  }
  gift_group* G = new (std::nothrow) gift_group;
  if (!G) return GIFT_ERR_INVALID_ARG;
  G->n = n;
  G->R = R;
  G->fmt = fmt;
  G->scaling = scaling;
  G->grid = grid;
  G->table = static_cast<gift::FusedArgs*>(d_table);
  for (int i = 0; i < n; ++i) G->layers.push_back(items[i].layer);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(d_table, host.data(), host.size() * sizeof(gift::FusedArgs), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);   // the host copy source must outlive the transfer
  if (e != hipSuccess) {
    delete G;
    return hip_fail(e);
  }
  *out = G;
  return GIFT_OK;
}

gift_status gift_group_destroy(gift_group_t G) {
  delete G;
  return GIFT_OK;
}

static gift_status group_call(gift_group_t G, int decode, gift_stream_t stream) {
  if (!G) return GIFT_ERR_INVALID_ARG;
  for (gift_layer_t L : G->layers)
    if (!L->ready) return GIFT_ERR_NOT_READY;
  gift::GroupEpochs ep{};
  for (int i = 0; i < G->n; ++i) ep.v[i] = (unsigned)(++G->layers[(size_t)i]->counters[decode ? 6 : 5]);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = gift::order_persistent(s);
  if (e == hipSuccess)
    e = gift::launch_group(G->table + (decode ? G->n : 0), G->n, ep, decode, G->fmt, G->scaling, G->R, G->grid, s);
  if (e != hipSuccess) {
    for (int i = 0; i < G->n; ++i) --G->layers[(size_t)i]->counters[decode ? 6 : 5];
    return hip_fail(e);
  }
  return GIFT_OK;
}

gift_status gift_group_encode(gift_group_t G, gift_stream_t stream) { return group_call(G, 0, stream); }
gift_status gift_group_decode_reduce(gift_group_t G, gift_stream_t stream) { return group_call(G, 1, stream); }

// ---------------------------------------------------------------------------
// Profiler
// ---------------------------------------------------------------------------

size_t gift_profiler_workspace_bytes(int32_t n_layers, int32_t scaling, int64_t max_numel) {
  (void)scaling;
  (void)max_numel;
  if (n_layers < 1) return 0;
  return gift::align256((size_t)n_layers * 4);
}

gift_status gift_profiler_create(int32_t n_layers, int32_t fmt, int32_t scaling, uint64_t* d_counts,
                                 gift_stream_t stream, gift_profiler_t* out) {
  if (n_layers < 1 || !d_counts || !out || (reinterpret_cast<uintptr_t>(d_counts) & 7u)) return GIFT_ERR_INVALID_ARG;
  if (fmt != GIFT_E4M3 && fmt != GIFT_E5M2) return GIFT_ERR_INVALID_ARG;
  if (scaling != GIFT_SCALE_TENSOR) return GIFT_ERR_UNSUPPORTED;
  gift_profiler* P = new (std::nothrow) gift_profiler;
  if (!P) return GIFT_ERR_INVALID_ARG;
  P->n_layers = n_layers;
  P->fmt = fmt;
  P->scaling = scaling;
  P->counts = d_counts;
  P->steps = 0;
  P->numel.assign((size_t)n_layers, -1);
  hipError_t e = gift::launch_fill_u32(reinterpret_cast<uint32_t*>(d_counts), 0u, (size_t)n_layers * 4,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    delete P;
    return hip_fail(e);
  }
  *out = P;
  return GIFT_OK;
}

gift_status gift_profiler_destroy(gift_profiler_t P) {
  delete P;
  return GIFT_OK;
}

gift_status gift_profile_step(gift_profiler_t P, int32_t n_layers, const float* const* h_grads,
                              const int64_t* h_numel, void* d_work, size_t work_bytes, gift_stream_t stream) {
  if (!P || n_layers != P->n_layers || !h_grads || !h_numel || !d_work) return GIFT_ERR_INVALID_ARG;
  if (work_bytes < gift_profiler_workspace_bytes(n_layers, P->scaling, 0)) return GIFT_ERR_WORKSPACE;
  for (int i = 0; i < n_layers; ++i) {
    if (h_numel[i] < 0 || (h_numel[i] > 0 && !h_grads[i])) return GIFT_ERR_INVALID_ARG;
    if (P->numel[(size_t)i] >= 0 && P->numel[(size_t)i] != h_numel[i]) return GIFT_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* slots = static_cast<uint32_t*>(d_work);
  GIFT_HIP(gift::launch_fill_u32(slots, 0u, (size_t)n_layers, s));
  for (int i = 0; i < n_layers; ++i) {
    GIFT_HIP(gift::launch_amax_flat(h_grads[i], h_numel[i], slots + i, s));
    GIFT_HIP(gift::launch_hits(h_grads[i], h_numel[i], P->fmt, slots + i,
                               reinterpret_cast<unsigned long long*>(P->counts) + 2 * i, s));
  }
  for (int i = 0; i < n_layers; ++i) P->numel[(size_t)i] = h_numel[i];
  ++P->steps;
  return GIFT_OK;
}

gift_status gift_select_layers(gift_profiler_t P, int32_t max_select, double* h_scores, int32_t* h_order,
                               int32_t* h_selected, int32_t* h_n_selected, gift_stream_t stream) {
  if (!P || max_select < 1 || !h_scores || !h_order || !h_selected || !h_n_selected) return GIFT_ERR_INVALID_ARG;
  if (P->steps == 0) return GIFT_ERR_NOT_READY;
  const int n = P->n_layers;
  std::vector<uint64_t> c((size_t)n * 2);
  hipStream_t s = static_cast<hipStream_t>(stream);
  GIFT_HIP(hipMemcpyAsync(c.data(), P->counts, c.size() * 8, hipMemcpyDeviceToHost, s));
  GIFT_HIP(hipStreamSynchronize(s));
  for (int i = 0; i < n; ++i) {
    double den = (double)P->numel[(size_t)i] * (double)P->steps;
    h_scores[i] = den > 0 ? ((double)c[2 * (size_t)i] + (double)c[2 * (size_t)i + 1]) / den : 0.0;
  }
  std::vector<int32_t> order((size_t)n);
  for (int i = 0; i < n; ++i) order[(size_t)i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return h_scores[a] > h_scores[b]; });
  int best_i = 1;
  double best = -1.0;
  for (int i = 1; i <= std::min(n - 1, max_select); ++i) {
    double a = h_scores[order[(size_t)i - 1]], b = h_scores[order[(size_t)i]];
    double ratio = b > 0 ? a / b : (a > 0 ? INFINITY : 1.0);
    if (ratio > best) {
      best = ratio;
      best_i = i;
    }
  }
  int nsel = std::min(best_i, max_select);
  if (n == 1) nsel = 1;
  for (int i = 0; i < n; ++i) h_order[i] = order[(size_t)i];
  for (int i = 0; i < nsel; ++i) h_selected[i] = order[(size_t)i];
  *h_n_selected = nsel;
  return GIFT_OK;
}

// ---------------------------------------------------------------------------
// Flat gradient buckets
// ---------------------------------------------------------------------------

size_t gift_bucket_table_bytes(int32_t n) {
  if (n < 1) return 0;
  return gift::align256((size_t)(n + 1) * 3 * 8) + 256;
}

gift_status gift_bucket_create(int32_t n, const int64_t* h_numel, int32_t scaling, void* d_table, size_t table_bytes,
                               gift_stream_t stream, gift_bucket_t* out) {
  if (n < 1 || !h_numel || !d_table || !out || (reinterpret_cast<uintptr_t>(d_table) & 255u)) return GIFT_ERR_INVALID_ARG;
  if (scaling != GIFT_SCALE_TENSOR && scaling != GIFT_SCALE_BLOCK512) return GIFT_ERR_INVALID_ARG;
  if (table_bytes < gift_bucket_table_bytes(n)) return GIFT_ERR_WORKSPACE;
  for (int32_t i = 0; i < n; ++i)
    if (h_numel[i] < 4 || h_numel[i] % 4 != 0) return GIFT_ERR_INVALID_ARG;
  gift_bucket* B = new (std::nothrow) gift_bucket;
  if (!B) return GIFT_ERR_INVALID_ARG;
  const size_t n1 = (size_t)n + 1;
  B->n = n;
  B->scaling = scaling;
  B->host.assign(3 * n1, 0);
  int64_t* cs = B->host.data();
  int64_t* eo = cs + n1;
  int64_t* so = eo + n1;
  for (int32_t i = 0; i < n; ++i) {
    cs[i + 1] = cs[i] + gift::cdiv(h_numel[i], 4096);   // 4096-element chunks
    eo[i + 1] = eo[i] + h_numel[i];
    so[i + 1] = so[i] + (scaling == GIFT_SCALE_TENSOR ? 1 : gift::cdiv(h_numel[i], 512));
  }
  B->numel = eo[n];
  B->nscales = so[n];
  char* tb = static_cast<char*>(d_table);
  B->t.chunk_start = reinterpret_cast<const int64_t*>(tb);
  B->t.elem_off = reinterpret_cast<const int64_t*>(tb) + n1;
  B->t.scale_off = reinterpret_cast<const int64_t*>(tb) + 2 * n1;
  B->t.n = n;
  B->t.chunks = cs[n];
  B->t.flags = reinterpret_cast<uint32_t*>(tb + gift::align256(n1 * 3 * 8));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(tb, B->host.data(), n1 * 3 * 8, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = gift::launch_fill_u32(B->t.flags, 0u, 1, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);   // the host copy source must outlive the transfer
  if (e != hipSuccess) {
    delete B;
    return hip_fail(e);
  }
  *out = B;
  return GIFT_OK;
}

gift_status gift_bucket_destroy(gift_bucket_t B) {
  delete B;
  return GIFT_OK;
}

gift_status gift_bucket_sizes(gift_bucket_t B, int64_t* h_numel, int64_t* h_nscales, size_t* h_workspace_bytes) {
  if (!B) return GIFT_ERR_INVALID_ARG;
  if (h_numel) *h_numel = B->numel;
  if (h_nscales) *h_nscales = B->nscales;
  if (h_workspace_bytes) *h_workspace_bytes = gift::align256((size_t)B->nscales * 4);
  return GIFT_OK;
}

gift_status gift_bucket_flags(gift_bucket_t B, gift_stream_t stream, uint32_t* h_flags) {
  if (!B || !h_flags) return GIFT_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GIFT_HIP(hipMemcpyAsync(h_flags, B->t.flags, 4, hipMemcpyDeviceToHost, s));
  GIFT_HIP(hipStreamSynchronize(s));
  return GIFT_OK;
}

gift_status gift_bucket_amax(gift_bucket_t B, const float* d_grad, float* d_amax_out, gift_stream_t stream) {
  if (!B || !d_grad || !d_amax_out || !aligned16(d_grad)) return GIFT_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* slots = reinterpret_cast<uint32_t*>(d_amax_out);   // |x| bit patterns order like the floats
  GIFT_HIP(gift::launch_fill_u32(slots, 0u, (size_t)B->nscales, s));
  GIFT_HIP(gift::launch_bucket_amax(B->t, d_grad, B->scaling == GIFT_SCALE_BLOCK512, slots, device_cus(), s));
  return GIFT_OK;
}

gift_status gift_bucket_encode(gift_bucket_t B, const float* d_grad, int32_t fmt, const float* d_amax_in,
                               float* d_amax_out, uint8_t* d_codes, float* d_scales, void* d_work, size_t work_bytes,
                               gift_stream_t stream) {
  if (!B || !d_grad || !d_codes || !d_scales || !aligned16(d_grad) || !aligned16(d_codes)) return GIFT_ERR_INVALID_ARG;
  if (fmt != GIFT_E4M3 && fmt != GIFT_E5M2) return GIFT_ERR_INVALID_ARG;
  const bool local = !d_amax_in || d_amax_out;
  if (local && (!d_work || (reinterpret_cast<uintptr_t>(d_work) & 255u))) return GIFT_ERR_INVALID_ARG;
  if (local && work_bytes < (size_t)B->nscales * 4) return GIFT_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int blk = B->scaling == GIFT_SCALE_BLOCK512;
  const int cus = device_cus();
  uint32_t* slots = static_cast<uint32_t*>(d_work);
  if (local) {
    GIFT_HIP(gift::launch_fill_u32(slots, 0u, (size_t)B->nscales, s));
    GIFT_HIP(gift::launch_bucket_amax(B->t, d_grad, blk, slots, cus, s));
  }
  GIFT_HIP(gift::launch_bucket_quantize(B->t, d_grad, fmt, blk, slots, d_amax_in, d_amax_out, d_codes, d_scales, cus,
                                        s));
  return GIFT_OK;
}

gift_status gift_bucket_encode_static(gift_bucket_t B, const float* d_grad, int32_t fmt, const float* d_amax_in,
                                      float* d_amax_out, uint8_t* d_codes, float* d_scales, gift_stream_t stream) {
  if (!B || !d_grad || !d_codes || !d_scales || !aligned16(d_grad) || !aligned16(d_codes)) return GIFT_ERR_INVALID_ARG;
  if (fmt != GIFT_E4M3 && fmt != GIFT_E5M2) return GIFT_ERR_INVALID_ARG;
  const bool local = !d_amax_in || d_amax_out;
  if (local && (size_t)B->nscales * 4 > kStaticScratchBytes) return GIFT_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int blk = B->scaling == GIFT_SCALE_BLOCK512;
  const int cus = device_cus();
  uint32_t* slots = nullptr;
  if (local) {
    hipError_t e = hipSuccess;
    slots = static_cast<uint32_t*>(scratch_address(&e));
    if (!slots) return hip_fail(e);
    GIFT_HIP(gift::launch_fill_u32(slots, 0u, (size_t)B->nscales, s));
    GIFT_HIP(gift::launch_bucket_amax(B->t, d_grad, blk, slots, cus, s));
  }
  GIFT_HIP(gift::launch_bucket_quantize(B->t, d_grad, fmt, blk, slots, d_amax_in, d_amax_out, d_codes, d_scales, cus,
                                        s));
  return GIFT_OK;
}

gift_status gift_bucket_decode_reduce(gift_bucket_t B, const uint8_t* d_codes, int64_t code_stride,
                                      const float* d_scales, int64_t scale_stride, int32_t R, int32_t fmt,
                                      float* d_out, gift_stream_t stream) {
  if (!B || !d_codes || !d_scales || !d_out || R < 1 || !aligned16(d_codes) || !aligned16(d_out))
    return GIFT_ERR_INVALID_ARG;
  if (fmt != GIFT_E4M3 && fmt != GIFT_E5M2) return GIFT_ERR_INVALID_ARG;
  if (R > 1 && (code_stride < B->numel || code_stride % 16 != 0 || scale_stride < B->nscales))
    return GIFT_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GIFT_HIP(gift::launch_bucket_dequant_sum(B->t, d_codes, code_stride, d_scales, scale_stride, R, fmt,
                                           B->scaling == GIFT_SCALE_BLOCK512, d_out, device_cus(), s));
  return GIFT_OK;
}

int32_t gift_scale_sync_due(int64_t step, int32_t period) {
  return (period > 0 && step >= 0 && step % period == 0) ? 1 : 0;
}

}  // extern "C"
