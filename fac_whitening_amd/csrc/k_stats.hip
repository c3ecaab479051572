// Input / output statistics: S += x^T x over T tokens, and the EMA commit.
//
// GIFT 阅读笔记, §前置知识 Eq. (4): A = E[a a^T] (d_in x d_in), G = E[delta
// delta^T] (d_out x d_out).  Activations are token-major ([T][n]); the
// product is symmetric, so only tiles on or below the diagonal are computed
// and the commit mirrors them.
#include <hip/hip_bf16.h>

#include "gift_internal.hpp"

namespace gift {

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__hip_bfloat16 v) { return __bfloat162float(v); }

// Decode the linear index of a lower-triangle tile (bi >= bj).
__device__ __forceinline__ void tri_tile(int idx, int& bi, int& bj) {
  int i = (int)((sqrtf(8.0f * (float)idx + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= idx) ++i;
  while (i * (i + 1) / 2 > idx) --i;
  bi = i;
  bj = idx - i * (i + 1) / 2;
}

// VALU tiling: 64 x 64 output tile per workgroup, 32 tokens per LDS stage,
// 4 x 4 outputs per thread; fp32 sums over 256-token chunks folded into fp64
// (keeps the relative error of A near the fp32 storage rounding).
// overwrite: the first call of a window stores the sums instead of adding
// them to S (which then needs no clearing between windows).
template <typename TX>
__global__ void __launch_bounds__(256) k_stats_valu(const TX* __restrict__ x, int64_t T, int64_t ld, int n,
                                                    float* __restrict__ S, int overwrite) {
  __shared__ float Ai[32][64 + 4];
  __shared__ float Aj[32][64 + 4];
  int bi, bj;
  tri_tile(blockIdx.x, bi, bj);
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  double acc64[4][4] = {};
  for (int64_t t0 = 0; t0 < T; t0 += 32) {
    for (int e = tid; e < 32 * 64; e += 256) {
      int tt = e / 64, c = e % 64;
      int64_t t = t0 + tt;
      int ci = bi * 64 + c, cj = bj * 64 + c;
      Ai[tt][c] = (t < T && ci < n) ? to_f32(x[t * ld + ci]) : 0.f;
      Aj[tt][c] = (t < T && cj < n) ? to_f32(x[t * ld + cj]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int tt = 0; tt < 32; ++tt) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = Ai[tt][ty * 4 + q];
        b[q] = Aj[tt][tx * 4 + q];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] += a[p] * b[q];
    }
    __syncthreads();
    if (((t0 / 32) & 7) == 7 || t0 + 32 >= T) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc64[p][q] += (double)acc[p][q];
          acc[p][q] = 0.f;
        }
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    int i = bi * 64 + ty * 4 + p;
    if (i >= n) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int j = bj * 64 + tx * 4 + q;
      if (j < n)
        S[(int64_t)i * n + j] = overwrite ? (float)acc64[p][q] : (float)((double)S[(int64_t)i * n + j] + acc64[p][q]);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 matrix-core statistics: S += X^T X for 256 x 256 output tiles on or
// below the diagonal, one workgroup (4 waves, 2 x 2) per tile.
//  * X is token-major and stays so in LDS: each side of a stage is 32 token
//    rows x 256 columns (512 bytes a row), filled by direct global-to-LDS
//    loads (16 bytes a lane; no registers), five stages deep: four stages
//    of loads are in flight while one is multiplied.  The LDS pipe, not the
//    matrix pipe, bounds this loop: the transposing 8-byte reads run at
//    about 48 bytes a clock per compute unit (16-byte reads about 130).
//  * The 32x32x16 bf16 MFMA wants 8 consecutive tokens of one column per
//    lane.  The transposing LDS read (ds_read_b64_tr_b16) gives them: in a
//    16-lane group, lane j points at 4 columns of token k0 + j / 4, and
//    lane i receives column C + i at tokens k0 .. k0 + 3.  Two such reads
//    make one operand.
//  * Row t of a stage holds global 16-byte chunk g at slot g ^ 4 (t % 4):
//    the loads write whole rows (the swizzle is in the global addresses)
//    and the transposing reads of 32 lanes touch all 64 banks once.
//  * Wave (wm, wn) owns rows 128 wm .. +127 and columns 128 wn .. +127 of
//    the tile: 4 x 4 MFMA tiles of 32 x 32, 256 fp32 accumulators per
//    lane.  With one wave per SIMD the 32 x 32 shape keeps the matrix pipe
//    fuller than 16 x 16 (measured: about 0.84 against 0.55 of the bf16
//    peak for back-to-back independent products).
//  * bf16 x bf16 products are exact in fp32; sums are fp32 (exact for the
//    integer-valued inputs of the exactness test).
//  * Tokens past T and columns past n read as zero (buffer bounds); columns
//    past n are never written back; diagonal tiles write only i >= j.
// ---------------------------------------------------------------------------
typedef __bf16 sbf16x8 __attribute__((ext_vector_type(8)));
typedef float sfloatx16 __attribute__((ext_vector_type(16)));
typedef short sshort4 __attribute__((ext_vector_type(4)));

constexpr int kSB = 256;            // output tile
constexpr int kSK = 32;             // tokens per stage
constexpr int kSStages = 5;         // LDS stages (four in flight; 160 KiB)
constexpr int kSRow = kSB * 2;      // bytes per token row of a side tile
constexpr int kSSide = kSK * kSRow; // bytes per side and stage (16 KiB)
constexpr int kOffOOB = (int)0x80000000u;   // an offset past any buffer: the load returns zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stats_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

constexpr int kStatsSpinLimit = 1 << 22;

typedef __attribute__((address_space(3))) void lds_void;
typedef int sint32x4 __attribute__((ext_vector_type(4)));

// 16-byte global-to-LDS load of every lane: lane l's 16 bytes from rsrc at
// voff land at LDS byte lds + 16 l (lds wave-uniform, through M0).  Issued
// as inline assembly so that the compiler does not track these LDS writes
// (it would wait for every load in flight before each LDS read); the kernel
// orders them itself with s_waitcnt vmcnt and barriers.
__device__ __forceinline__ void lds_load16(sint32x4 rsrc, uint32_t lds, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// Stages [s_a, s_b) of output tile (bi, bj), added into S.  A tile whose
// stages are split over consecutive workgroups is added in a fixed order:
// the workgroup holding the later stages adds first and raises its flag;
// the one holding the earlier stages (its range ends inside the tile) waits
// for the next workgroup's flag before adding.  Deterministic, no workspace.
template <bool DIAG, bool OW>
__device__ __forceinline__ void stats_segment(const uint16_t* __restrict__ x, int64_t T, int64_t ld, int n,
                                              float* __restrict__ S, int bi, int bj, int s_a, int s_b, int nst,
                                              char* As, char* Bs, unsigned* __restrict__ sync, unsigned epoch,
                                              uint32_t* __restrict__ flags) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int row0 = bi * kSB, col0 = bj * kSB;   // i (A side) and j (B side) origins
  // loads: instruction q of wave w fills slots 64 (4 w + q) .. + 63 of a
  // side tile: token row t = 2 (4 w + q) + lane / 32, slot lane % 32, which
  // holds global chunk (lane % 32) ^ 4 (t % 4) of that row
  int voff_a[4], voff_b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 2 * (4 * wave + q) + (lane >> 5);
    const int gch = (lane & 31) ^ (4 * (t & 3));
    const int ca = row0 + 8 * gch, cb = col0 + 8 * gch;
    voff_a[q] = ca < n ? (int)((t * ld + ca) * 2) : kOffOOB;
    voff_b[q] = cb < n ? (int)((t * ld + cb) * 2) : kOffOOB;
  }
  // Stage st into LDS buffer buf (stages past T read zeros, no traffic).
  const uint32_t lds_a = (uint32_t)(uintptr_t)(lds_void*)As, lds_b = (uint32_t)(uintptr_t)(lds_void*)Bs;
  // buffer descriptor of stage st: base, stride 0, bytes, raw-buffer flags
  auto stage_rsrc = [&](int st) {
    const int64_t t0 = (int64_t)st * kSK;
    const int64_t rows = T - t0 < kSK ? T - t0 : kSK;
    const uint64_t base = (uint64_t)(uintptr_t)(x + (rows > 0 ? t0 * ld : 0));
    const sint32x4 rs = {__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                         __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32) & 0xFFFF),
                         __builtin_amdgcn_readfirstlane((int)(uint32_t)(rows > 0 ? rows * ld * 2 : 0)),
                         0x00020000};
    return rs;
  };
  // load k of this thread's share of a stage: A side k < 4, B side k - 4
  auto issue_one = [&](const sint32x4& rs, int buf, int k) {
    const int q = k & 3;
    const uint32_t slot = (uint32_t)(buf * kSSide + 64 * (4 * wave + q) * 16);
    if (k < 4) lds_load16(rs, __builtin_amdgcn_readfirstlane(lds_a + slot), voff_a[q]);
    else lds_load16(rs, __builtin_amdgcn_readfirstlane(lds_b + slot), voff_b[q]);
  };
  auto issue = [&](int st, int buf) {
    const sint32x4 rs = stage_rsrc(st);
#pragma unroll
    for (int k = 0; k < (DIAG ? 4 : 8); ++k) issue_one(rs, buf, k);
  };
  constexpr int kLoads = DIAG ? 4 : 8;   // loads per thread per stage
  sfloatx16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  // Operand reads.  Lane l (group g = l / 16, i = l % 16) points at token
  // 16 ks + 8 (g / 2) + 4 r + i / 4 and column 128 w + 32 mt + 16 (g % 2) +
  // 4 (i % 4) of a side tile; with the swizzle its byte address is
  //   8192 ks + 2048 r + [4096 (g / 2) + 512 (i / 4) + 16 (2 (g % 2) +
  //   (i % 4) / 2 + 16 w) + 8 (i % 2)] + 64 (mt ^ (i / 4)):
  // per lane, four offsets per side (one per mt), the rest immediate.
  const int g = lane >> 4, li = lane & 15;
  int offa[4], offb[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int common = 4096 * (g >> 1) + 512 * (li >> 2) + 16 * (2 * (g & 1) + ((li & 3) >> 1)) + 8 * (li & 1) +
                       64 * (mt ^ (li >> 2));
    offa[mt] = common + 256 * wm;
    offb[mt] = common + 256 * wn;
  }
  auto frag = [&](const char* base, int off, int ks) {
    const sshort4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) sshort4*)(base + off + 8192 * ks));
    const sshort4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) sshort4*)(base + off + 8192 * ks + 2048));
    const sshort4 v[2] = {lo, hi};
    return __builtin_bit_cast(sbf16x8, v);
  };
  struct Frags {
    sbf16x8 a[4], b[4];
  };
  auto load_frags = [&](Frags& F, int buf, int ks) {
    const char* LA = As + buf * kSSide;
    const char* LB = (DIAG ? As : Bs) + buf * kSSide;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      F.b[t] = frag(LB, offb[t], ks);
      F.a[t] = frag(LA, offa[t], ks);
    }
  };
  // products of row tiles mt0 .. mt1 - 1 with F; after every fourth one the
  // next load of the stage being prefetched (loads k .. kmax - 1)
  auto products = [&](const Frags& F, int mt0, int mt1, const sint32x4& lrs, int lbuf, int& k) {
#pragma unroll
    for (int mt = mt0; mt < mt1; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[mt], F.b[nt], acc[mt][nt], 0, 0, 0);
        if (nt == 1 && k < kLoads) {
          issue_one(lrs, lbuf, k);
          ++k;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // Pipeline (five LDS stages, four in flight): an iteration multiplies
  // stage st; the operands of its second 16-token step are read while the
  // first step multiplies; half way through the second step the wave waits
  // for stage st + 1 and syncs, and reads that stage's first operands under
  // the last eight products.  The loads of stage st + 4 (into the buffer of
  // stage st - 1, free since the previous sync) go out one after every
  // fourth product.
  __syncthreads();   // the previous segment's waves are done with the LDS stages
#pragma unroll
  for (int p = 0; p < kSStages - 1; ++p) issue(s_a + p, p);
  // counts of this wave's loads that may stay in flight
  constexpr int kAheadStart = (kSStages - 2) * kLoads;                 // stage s_a complete
  constexpr int kAheadMid = 2 * kLoads + (kLoads > 4 ? 6 : kLoads);     // stage st + 1 complete
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kAheadStart & 0xF) | ((kAheadStart >> 4) << 14));
  __syncthreads();
  Frags F0, F1;
  load_frags(F0, 0, 0);
  int buf = 0;
  for (int st = s_a; st < s_b; ++st) {
    const sint32x4 lrs = stage_rsrc(st + kSStages - 1);
    const int lbuf = buf == 0 ? kSStages - 1 : buf - 1;
    int k = 0;
    load_frags(F1, buf, 1);
    __builtin_amdgcn_sched_barrier(0);
    products(F0, 0, 4, lrs, lbuf, k);
    products(F1, 0, 2, lrs, lbuf, k);
    const int nbuf = buf + 1 == kSStages ? 0 : buf + 1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of buffer buf are done
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kAheadMid & 0xF) | ((kAheadMid >> 4) << 14));
    __syncthreads();
    load_frags(F0, nbuf, 0);
    __builtin_amdgcn_sched_barrier(0);
    products(F1, 2, 4, lrs, lbuf, k);
    buf = nbuf;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // drain the loads past the range before the LDS is reused
  const int gw = blockIdx.x, tid2 = threadIdx.x;
  // A tile shared with another workgroup is read and written with
  // device-coherent (agent-scope relaxed atomic) accesses, and the hand-off
  // is ordered by waiting for those accesses to complete before the flag is
  // raised, and by reading only after the flag is seen: no cache-wide
  // release / acquire (on this multi-die device those write back and
  // invalidate a whole L2 and stall every other workgroup on it).
  const bool shared = s_a > 0 || s_b < nst;
  // a hand-over that never came (a wait that ran out) poisons this part of
  // the tile with NaN, so the committed A, and the factor, show it
  bool late = false;
  if (s_b < nst) {
    // the next workgroup holds the later stages of this tile: it adds first.
    // Lane 0 of every wave polls, so each wave knows the outcome itself.
    int out = 0;
    if ((tid2 & 63) == 0) {
      int spins = 0;
      while (__hip_atomic_load(sync + gw + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
        if (++spins > kStatsSpinLimit) {
          atomicOr(flags, (uint32_t)GIFT_FLAG_SPIN_TIMEOUT);
          out = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    late = __builtin_amdgcn_readfirstlane(out) != 0;
    __syncthreads();
  }
  // S += acc (S = acc for the first writer of a tile when the call opens a
  // window: the workgroup holding the tile's last stages, which adds first):
  // register v of MFMA tile (mt, nt) is element
  // (8 (v / 4) + 4 (lane / 32) + v % 4, lane % 32) of the 32 x 32 tile
  const int lr = lane & 31, lh = lane >> 5;
  const bool store_only = OW && s_b == nst;
  // (the old value is loaded in either case and dropped when the sums are
  // stored: the same code as for adding, whose registers this loop fits)
  if (shared) {
    // device-coherent loads and stores (sc0 sc1), 64 loads in flight per
    // row block; elements outside the output go to an offset past the end
    const uint32_t nbytes = (uint32_t)((int64_t)n * n * 4);
    const auto rs = stats_rsrc(S, nbytes);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      int off[4][16];
      float v[4][16];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = row0 + 128 * wm + 32 * mt + 8 * (e / 4) + 4 * lh + e % 4;
          const int j = col0 + 128 * wn + 32 * nt + lr;
          const bool ok = i < n && j < n && (!DIAG || i >= j);
          off[nt][e] = ok ? (int)(uint32_t)(((int64_t)i * n + j) * 4) : (int)nbytes;
          v[nt][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off[nt][e], 0, 17));
        }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(
              __float_as_uint(late ? __builtin_nanf("") : (store_only ? acc[mt][nt][e] : v[nt][e] + acc[mt][nt][e])),
              rs, off[nt][e], 0, 17);
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = row0 + 128 * wm + 32 * mt + 8 * (e / 4) + 4 * lh + e % 4;
          const int j = col0 + 128 * wn + 32 * nt + lr;
          if (i < n && j < n && (!DIAG || i >= j)) {
            const float old = S[(int64_t)i * n + j];
            S[(int64_t)i * n + j] = store_only ? acc[mt][nt][e] : old + acc[mt][nt][e];
          }
        }
  }
  if (s_a > 0) {
    // the previous workgroup (earlier stages of this tile) adds after us:
    // every store of this workgroup has completed before the flag is set
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid2 == 0) __hip_atomic_store(sync + gw, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Persistent: workgroup g first takes whole tiles in rounds (tile g, g + G,
// ... while a full round of G tiles remains), so the workgroups of a round
// walk the token stages in step and share each stage's columns through the
// L2; the tiles left over (fewer than G) are cut into equal, contiguous
// ranges of (tile, stage) units, one per workgroup (in lower-triangle tile
// order, stages in token order).  All workgroups are resident (one per
// compute unit: the LDS stages fill it).
// OW: the call opens a window (the first writer of each tile stores its
// sums instead of adding them); a separate kernel, so that the adding form
// keeps its own register allocation.
template <bool OW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_stats_mfma(const uint16_t* __restrict__ x, int64_t T, int64_t ld, int n, float* __restrict__ S, int ntiles,
             unsigned* __restrict__ sync, unsigned epoch, uint32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) char As[kSStages * kSSide];
  __shared__ __attribute__((aligned(16))) char Bs[kSStages * kSSide];
  const int nst = (int)cdiv(T, kSK);
  const int G = gridDim.x, gid = blockIdx.x;
  const int rounds = ntiles / G;
  for (int rd = 0; rd < rounds; ++rd) {
    int bi, bj;
    tri_tile(rd * G + gid, bi, bj);
    if (bi == bj)
      stats_segment<true, OW>(x, T, ld, n, S, bi, bj, 0, nst, nst, As, Bs, sync, epoch, flags);
    else
      stats_segment<false, OW>(x, T, ld, n, S, bi, bj, 0, nst, nst, As, Bs, sync, epoch, flags);
  }
  const int first = rounds * G;
  const int64_t U = (int64_t)(ntiles - first) * nst;
  const int64_t base = U / G, rem = U % G;
  const int64_t u0 = gid * base + (gid < rem ? gid : rem), u1 = u0 + base + (gid < rem ? 1 : 0);
  for (int64_t u = u0; u < u1;) {
    const int tile = first + (int)(u / nst), s_a = (int)(u % nst);
    const int s_b = (int)((u1 - u) < (int64_t)(nst - s_a) ? s_a + (u1 - u) : nst);
    int bi, bj;
    tri_tile(tile, bi, bj);
    if (bi == bj)
      stats_segment<true, OW>(x, T, ld, n, S, bi, bj, s_a, s_b, nst, As, Bs, sync, epoch, flags);
    else
      stats_segment<false, OW>(x, T, ld, n, S, bi, bj, s_a, s_b, nst, As, Bs, sync, epoch, flags);
    u += s_b - s_a;
  }
}

int stats_resident_groups() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cache[dev]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_stats_mfma<false>), 256, 0) !=
        hipSuccess)
      return 0;
    cache[dev] = cus * per_cu;
  }
  return cache[dev];
}

hipError_t launch_stats(const void* x, int dtype, int64_t T, int64_t ld, int n, float* S, unsigned* sync,
                        unsigned epoch, uint32_t* flags, int cus, bool overwrite, hipStream_t s) {
  if (T == 0 || n == 0) return hipSuccess;
  int nb = (int)cdiv(n, 64);
  unsigned tiles = (unsigned)(nb * (nb + 1) / 2);
  if (dtype == GIFT_BF16 && n % 8 == 0 && ld % 8 == 0 && (int64_t)kSK * ld * 2 < ((int64_t)1 << 31) && cus > 0) {
    const int nb2 = (int)cdiv(n, kSB);
    const int ntiles = nb2 * (nb2 + 1) / 2;
    const int64_t units = (int64_t)ntiles * cdiv(T, kSK);
    // workgroups that share a tile wait on one another: the grid is at most
    // what the device holds at once (the kernel's occupancy times the
    // compute units, or the gift_set_max_resident cap)
    int grid = cus < kStatsMaxGroups ? cus : kStatsMaxGroups;
    const int res = stats_resident_groups(), cap = max_resident_cap();
    if (res > 0 && res < grid) grid = res;
    if (cap > 0 && cap < grid) grid = cap;
    if (units < grid) grid = (int)units;
    const hipError_t e = order_persistent(s);
    if (e != hipSuccess) return e;
    if (overwrite)
      hipLaunchKernelGGL(k_stats_mfma<true>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                         T, ld, n, S, ntiles, sync, epoch, flags);
    else
      hipLaunchKernelGGL(k_stats_mfma<false>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                         T, ld, n, S, ntiles, sync, epoch, flags);
  } else if (dtype == GIFT_BF16)
    hipLaunchKernelGGL(k_stats_valu<__hip_bfloat16>, dim3(tiles), dim3(256), 0, s,
                       static_cast<const __hip_bfloat16*>(x), T, ld, n, S, overwrite ? 1 : 0);
  else
    hipLaunchKernelGGL(k_stats_valu<float>, dim3(tiles), dim3(256), 0, s, static_cast<const float*>(x), T, ld,
                       n, S, overwrite ? 1 : 0);
  return hipGetLastError();
}

// A = first ? S/count : beta A + (1 - beta) S/count  (fp64 arithmetic, fp32
// storage), for the lower-triangle tile (bi, bj) and its mirror.  S is left
// as it is: the next window's first call overwrites it.
__global__ void __launch_bounds__(256) k_commit(const float* __restrict__ S, float* __restrict__ A, int n,
                                                double inv_count, double beta, int first) {
  __shared__ float tile[64][65];
  int bi, bj;
  tri_tile(blockIdx.x, bi, bj);
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * 64; e += 256) {
    int r = e / 64, c = e % 64;
    int i = bi * 64 + r, j = bj * 64 + c;
    float v = 0.f;
    if (i < n && j < n) {
      int64_t o = (int64_t)i * n + j;
      if (bi != bj || j <= i) {
        double a = (double)S[o] * inv_count;
        if (!first) a = beta * (double)A[o] + (1.0 - beta) * a;
        v = (float)a;
        A[o] = v;
      }
    }
    tile[r][c] = v;
  }
  __syncthreads();
  // mirror: A[j][i] = A[i][j] for the tile (coalesced through LDS)
  for (int e = tid; e < 64 * 64; e += 256) {
    int r = e / 64, c = e % 64;       // r indexes j, c indexes i
    int j = bj * 64 + r, i = bi * 64 + c;
    if (i < n && j < n && (bi != bj || j < i)) A[(int64_t)j * n + i] = tile[c][r];
  }
}

hipError_t launch_commit(const float* S, float* A, int n, double inv_count, float beta, int first, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int nb = (int)cdiv(n, 64);
  unsigned tiles = (unsigned)(nb * (nb + 1) / 2);
  hipLaunchKernelGGL(k_commit, dim3(tiles), dim3(256), 0, s, S, A, n, inv_count, (double)beta, first);
  return hipGetLastError();
}

}  // namespace gift
