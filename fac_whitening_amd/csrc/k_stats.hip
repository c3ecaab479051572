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
template <typename TX>
__global__ void __launch_bounds__(256) k_stats_valu(const TX* __restrict__ x, int64_t T, int64_t ld, int n,
                                                    float* __restrict__ S) {
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
      if (j < n) S[(int64_t)i * n + j] = (float)((double)S[(int64_t)i * n + j] + acc64[p][q]);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 matrix-core statistics: S += X^T X for 256 x 256 output tiles on or
// below the diagonal, one workgroup (4 waves, 2 x 2) per tile.
//  * X is token-major; the MFMA (16x16x32 bf16) wants 8 consecutive tokens
//    per lane, so every thread loads 4 tokens x 8 columns (four 16-byte
//    row segments), transposes them in registers (v_perm) and writes 8-byte
//    column runs into LDS ([column][token], 64 tokens per stage, padded).
//  * Two LDS stages: while a stage is multiplied, the next one's global
//    loads are in flight in registers.
//  * Wave (wm, wn) owns rows 128 wm .. +127 and columns 128 wn .. +127 of
//    the tile: 8 x 8 MFMA tiles, 256 fp32 accumulators per lane.
//  * bf16 x bf16 products are exact in fp32; sums are fp32 (exact for the
//    integer-valued inputs of the exactness test).
//  * Tokens past T read as zero (buffer bounds); columns past n are zeroed
//    after the load and never written back; diagonal tiles write only i >= j.
// ---------------------------------------------------------------------------
typedef __bf16 sbf16x8 __attribute__((ext_vector_type(8)));
typedef float sfloatx4 __attribute__((ext_vector_type(4)));
typedef int sint32x4 __attribute__((ext_vector_type(4)));
typedef int sint32x2 __attribute__((ext_vector_type(2)));

constexpr int kSB = 256;            // output tile
constexpr int kSK = 64;             // tokens per stage
constexpr int kSPad = kSK;          // LDS row pitch (bf16): 128 bytes, one pass over the 32 banks
// The 16-byte token chunks of LDS row c are stored XOR-swizzled by
// f(c) = (c ^ c >> 3) & 7: the fragment reads (8 consecutive rows, one chunk)
// and the transposed writes (rows 8 apart, one chunk) both touch 8 distinct
// chunk positions, i.e. all 32 banks once.
__device__ __forceinline__ int swz(int c) { return (c ^ (c >> 3)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stats_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

constexpr int kStatsSpinLimit = 1 << 22;

// Stages [s_a, s_b) of output tile (bi, bj), added into S.  A tile whose
// stages are split over consecutive workgroups is added in a fixed order:
// the workgroup holding the later stages adds first and raises its flag;
// the one holding the earlier stages (its range ends inside the tile) waits
// for the next workgroup's flag before adding.  Deterministic, no workspace.
template <bool DIAG>
__device__ __forceinline__ void stats_segment(const uint16_t* __restrict__ x, int64_t T, int64_t ld, int n,
                                              float* __restrict__ S, int bi, int bj, int s_a, int s_b, int nst,
                                              uint16_t (*As)[kSB][kSPad], uint16_t (*Bs)[kSB][kSPad],
                                              unsigned* __restrict__ sync, unsigned epoch,
                                              uint32_t* __restrict__ flags) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int row0 = bi * kSB, col0 = bj * kSB;   // i (A side) and j (B side) origins
  // staging: block u (0, 1) of this thread: tokens 4 tg .. 4 tg + 3, columns
  // 8 ig .. 8 ig + 7.  Eight consecutive lanes read 128 contiguous bytes of
  // one token row; a 16-lane LDS write cycle covers 8 column groups x 2 token
  // groups.
  int tg[2], ig[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int b = tid + 256 * u;
    ig[u] = (b & 7) + 8 * ((b >> 7) & 3);
    tg[u] = (b >> 3) & 15;
  }
  struct Regs {
    sint32x4 a[2][4], b[2][4];
  };
  // Stages past T read through an empty buffer resource (zeros, no traffic).
  auto gload = [&](int64_t t0, Regs& R) {
    const int64_t rows = T - t0 < kSK ? T - t0 : kSK;
    const auto rs = stats_rsrc(x + (rows > 0 ? t0 * ld : 0), rows > 0 ? rows * ld * 2 : 0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tg[u] + r;
        R.a[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((t * ld + row0 + 8 * ig[u]) * 2), 0, 0);
        if constexpr (!DIAG)
          R.b[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((t * ld + col0 + 8 * ig[u]) * 2), 0, 0);
      }
  };
  // Columns past n are zeroed here, where the loaded registers are used (a
  // select right after the load would wait for it).
  auto lstore = [&](uint16_t (*L)[kSPad], const sint32x4 (*v)[4], int cbase) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool ok = cbase + 8 * ig[u] < n;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // column 8 ig + 2w: low halves; column 8 ig + 2w + 1: high halves
        const uint32_t a0 = ok ? (uint32_t)v[u][0][w] : 0u, a1 = ok ? (uint32_t)v[u][1][w] : 0u;
        const uint32_t a2 = ok ? (uint32_t)v[u][2][w] : 0u, a3 = ok ? (uint32_t)v[u][3][w] : 0u;
        const uint32_t l0 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
        const uint32_t l1 = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
        const uint32_t h0 = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
        const uint32_t h1 = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
        const int c0 = 8 * ig[u] + 2 * w, c1 = c0 + 1;
        const int ch = tg[u] >> 1, half = (tg[u] & 1) * 4;
        *reinterpret_cast<sint32x2*>(&L[c0][8 * (ch ^ swz(c0)) + half]) = (sint32x2){(int)l0, (int)l1};
        *reinterpret_cast<sint32x2*>(&L[c1][8 * (ch ^ swz(c1)) + half]) = (sint32x2){(int)h0, (int)h1};
      }
    }
  };
  sfloatx4 acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = (sfloatx4){0.f, 0.f, 0.f, 0.f};
  const int lr = lane & 15, lq = lane >> 4;
  // One 32-token half of a stage: the 8 B fragments are loaded first, the A
  // fragments stream two row tiles ahead of their MFMAs.
  auto half_mfma = [&](uint16_t (*LA)[kSPad], uint16_t (*LB)[kSPad], int kk) {
    sbf16x8 fb[8];
    const int ch = kk / 8 + lq;   // this lane's 8-token chunk
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int c = 128 * wn + 16 * nt + lr;
      fb[nt] = __builtin_bit_cast(sbf16x8, *reinterpret_cast<const sint32x4*>(&LB[c][8 * (ch ^ swz(c))]));
    }
    auto fa_of = [&](int mt) {
      const int c = 128 * wm + 16 * mt + lr;
      return __builtin_bit_cast(sbf16x8, *reinterpret_cast<const sint32x4*>(&LA[c][8 * (ch ^ swz(c))]));
    };
    sbf16x8 f0 = fa_of(0), f1 = fa_of(1);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const sbf16x8 f2 = fa_of(mt + 2 < 8 ? mt + 2 : 7);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, fb[nt], acc[mt][nt], 0, 0, 0);
      f0 = f1;
      f1 = f2;
    }
  };
  // Stage pipeline: LDS holds stages st (being multiplied) and st + 1; the
  // registers hold the global loads of stage st + 2.  The transposed stores
  // of stage st + 1 are issued after the first half's MFMAs, so they run
  // while the matrix pipe works; the next global loads follow them.  The
  // loop body has no branch: a store of a stage past the end lands in a
  // buffer nobody reads.
  Regs R0;
  __syncthreads();   // the previous segment's waves are done with the LDS stages
  gload((int64_t)s_a * kSK, R0);
  lstore(As[0], R0.a, row0);
  if constexpr (!DIAG) lstore(Bs[0], R0.b, col0);
  gload((int64_t)(s_a + 1) * kSK, R0);
  auto iter = [&](int st, int buf) {
    __syncthreads();   // stage st is in LDS; nobody reads buf ^ 1 any more
    uint16_t (*LA)[kSPad] = As[buf];
    uint16_t (*LB)[kSPad] = DIAG ? As[buf] : Bs[buf];
    half_mfma(LA, LB, 0);
    lstore(As[buf ^ 1], R0.a, row0);
    if constexpr (!DIAG) lstore(Bs[buf ^ 1], R0.b, col0);
    __builtin_amdgcn_sched_barrier(0);   // the prefetch registers are free before they are reloaded
    gload((int64_t)(st + 2) * kSK, R0);
    half_mfma(LA, LB, 32);
  };
  for (int st = s_a; st < s_b; ++st) iter(st, (st - s_a) & 1);
  const int g = blockIdx.x, tid2 = threadIdx.x;
  if (s_b < nst) {
    // the next workgroup holds the later stages of this tile: it adds first
    if (tid2 == 0) {
      int spins = 0;
      // relaxed polls (an acquire per poll would invalidate the caches each
      // time); one acquire fence once the flag is seen
      while (__hip_atomic_load(sync + g + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
        if (++spins > kStatsSpinLimit) {
          atomicOr(flags, (uint32_t)GIFT_FLAG_SPIN_TIMEOUT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  // S += acc: element (i, j) = (4 (lane / 16) + e, lane % 16) of MFMA tile (mt, nt)
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = row0 + 128 * wm + 16 * mt + 4 * (lane >> 4) + e;
        const int j = col0 + 128 * wn + 16 * nt + lr;
        if (i < n && j < n && (!DIAG || i >= j)) {
          float* p = S + (int64_t)i * n + j;
          *p += acc[mt][nt][e];
        }
      }
  if (s_a > 0) {
    // the previous workgroup (earlier stages of this tile) adds after us
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid2 == 0) __hip_atomic_store(sync + g, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Persistent: workgroup g takes an equal, contiguous range of the
// (tile, stage) units (tiles in lower-triangle order, stages in token
// order), so every compute unit gets the same amount of work.  All
// workgroups are resident (one per compute unit: the LDS stages fill it).
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_stats_mfma(const uint16_t* __restrict__ x, int64_t T, int64_t ld, int n, float* __restrict__ S, int ntiles,
             unsigned* __restrict__ sync, unsigned epoch, uint32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kSB][kSPad];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kSB][kSPad];
  const int nst = (int)cdiv(T, kSK);
  const int64_t U = (int64_t)ntiles * nst, G = gridDim.x, g = blockIdx.x;
  const int64_t base = U / G, rem = U % G;
  const int64_t u0 = g * base + (g < rem ? g : rem), u1 = u0 + base + (g < rem ? 1 : 0);
  for (int64_t u = u0; u < u1;) {
    const int tile = (int)(u / nst), s_a = (int)(u % nst);
    const int s_b = (int)((u1 - u) < (int64_t)(nst - s_a) ? s_a + (u1 - u) : nst);
    int bi, bj;
    tri_tile(tile, bi, bj);
    if (bi == bj)
      stats_segment<true>(x, T, ld, n, S, bi, bj, s_a, s_b, nst, As, Bs, sync, epoch, flags);
    else
      stats_segment<false>(x, T, ld, n, S, bi, bj, s_a, s_b, nst, As, Bs, sync, epoch, flags);
    u += s_b - s_a;
  }
}

hipError_t launch_stats(const void* x, int dtype, int64_t T, int64_t ld, int n, float* S, unsigned* sync,
                        unsigned epoch, uint32_t* flags, int cus, hipStream_t s) {
  if (T == 0 || n == 0) return hipSuccess;
  int nb = (int)cdiv(n, 64);
  unsigned tiles = (unsigned)(nb * (nb + 1) / 2);
  if (dtype == GIFT_BF16 && n % 8 == 0 && ld % 8 == 0 && (int64_t)kSK * ld * 2 < ((int64_t)1 << 31) && cus > 0) {
    const int nb2 = (int)cdiv(n, kSB);
    const int ntiles = nb2 * (nb2 + 1) / 2;
    const int64_t units = (int64_t)ntiles * cdiv(T, kSK);
    // at most two workgroups per tile: a tile's hand-off chain stays one link
    // long (each link costs a cache write-back and a cold read of the tile)
    int grid = cus < kStatsMaxGroups ? cus : kStatsMaxGroups;
    if (2 * ntiles < grid) grid = 2 * ntiles;
    if (units < grid) grid = (int)units;
    hipLaunchKernelGGL(k_stats_mfma, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint16_t*>(x), T,
                       ld, n, S, ntiles, sync, epoch, flags);
  } else if (dtype == GIFT_BF16)
    hipLaunchKernelGGL(k_stats_valu<__hip_bfloat16>, dim3(tiles), dim3(256), 0, s,
                       static_cast<const __hip_bfloat16*>(x), T, ld, n, S);
  else
    hipLaunchKernelGGL(k_stats_valu<float>, dim3(tiles), dim3(256), 0, s, static_cast<const float*>(x), T, ld,
                       n, S);
  return hipGetLastError();
}

// A = first ? S/count : beta A + (1 - beta) S/count  (fp64 arithmetic, fp32
// storage), for the lower-triangle tile (bi, bj) and its mirror; S <- 0.
__global__ void __launch_bounds__(256) k_commit(float* __restrict__ S, float* __restrict__ A, int n,
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
      S[o] = 0.f;   // the upper half of diagonal tiles is accumulated but unused
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

hipError_t launch_commit(float* S, float* A, int n, double inv_count, float beta, int first, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int nb = (int)cdiv(n, 64);
  unsigned tiles = (unsigned)(nb * (nb + 1) / 2);
  hipLaunchKernelGGL(k_commit, dim3(tiles), dim3(256), 0, s, S, A, n, inv_count, (double)beta, first);
  return hipGetLastError();
}

}  // namespace gift
