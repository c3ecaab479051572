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

hipError_t launch_stats(const void* x, int dtype, int64_t T, int64_t ld, int n, float* S, hipStream_t s) {
  if (T == 0 || n == 0) return hipSuccess;
  int nb = (int)cdiv(n, 64);
  unsigned tiles = (unsigned)(nb * (nb + 1) / 2);
  if (dtype == GIFT_BF16)
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
