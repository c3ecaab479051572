// Full variants: blocked Cholesky of A + lam I (and G + lam_G I), the
// triangular inverse, and the triangular products that apply them.
//
// GIFT 阅读笔记, §核心想法 Eq. (7): A = L_A L_A^T, G = L_G L_G^T; Eq. (11):
// W~ = L_G^-1 W L_A^-T; Eq. (14): W^ = L_G U L_A^T; §简化一 Eq. (16): the
// input-side-only form W~ = W L_A^-T.  The factor is computed in fp64 (the
// damped A of a power-law spectrum has a condition number near 1e5..1e6) and
// stored as fp32 triangles; the products accumulate in fp64.
//
// Cholesky: right-looking, 64 x 64 blocks: factor the diagonal block (and
// invert it) in one workgroup, solve the panel below it, update the trailing
// lower triangle.  Inverse: X = L^-1 block row by block row,
// X_ij = -X_ii sum_{k=j}^{i-1} L_ik X_kj (i > j), X_ii from the diagonal step.
#include "gift_internal.hpp"

namespace gift {

constexpr int NB = 64;

// Load block (bi, bj) of a [n][n] fp64 matrix into LDS; outside [0, n) the
// block is zero, except ones on the diagonal of a diagonal block (so padded
// diagonal blocks stay invertible).
__device__ __forceinline__ void load_block(const double* __restrict__ M, int n, int bi, int bj,
                                           double (*dst)[NB + 1]) {
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    int r = e / NB, c = e % NB;
    int i = bi * NB + r, j = bj * NB + c;
    double v;
    if (i < n && j < n) v = M[(int64_t)i * n + j];
    else v = (bi == bj && r == c) ? 1.0 : 0.0;
    dst[r][c] = v;
  }
}

__device__ __forceinline__ void store_block(double* __restrict__ M, int n, int bi, int bj,
                                            const double (*src)[NB + 1]) {
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    int r = e / NB, c = e % NB;
    int i = bi * NB + r, j = bj * NB + c;
    if (i < n && j < n) M[(int64_t)i * n + j] = src[r][c];
  }
}

// lam = damping_rel * tr(A) / n -> lam_out; W = A + lam I (fp64, lower used).
__global__ void __launch_bounds__(1024) k_chol_lambda(const float* __restrict__ A, int n, float damping_rel,
                                                      double* __restrict__ lam_out) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += (double)A[(int64_t)i * n + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) lam_out[0] = (double)damping_rel * red[0] / (double)n;
}

__global__ void k_chol_init(const float* __restrict__ A, int n, const double* __restrict__ lam,
                            double* __restrict__ W) {
  int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)n * n) return;
  int i = (int)(e / n), j = (int)(e % n);
  double v = (double)A[e];
  if (i == j) v += lam[0];
  W[e] = v;
}

// Factor the diagonal block kb in place and write its inverse into X.
__global__ void __launch_bounds__(256) k_potrf_diag(double* __restrict__ W, double* __restrict__ X, int n, int kb,
                                                    uint32_t* __restrict__ flags) {
  __shared__ double L[NB][NB + 1];
  __shared__ double Li[NB][NB + 1];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  load_block(W, n, kb, kb, L);
  __syncthreads();
  for (int j = 0; j < NB; ++j) {
    if (threadIdx.x == 0) {
      double p = L[j][j];
      if (!(p > 0.0)) {
        bad = 1;
        p = __longlong_as_double(0x7FF8000000000000LL);
      }
      L[j][j] = sqrt(p);
    }
    __syncthreads();
    for (int i = j + 1 + threadIdx.x; i < NB; i += 256) L[i][j] /= L[j][j];
    __syncthreads();
    for (int e = threadIdx.x; e < NB * NB; e += 256) {
      int i = e / NB, c = e % NB;
      if (c > j && c <= i) L[i][c] -= L[i][j] * L[c][j];
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    int r = e / NB, c = e % NB;
    if (c > r) L[r][c] = 0.0;
    Li[r][c] = 0.0;
  }
  __syncthreads();
  if (threadIdx.x < NB) {
    const int c = threadIdx.x;
    for (int i = c; i < NB; ++i) {
      double s = (i == c) ? 1.0 : 0.0;
      for (int q = c; q < i; ++q) s -= L[i][q] * Li[q][c];
      Li[i][c] = s / L[i][i];
    }
  }
  __syncthreads();
  store_block(W, n, kb, kb, L);
  store_block(X, n, kb, kb, Li);
  if (threadIdx.x == 0 && bad) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
}

// 64 x 64 fp64 tile product helper: acc (4 x 4 per thread) += P * Q^T where
// P, Q are [NB][NB + 1] in LDS (rows of P times rows of Q).
__device__ __forceinline__ void tile_abt(const double (*P)[NB + 1], const double (*Q)[NB + 1], double acc[4][4]) {
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  for (int q = 0; q < NB; ++q) {
    double a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = P[ty * 4 + u][q];
      b[u] = Q[tx * 4 + u][q];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
  }
}

// Panel: L_ik = A_ik L_kk^-T for i > kb  (out[r][c] = sum_q A[r][q] Li[c][q]).
__global__ void __launch_bounds__(256) k_trsm_panel(double* __restrict__ W, const double* __restrict__ X, int n,
                                                    int kb) {
  __shared__ double Ab[NB][NB + 1];
  __shared__ double Li[NB][NB + 1];
  const int bi = kb + 1 + blockIdx.x;
  load_block(W, n, bi, kb, Ab);
  load_block(X, n, kb, kb, Li);
  __syncthreads();
  double acc[4][4] = {};
  tile_abt(Ab, Li, acc);
  __syncthreads();
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) Ab[ty * 4 + u][tx * 4 + v] = acc[u][v];
  __syncthreads();
  store_block(W, n, bi, kb, Ab);
}

// Trailing update of the lower triangle: A_ij -= L_ik L_jk^T, kb < j <= i.
__global__ void __launch_bounds__(256) k_syrk_update(double* __restrict__ W, int n, int kb) {
  __shared__ double Pi[NB][NB + 1];
  __shared__ double Pj[NB][NB + 1];
  int idx = blockIdx.x;
  int i = (int)((sqrt(8.0 * idx + 1.0) - 1.0) * 0.5);
  while ((i + 1) * (i + 2) / 2 <= idx) ++i;
  while (i * (i + 1) / 2 > idx) --i;
  int j = idx - i * (i + 1) / 2;
  const int bi = kb + 1 + i, bj = kb + 1 + j;
  load_block(W, n, bi, kb, Pi);
  load_block(W, n, bj, kb, Pj);
  __syncthreads();
  double acc[4][4] = {};
  tile_abt(Pi, Pj, acc);
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int r = bi * NB + ty * 4 + u;
    if (r >= n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int c = bj * NB + tx * 4 + v;
      if (c < n) W[(int64_t)r * n + c] -= acc[u][v];
    }
  }
}

// Inverse, block row bi: X_ij = -X_ii sum_{k=j}^{bi-1} L_ik X_kj for j < bi.
__global__ void __launch_bounds__(256) k_trinv_row(const double* __restrict__ W, double* __restrict__ X, int n,
                                                   int bi) {
  __shared__ double P[NB][NB + 1];
  __shared__ double Q[NB][NB + 1];
  const int bj = blockIdx.x;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  double acc[4][4] = {};
  for (int kb = bj; kb < bi; ++kb) {
    __syncthreads();
    load_block(W, n, bi, kb, P);                  // L_ik
    // Q = X_kj^T so that tile_abt computes L_ik X_kj
    for (int e = threadIdx.x; e < NB * NB; e += 256) {
      int r = e / NB, c = e % NB;
      int ii = kb * NB + r, jj = bj * NB + c;
      double v = (ii < n && jj < n) ? X[(int64_t)ii * n + jj] : ((kb == bj && r == c) ? 1.0 : 0.0);
      Q[c][r] = v;
    }
    __syncthreads();
    tile_abt(P, Q, acc);
  }
  __syncthreads();
  // T (in P) then X_ij = -X_ii T
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) P[ty * 4 + u][tx * 4 + v] = acc[u][v];
  for (int e = threadIdx.x; e < NB * NB; e += 256) {   // Q = X_ii
    int r = e / NB, c = e % NB;
    int ii = bi * NB + r, jj = bi * NB + c;
    Q[r][c] = (ii < n && jj < n) ? X[(int64_t)ii * n + jj] : (r == c ? 1.0 : 0.0);
  }
  __syncthreads();
  double out[4][4] = {};
  for (int q = 0; q < NB; ++q) {
    double a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = Q[ty * 4 + u][q];
      b[u] = P[q][tx * 4 + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) out[u][v] -= a[u] * b[v];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int r = bi * NB + ty * 4 + u;
    if (r >= n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int c = bj * NB + tx * 4 + v;
      if (c < n) X[(int64_t)r * n + c] = out[u][v];
    }
  }
}

// fp32 outputs.  lower_out = 0: tinv = X^T (= L^-T, upper), t = L^T (upper).
// lower_out = 1: tinv = X (= L^-1, lower), t = L (lower).  Other triangle 0.
__global__ void __launch_bounds__(256) k_chol_out(const double* __restrict__ W, const double* __restrict__ X, int n,
                                                  int lower_out, float* __restrict__ tinv, float* __restrict__ t) {
  __shared__ float Ts[2][NB][NB + 1];
  const int bi = blockIdx.y, bj = blockIdx.x;
  // source block: (bi, bj) for lower_out, (bj, bi) transposed otherwise
  const int si = lower_out ? bi : bj, sj = lower_out ? bj : bi;
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    int r = e / NB, c = e % NB;
    int i = si * NB + r, j = sj * NB + c;
    float a = 0.f, b = 0.f;
    if (i < n && j < n && j <= i) {
      a = (float)X[(int64_t)i * n + j];
      b = (float)W[(int64_t)i * n + j];
    }
    Ts[0][r][c] = a;
    Ts[1][r][c] = b;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    int r = e / NB, c = e % NB;
    int i = bi * NB + r, j = bj * NB + c;
    if (i >= n || j >= n) continue;
    float a = lower_out ? Ts[0][r][c] : Ts[0][c][r];
    float b = lower_out ? Ts[1][r][c] : Ts[1][c][r];
    tinv[(int64_t)i * n + j] = a;
    t[(int64_t)i * n + j] = b;
  }
}

hipError_t launch_refresh_chol(const float* A, int n, float damping_rel, float* tinv, float* t, int lower_out,
                               double* Wk, double* Xk, uint32_t* flags, hipStream_t s) {
  const int nb = (int)cdiv(n, NB);
  double* lam = Xk + (int64_t)n * n;   // the workspace region holds n*n + 32 doubles
  hipLaunchKernelGGL(k_chol_lambda, dim3(1), dim3(1024), 0, s, A, n, damping_rel, lam);
  hipLaunchKernelGGL(k_chol_init, dim3((unsigned)cdiv((int64_t)n * n, 256)), dim3(256), 0, s, A, n, lam, Wk);
  for (int kb = 0; kb < nb; ++kb) {
    hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(256), 0, s, Wk, Xk, n, kb, flags);
    const int rest = nb - kb - 1;
    if (rest > 0) {
      hipLaunchKernelGGL(k_trsm_panel, dim3((unsigned)rest), dim3(256), 0, s, Wk, Xk, n, kb);
      hipLaunchKernelGGL(k_syrk_update, dim3((unsigned)(rest * (rest + 1) / 2)), dim3(256), 0, s, Wk, n, kb);
    }
  }
  for (int bi = 1; bi < nb; ++bi)
    hipLaunchKernelGGL(k_trinv_row, dim3((unsigned)bi), dim3(256), 0, s, Wk, Xk, n, bi);
  hipLaunchKernelGGL(k_chol_out, dim3((unsigned)nb, (unsigned)nb), dim3(256), 0, s, Wk, Xk, n, lower_out, tinv, t);
  return hipGetLastError();
}

// Triangular products with fp64 accumulation, 64 x 64 output tiles:
//   side 0: out[m][d] = x[m][d] * M[d][d], M upper: column tile j uses k <= j.
//   side 1: out[m][d] = M[m][m] * x[m][d], M lower: row tile i uses k <= i.
__global__ void __launch_bounds__(256) k_trmm(const float* __restrict__ x, int64_t ldx, int m, int d,
                                              const float* __restrict__ M, int side, float* __restrict__ out,
                                              int64_t ldo) {
  __shared__ float As[32][NB + 4];   // [k][row]
  __shared__ float Bs[32][NB + 4];   // [k][col]
  const int i0 = blockIdx.y * NB, j0 = blockIdx.x * NB;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  const int K = side == 0 ? d : m;
  const int kend = side == 0 ? min(K, j0 + NB) : min(K, i0 + NB);
  double acc[4][4] = {};
  for (int k0 = 0; k0 < kend; k0 += 32) {
    for (int e = threadIdx.x; e < 32 * NB; e += 256) {
      int kk = e % 32, r = e / 32;      // A element (row r, k kk)
      int kg = k0 + kk;
      float av = 0.f;
      if (side == 0) {
        if (i0 + r < m && kg < d) av = x[(int64_t)(i0 + r) * ldx + kg];
      } else {
        if (i0 + r < m && kg < m) av = M[(int64_t)(i0 + r) * m + kg];
      }
      As[kk][r] = av;
    }
    for (int e = threadIdx.x; e < 32 * NB; e += 256) {
      int kk = e / NB, c = e % NB;      // B element (k kk, col c)
      int kg = k0 + kk;
      float bv = 0.f;
      if (side == 0) {
        if (kg < d && j0 + c < d) bv = M[(int64_t)kg * d + j0 + c];
      } else {
        if (kg < m && j0 + c < d) bv = x[(int64_t)kg * ldx + j0 + c];
      }
      Bs[kk][c] = bv;
    }
    __syncthreads();
    for (int kk = 0; kk < 32; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = (double)As[kk][ty * 4 + u];
        b[u] = (double)Bs[kk][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int r = i0 + ty * 4 + u;
    if (r >= m) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int c = j0 + tx * 4 + v;
      if (c < d) out[(int64_t)r * ldo + c] = (float)acc[u][v];
    }
  }
}

hipError_t launch_trmm(const float* x, int64_t ldx, int m, int d, const float* M, int side, float* out, int64_t ldo,
                       hipStream_t s) {
  if (m == 0 || d == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(d, NB), (unsigned)cdiv(m, NB));
  hipLaunchKernelGGL(k_trmm, grid, dim3(256), 0, s, x, ldx, m, d, M, side, out, ldo);
  return hipGetLastError();
}

}  // namespace gift
