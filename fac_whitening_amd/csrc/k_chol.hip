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
// invert it) in one wave, solve the panel below it, update the trailing
// lower triangle.  Inverse: X = L^-1 by a right-looking block solve of
// L X = I (X_ii from the diagonal step), one launch of independent 64 x 64
// products per step.
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

// Factor the diagonal block kb in one wave and write its inverse into X:
// lane i keeps row i of the block in registers (left-looking: at step j it
// forms L[i][j] from its own row and row j of L, read from LDS where every
// lane stores its new element), then column i of L^-1 by forward
// substitution against the rows of L in LDS.  Both loops are unrolled, so
// every register index is a constant.  Rows past n are the identity.
__device__ __forceinline__ double rsq_nr64(double x) {
  double y = __builtin_amdgcn_rsq(x);   // estimate, then two Newton steps
  y = y * (1.5 - 0.5 * x * y * y);
  return y * (1.5 - 0.5 * x * y * y);
}

__global__ void __launch_bounds__(64) k_potrf_diag(double* __restrict__ W, double* __restrict__ X, int n, int kb,
                                                   uint32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) double Ls[NB][NB + 2];
  __shared__ double Dinv[NB];
  const int i = threadIdx.x;
  const int r0 = kb * NB;
  const bool live_row = r0 + i < n;
  double row[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const bool ok = live_row && r0 + q < n;
    row[q] = ok ? W[(int64_t)(r0 + i) * n + r0 + q] : (i == q ? 1.0 : 0.0);
  }
  bool bad = false;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < j; ++q) acc[q & 3] += row[q] * Ls[j][q];
    const double r = row[j] - ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    const double dj = __shfl(r, j, 64);   // the pivot, from lane j
    double rs = rsq_nr64(dj);
    if (!(dj > 0.0)) {
      bad = true;
      rs = __longlong_as_double(0x7FF8000000000000LL);
    }
    row[j] = i > j ? r * rs : (i == j ? dj * rs : 0.0);
    Ls[i][j] = row[j];
    if (i == 0) Dinv[j] = rs;
  }
  double x[NB];   // column i of L^-1
#pragma unroll
  for (int rr = 0; rr < NB; ++rr) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < rr; ++q) acc[q & 3] += Ls[rr][q] * x[q];
    const double v = (rr == i ? 1.0 : 0.0) - ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    x[rr] = rr >= i ? v * Dinv[rr] : 0.0;
  }
  if (live_row) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (r0 + q < n) W[(int64_t)(r0 + i) * n + r0 + q] = q <= i ? row[q] : 0.0;
  }
  if (r0 + i < n) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (r0 + q < n) X[(int64_t)(r0 + q) * n + r0 + i] = x[q];   // column i of the block's inverse
  }
  if (i == 0 && bad) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
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

// Inverse X = L^-1 by a right-looking block solve of L X = I.  X's blocks
// below the diagonal start at zero and accumulate
// -sum_{k < i} L_ik X_kj; at step kb block row kb is finished,
// X_kb,j <- X_kb,kb (X_kb,j) for j < kb (X_kb,kb = L_kb,kb^-1 from the
// diagonal step), and every later block row takes its share,
// X_i,j -= L_i,kb X_kb,j for i > kb, j <= kb (one 64 x 64 product per
// workgroup, all of a step in one launch).

// k_inv_row: X_kb,j <- X_kb,kb X_kb,j, workgroup j < kb.
__global__ void __launch_bounds__(256) k_inv_row(double* __restrict__ X, int n, int kb) {
  __shared__ double P[NB][NB + 1];   // X_kb,kb
  __shared__ double Q[NB][NB + 1];   // X_kb,j transposed (so tile_abt forms P X_kb,j)
  const int bj = blockIdx.x;
  load_block(X, n, kb, kb, P);
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    const int ii = kb * NB + r, jj = bj * NB + c;
    Q[c][r] = (ii < n && jj < n) ? X[(int64_t)ii * n + jj] : 0.0;
  }
  __syncthreads();
  double acc[4][4] = {};
  tile_abt(P, Q, acc);
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = kb * NB + ty * 4 + u;
    if (r >= n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = bj * NB + tx * 4 + v;
      if (c < n) X[(int64_t)r * n + c] = acc[u][v];
    }
  }
}

// k_inv_update: X_i,j -= L_i,kb X_kb,j for i > kb, j <= kb; workgroup t is
// (i, j) = (kb + 1 + t / (kb + 1), t % (kb + 1)).
__global__ void __launch_bounds__(256) k_inv_update(const double* __restrict__ W, double* __restrict__ X, int n,
                                                    int kb) {
  __shared__ double P[NB][NB + 1];   // L_i,kb
  __shared__ double Q[NB][NB + 1];   // X_kb,j transposed
  const int t = blockIdx.x;
  const int bi = kb + 1 + t / (kb + 1), bj = t % (kb + 1);
  load_block(W, n, bi, kb, P);
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    const int ii = kb * NB + r, jj = bj * NB + c;
    Q[c][r] = (ii < n && jj < n) ? X[(int64_t)ii * n + jj] : 0.0;
  }
  __syncthreads();
  double acc[4][4] = {};
  tile_abt(P, Q, acc);
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = bi * NB + ty * 4 + u;
    if (r >= n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = bj * NB + tx * 4 + v;
      if (c < n) X[(int64_t)r * n + c] -= acc[u][v];
    }
  }
}

__global__ void k_zero64(double* __restrict__ p, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) p[e] = 0.0;
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
  hipLaunchKernelGGL(k_zero64, dim3((unsigned)cdiv((int64_t)n * n, 256)), dim3(256), 0, s, Xk, (int64_t)n * n);
  for (int kb = 0; kb < nb; ++kb) {
    hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(64), 0, s, Wk, Xk, n, kb, flags);
    const int rest = nb - kb - 1;
    if (rest > 0) {
      hipLaunchKernelGGL(k_trsm_panel, dim3((unsigned)rest), dim3(256), 0, s, Wk, Xk, n, kb);
      hipLaunchKernelGGL(k_syrk_update, dim3((unsigned)(rest * (rest + 1) / 2)), dim3(256), 0, s, Wk, n, kb);
    }
  }
  for (int kb = 0; kb < nb; ++kb) {
    if (kb > 0) hipLaunchKernelGGL(k_inv_row, dim3((unsigned)kb), dim3(256), 0, s, Xk, n, kb);
    const int rest = nb - kb - 1;
    if (rest > 0)
      hipLaunchKernelGGL(k_inv_update, dim3((unsigned)(rest * (kb + 1))), dim3(256), 0, s, Wk, Xk, n, kb);
  }
  hipLaunchKernelGGL(k_chol_out, dim3((unsigned)nb, (unsigned)nb), dim3(256), 0, s, Wk, Xk, n, lower_out, tinv, t);
  return hipGetLastError();
}

// Triangular products on the fp64 matrix cores (v_mfma_f64_16x16x4f64; the
// fp32 operands are exact in fp64), 64 x 64 output tiles:
//   side 0: out[m][d] = x[m][d] * M[d][d], M upper: column tile j uses k < j0 + 64.
//   side 1: out[m][d] = M[m][m] * x[m][d], M lower: row tile i uses k < i0 + 64.
// Four waves, each a 32 x 32 quarter of the tile (2 x 2 MFMA tiles).  Stages
// of 32 k: the next stage's fp32 values are loaded into registers while the
// current one (fp64 in LDS) is multiplied.  MFMA operands: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; slot e of lane l holds
// D[4 e + l / 16][l % 16].
typedef double double4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_trmm(const float* __restrict__ x, int64_t ldx, int m, int d,
                                              const float* __restrict__ M, int side, float* __restrict__ out,
                                              int64_t ldo) {
  // row strides chosen so that the 64 lanes of an operand read (16 rows or
  // columns x 4 k) touch every bank twice, the minimum for 8-byte reads
  __shared__ double As[64][36];   // [row][k]
  __shared__ double Bs[32][80];   // [k][col]
  const int i0 = blockIdx.y * NB, j0 = blockIdx.x * NB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lm = lane & 15, lk = lane >> 4;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;   // this wave's quarter
  const int K = side == 0 ? d : m;
  const int kend = side == 0 ? min(K, j0 + NB) : min(K, i0 + NB);
  double4v acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (double4v){0.0, 0.0, 0.0, 0.0};
  // stage loads: A element (row r, k kk) and B element (k kk, col c), 8 each per thread
  float av[8], bv[8];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      const int kk = e % 32, r = e / 32;   // A: 64 rows x 32 k
      const int kg = k0 + kk;
      float v = 0.f;
      if (side == 0) {
        if (i0 + r < m && kg < d) v = x[(int64_t)(i0 + r) * ldx + kg];
      } else {
        if (i0 + r < m && kg < m) v = M[(int64_t)(i0 + r) * m + kg];
      }
      av[u] = v;
      const int kb = e / NB, c = e % NB;   // B: 32 k x 64 cols
      const int kgb = k0 + kb;
      float w = 0.f;
      if (side == 0) {
        if (kgb < d && j0 + c < d) w = M[(int64_t)kgb * d + j0 + c];
      } else {
        if (kgb < m && j0 + c < d) w = x[(int64_t)kgb * ldx + j0 + c];
      }
      bv[u] = w;
    }
  };
  load(0);
  for (int k0 = 0; k0 < kend; k0 += 32) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      As[e / 32][e % 32] = (double)av[u];
      Bs[e / NB][e % NB] = (double)bv[u];
    }
    __syncthreads();
    if (k0 + 32 < kend) load(k0 + 32);   // in flight while this stage is multiplied
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int kk = 4 * ks + lk;
      double a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = As[wr + 16 * t + lm][kk];
        b[t] = Bs[kk][wc + 16 * t + lm];
      }
#pragma unroll
      for (int ta = 0; ta < 2; ++ta)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[ta][tb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ta], b[tb], acc[ta][tb], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int ta = 0; ta < 2; ++ta)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = i0 + wr + 16 * ta + 4 * e + lk, c = j0 + wc + 16 * tb + lm;
        if (r < m && c < d) out[(int64_t)r * ldo + c] = (float)acc[ta][tb][e];
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
