// Factor refresh: rank-k basis of A by randomized subspace iteration, and the
// diagonal variant.
//
// GIFT 阅读笔记, §简化二 Eq. (17): A ~ U_r Lam_r U_r^T with r = 32, refreshed
// every K = 50 steps (Algorithm 1 preamble).  The pages do not say how the
// eigenpairs are obtained; here (randomized subspace iteration, Halko,
// Martinsson & Tropp 2011, specialised to symmetric A):
//   Y = A Omega;  q times { Q = orth(Y); Y = A Q };  Q = orth(Y);
//   B = Q^T (A Q) = V Theta V^T;  U = Q V[:, :k].
// orth is CholeskyQR2 (Fukaya et al. 2014) with fp64 Gram and Cholesky; the
// l x l eigenproblem is solved by cyclic two-sided Jacobi (Golub & Van Loan,
// §8.5) in fp64 inside one workgroup, with parallel (round-robin) ordering.
// A is read as fp32; every other quantity is fp64 until the basis U and the
// coefficient vectors are written as fp32.
#include "gift_internal.hpp"

namespace gift {

hipError_t launch_project_f64(const float* x, int64_t ldx, int m, int d, const double* Q, int lp,
                              double* part, hipStream_t s);

// Small-buffer layout (fp64 elements).
constexpr int kSmTrace = 0;            // [0] tr(A)
constexpr int kSmM = 64;               // [LP*LP] l x l matrix (R^-1 or V_k)
constexpr int kSmTheta = kSmM + 64 * 64;  // [LP] Ritz values (sorted)

__global__ void __launch_bounds__(1024) k_trace(const float* __restrict__ A, int d, double* __restrict__ out) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 1024) s += (double)A[(int64_t)i * d + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0];
}

// Omega (fp32 [d][l]) -> fp64 [d][lp], zero padded.
__global__ void k_omega64(const float* __restrict__ om, int d, int l, int lp, double* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)d * lp) return;
  int r = (int)(i / lp), c = (int)(i % lp);
  out[i] = c < l ? (double)om[(int64_t)r * l + c] : 0.0;
}

// part[ch][a][b] = sum_{i in rows of chunk ch} X[i][a] Y[i][b]  (fp64, LP <= 64)
template <int LP>
__global__ void __launch_bounds__(256) k_gram_parts(const double* __restrict__ X, const double* __restrict__ Y,
                                                    int d, double* __restrict__ part) {
  __shared__ double Xs[32][LP];
  __shared__ double Ys[32][LP];
  constexpr int PER = (LP * LP + 255) / 256;
  double acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0;
  const int r0 = blockIdx.x * 256;
  for (int s0 = r0; s0 < min(d, r0 + 256); s0 += 32) {
    for (int e = threadIdx.x; e < 32 * LP; e += 256) {
      int rr = e / LP, c = e % LP;
      bool ok = s0 + rr < d && s0 + rr < r0 + 256;
      Xs[rr][c] = ok ? X[(int64_t)(s0 + rr) * LP + c] : 0.0;
      Ys[rr][c] = ok ? Y[(int64_t)(s0 + rr) * LP + c] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      int o = threadIdx.x + e * 256;
      if (o < LP * LP) {
        int a = o / LP, b = o % LP;
        double s = acc[e];
        for (int rr = 0; rr < 32; ++rr) s += Xs[rr][a] * Ys[rr][b];
        acc[e] = s;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    int o = threadIdx.x + e * 256;
    if (o < LP * LP) part[(int64_t)blockIdx.x * LP * LP + o] = acc[e];
  }
}

// One workgroup: G = sum of Gram partials (l x l), G = L L^T, writes
// M = L^-T (upper triangular, zero outside l x l) into small[kSmM].
template <int LP>
__global__ void __launch_bounds__(256) k_chol_inv_small(const double* __restrict__ part, int nch, int l,
                                                        double* __restrict__ small, uint32_t* __restrict__ flags) {
  __shared__ double Gm[LP][LP + 1];
  __shared__ double Li[LP][LP + 1];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  for (int o = tid; o < LP * LP; o += 256) {
    double s = 0.0;
    for (int ch = 0; ch < nch; ++ch) s += part[(int64_t)ch * LP * LP + o];
    Gm[o / LP][o % LP] = s;
    Li[o / LP][o % LP] = 0.0;
  }
  __syncthreads();
  // right-looking Cholesky on the leading l x l block (lower triangle of Gm)
  for (int j = 0; j < l; ++j) {
    if (tid == 0) {
      double p = Gm[j][j];
      if (!(p > 0.0)) {
        bad = 1;
        p = __longlong_as_double(0x7FF8000000000000LL);
      }
      Gm[j][j] = sqrt(p);
    }
    __syncthreads();
    for (int i = j + 1 + tid; i < l; i += 256) Gm[i][j] /= Gm[j][j];
    __syncthreads();
    for (int o = tid; o < l * l; o += 256) {
      int i = o / l, c = o % l;
      if (i > j && c > j && c <= i) Gm[i][c] -= Gm[i][j] * Gm[c][j];
    }
    __syncthreads();
  }
  // L^-1 column by column (forward substitution), one thread per column
  if (tid < l) {
    int c = tid;
    for (int i = c; i < l; ++i) {
      double s = (i == c) ? 1.0 : 0.0;
      for (int q = c; q < i; ++q) s -= Gm[i][q] * Li[q][c];
      Li[i][c] = s / Gm[i][i];
    }
  }
  __syncthreads();
  // M = (L^-1)^T: M[a][b] = Li[b][a]
  for (int o = tid; o < LP * LP; o += 256) {
    int a = o / LP, b = o % LP;
    small[kSmM + o] = (a < l && b < l) ? Li[b][a] : 0.0;
  }
  if (tid == 0 && bad) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
}

// out[i][:NC] = X[i][:LP] * M[:LP][:NC] with M in small[kSmM] ([LP][LPM]).
template <int LP, int NC, typename TO>
__global__ void __launch_bounds__(256) k_right_small(const double* __restrict__ X, int d,
                                                     const double* __restrict__ small, int ldm,
                                                     TO* __restrict__ out) {
  __shared__ double Ms[LP][NC];
  for (int o = threadIdx.x; o < LP * NC; o += 256) Ms[o / NC][o % NC] = small[kSmM + (o / NC) * ldm + (o % NC)];
  __syncthreads();
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d) return;
  double xr[LP];
#pragma unroll
  for (int a = 0; a < LP; ++a) xr[a] = X[(int64_t)i * LP + a];
  for (int b = 0; b < NC; ++b) {
    double s = 0.0;
#pragma unroll
    for (int a = 0; a < LP; ++a) s += xr[a] * Ms[a][b];
    out[(int64_t)i * NC + b] = (TO)s;
  }
}

// One workgroup: B = sum of partials (Q^T A Q), symmetrised; cyclic Jacobi;
// Ritz values sorted descending (ties: lower index first); V_k (the first k
// sorted eigenvectors) into small[kSmM] as [LP][32]; coefficients into coef.
template <int LP>
__global__ void __launch_bounds__(256) k_jacobi_coef(const double* __restrict__ part, int nch, int l, int k,
                                                     int d, float damping_rel, double* __restrict__ small,
                                                     float* __restrict__ coef, uint32_t* __restrict__ flags) {
  __shared__ double B[LP][LP + 1];
  __shared__ double V[LP][LP + 1];
  __shared__ double cs[LP / 2][2];
  __shared__ int order[LP];
  __shared__ double offn, alln;
  const int tid = threadIdx.x;
  for (int o = tid; o < LP * LP; o += 256) {
    double s = 0.0;
    for (int ch = 0; ch < nch; ++ch) s += part[(int64_t)ch * LP * LP + o];
    B[o / LP][o % LP] = s;
  }
  __syncthreads();
  for (int o = tid; o < LP * LP; o += 256) V[o / LP][o % LP] = (o / LP == o % LP) ? 1.0 : 0.0;
  // symmetrise in place (pairs a < b handled by one thread each)
  for (int o = tid; o < LP * LP; o += 256) {
    int a = o / LP, b = o % LP;
    if (a < b) {
      double v = (a < l && b < l) ? 0.5 * (B[a][b] + B[b][a]) : 0.0;
      B[a][b] = v;
      B[b][a] = v;
    } else if (a == b && a >= l) {
      B[a][a] = 0.0;
    }
  }
  __syncthreads();
  const int n = (l + 1) & ~1;   // players in the round-robin (a dummy if l is odd)
  const int npair = n / 2;
  for (int sweep = 0; sweep < 30; ++sweep) {
    for (int round = 0; round < n - 1; ++round) {
      if (tid < npair) {
        int i = tid;
        int p = (i == 0) ? 0 : ((i - 1 + round) % (n - 1)) + 1;
        int q = ((n - 2 - i + round) % (n - 1)) + 1;
        if (p > q) { int t = p; p = q; q = t; }
        double c = 1.0, s = 0.0;
        if (q < l && B[p][q] != 0.0) {
          double tau = (B[q][q] - B[p][p]) / (2.0 * B[p][q]);
          double t = tau >= 0.0 ? 1.0 / (tau + sqrt(1.0 + tau * tau)) : -1.0 / (-tau + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        cs[i][0] = c;
        cs[i][1] = s;
      }
      __syncthreads();
      // rows: B <- J^T B
      for (int o = tid; o < npair * l; o += 256) {
        int i = o / l, jcol = o % l;
        int p = (i == 0) ? 0 : ((i - 1 + round) % (n - 1)) + 1;
        int q = ((n - 2 - i + round) % (n - 1)) + 1;
        if (p > q) { int t = p; p = q; q = t; }
        if (q >= l) continue;
        double c = cs[i][0], s = cs[i][1];
        double bp = B[p][jcol], bq = B[q][jcol];
        B[p][jcol] = c * bp - s * bq;
        B[q][jcol] = s * bp + c * bq;
      }
      __syncthreads();
      // columns: B <- B J, V <- V J
      for (int o = tid; o < npair * l; o += 256) {
        int i = o / l, r = o % l;
        int p = (i == 0) ? 0 : ((i - 1 + round) % (n - 1)) + 1;
        int q = ((n - 2 - i + round) % (n - 1)) + 1;
        if (p > q) { int t = p; p = q; q = t; }
        if (q >= l) continue;
        double c = cs[i][0], s = cs[i][1];
        double bp = B[r][p], bq = B[r][q];
        B[r][p] = c * bp - s * bq;
        B[r][q] = s * bp + c * bq;
        double vp = V[r][p], vq = V[r][q];
        V[r][p] = c * vp - s * vq;
        V[r][q] = s * vp + c * vq;
      }
      __syncthreads();
    }
    if (tid == 0) {
      double off = 0.0, all = 0.0;
      for (int a = 0; a < l; ++a)
        for (int b = 0; b < l; ++b) {
          double v = B[a][b] * B[a][b];
          all += v;
          if (a != b) off += v;
        }
      offn = off;
      alln = all;
    }
    __syncthreads();
    const bool done = offn <= 1e-30 * alln;
    __syncthreads();
    if (done) break;
  }
  // sort Ritz values descending (stable) -- one thread, l <= 64
  if (tid == 0) {
    for (int a = 0; a < l; ++a) order[a] = a;
    for (int a = 1; a < l; ++a) {
      int v = order[a];
      int b = a - 1;
      while (b >= 0 && (B[order[b]][order[b]] < B[v][v])) {
        order[b + 1] = order[b];
        --b;
      }
      order[b + 1] = v;
    }
  }
  __syncthreads();
  // V_k into small[kSmM] as [LP][32]
  for (int o = tid; o < LP * 32; o += 256) {
    int a = o / 32, t = o % 32;
    small[kSmM + o] = (a < l && t < k) ? V[a][order[t]] : 0.0;
  }
  if (tid < LP) small[kSmTheta + tid] = tid < l ? B[order[tid]][order[tid]] : 0.0;
  __syncthreads();
  if (tid == 0) {
    double tr = small[kSmTrace];
    double lam = (double)damping_rel * tr / (double)d;
    double sum = 0.0;
    for (int t = 0; t < k; ++t) sum += B[order[t]][order[t]];
    double rho;
    if (k < d) {
      rho = (tr - sum) / (double)(d - k);
      rho = (rho > 0.0 ? rho : 0.0) + lam;
    } else {
      rho = lam > 0.0 ? lam : 1.0;
    }
    double rm = 1.0 / sqrt(rho), rp = sqrt(rho);
    bool bad = !(rho > 0.0) || !isfinite(rm);
    for (int t = 0; t < 32; ++t) {
      double ce = 0.0, cd = 0.0;
      if (t < k) {
        double th = B[order[t]][order[t]];
        double lt = (th > 0.0 ? th : 0.0) + lam;
        if (!(lt > 0.0)) bad = true;
        ce = 1.0 / sqrt(lt) - rm;
        cd = sqrt(lt) - rp;
      }
      coef[t] = (float)ce;
      coef[32 + t] = (float)cd;
    }
    coef[64] = (float)rm;
    coef[65] = (float)rp;
    coef[66] = (float)lam;
    coef[67] = (float)rho;
    if (bad) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
  }
}

template <int LP>
static hipError_t refresh_lowrank_lp(const float* A, int d, int k, int l, int q, float damping_rel,
                                     const float* omega, float* U, float* coef, const WorkLayout& w,
                                     char* work, uint32_t* flags, hipStream_t s) {
  double* Y = reinterpret_cast<double*>(work + w.Y);
  double* Q = reinterpret_cast<double*>(work + w.Q);
  double* Z = reinterpret_cast<double*>(work + w.Z);
  double* small = reinterpret_cast<double*>(work + w.small);
  double* gpart = reinterpret_cast<double*>(work + w.gpart);
  const int nchG = (int)cdiv(d, 256);
  const unsigned eb = (unsigned)cdiv((int64_t)d * LP, 256);
  hipLaunchKernelGGL(k_trace, dim3(1), dim3(1024), 0, s, A, d, small + kSmTrace);
  hipLaunchKernelGGL(k_omega64, dim3(eb), dim3(256), 0, s, omega, d, l, LP, Q);
  auto product = [&](const double* X, double* out) {   // out = A X
    (void)launch_project_f64(A, d, d, d, X, LP, out, s);   // errors surface at the final hipGetLastError
  };
  auto orth = [&](const double* X, double* out) {       // CholeskyQR2
    const double* src = X;
    for (int pass = 0; pass < 2; ++pass) {
      hipLaunchKernelGGL((k_gram_parts<LP>), dim3(nchG), dim3(256), 0, s, src, src, d, gpart);
      hipLaunchKernelGGL((k_chol_inv_small<LP>), dim3(1), dim3(256), 0, s, gpart, nchG, l, small, flags);
      hipLaunchKernelGGL((k_right_small<LP, LP, double>), dim3((unsigned)cdiv(d, 256)), dim3(256), 0, s, src, d,
                         small, LP, out);
      src = out;
    }
  };
  product(Q, Y);                      // Y = A Omega
  for (int it = 0; it < q; ++it) {
    orth(Y, Q);                       // Q = orth(Y)
    product(Q, Y);                    // Y = A Q
  }
  orth(Y, Q);                         // Q = orth(Y)
  product(Q, Z);                      // Z = A Q
  hipLaunchKernelGGL((k_gram_parts<LP>), dim3(nchG), dim3(256), 0, s, Q, Z, d, gpart);
  hipLaunchKernelGGL((k_jacobi_coef<LP>), dim3(1), dim3(256), 0, s, gpart, nchG, l, k, d, damping_rel, small,
                     coef, flags);
  hipLaunchKernelGGL((k_right_small<LP, 32, float>), dim3((unsigned)cdiv(d, 256)), dim3(256), 0, s, Q, d, small,
                     32, U);
  return hipGetLastError();
}

hipError_t launch_refresh_lowrank(const float* A, int d, int k, int l, int q, float damping_rel,
                                  const float* omega, float* U, float* coef, const WorkLayout& w,
                                  char* work, uint32_t* flags, hipStream_t s) {
  if (l <= 48) return refresh_lowrank_lp<48>(A, d, k, l, q, damping_rel, omega, U, coef, w, work, flags, s);
  return refresh_lowrank_lp<64>(A, d, k, l, q, damping_rel, omega, U, coef, w, work, flags, s);
}

// Diagonal variant: coef[j] = (A_jj + lam)^-1/2, coef[d + j] = (A_jj + lam)^1/2.
__global__ void __launch_bounds__(1024) k_diag_factor(const float* __restrict__ A, int d, float damping_rel,
                                                      float* __restrict__ coef, uint32_t* __restrict__ flags) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 1024) s += (double)A[(int64_t)i * d + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const double lam = (double)damping_rel * red[0] / (double)d;
  bool bad = false;
  for (int i = threadIdx.x; i < d; i += 1024) {
    double v = (double)A[(int64_t)i * d + i] + lam;
    if (!(v > 0.0)) bad = true;
    coef[i] = (float)(1.0 / sqrt(v));
    coef[d + i] = (float)sqrt(v);
  }
  if (bad) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
}

hipError_t launch_refresh_diag(const float* A, int d, float damping_rel, float* coef, uint32_t* flags,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_diag_factor, dim3(1), dim3(1024), 0, s, A, d, damping_rel, coef, flags);
  return hipGetLastError();
}

}  // namespace gift
