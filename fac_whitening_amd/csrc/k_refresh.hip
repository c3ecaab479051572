// Factor refresh: rank-k basis of A by randomized subspace iteration, and the
// diagonal variant.
//
// GIFT 阅读笔记, §简化二 Eq. (17): A ~ U_r Lam_r U_r^T with r = 32, refreshed
// every K = 50 steps (Algorithm 1 preamble).  The pages do not say how the
// eigenpairs are obtained; here (randomized subspace iteration, Halko,
// Martinsson & Tropp 2011, specialised to symmetric A):
//   Y = A Omega;  q times { Q = orth(Y); Y = A Q };  Q = orth(Y);
//   B = Q^T (A Q) = V Theta V^T;  U = Q V[:, :k].
// orth is CholeskyQR with fp64 Gram and Cholesky (Fukaya et al. 2014): one
// pass between products, two (CholeskyQR2) for the Rayleigh-Ritz basis; the
// l x l eigenproblem is solved by cyclic two-sided Jacobi (Golub & Van Loan,
// §8.5) in fp64 in one wave, with parallel (round-robin) ordering.  The
// products A X of the iteration but the last run on the fp32 matrix cores
// (fp32 partial sums over row ranges, added in fp64), the last one and the
// Rayleigh-Ritz product Z = A Q on the fp64 ones.
// A is read as fp32; every other quantity is fp64 until the basis U and the
// coefficient vectors are written as fp32.
#include "gift_internal.hpp"

namespace gift {

// Small-buffer layout (fp64 elements).
constexpr int kSmTrace = 0;            // [0] tr(A)
constexpr int kSmSolved = 1;           // [1] 1: the tridiagonal solver wrote the factor
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

// Partial products of Y = A X for symmetric A (fp32, d x d) and X (fp64,
// d x LP): part[s][i][c] = sum_{j in row range s} A[j][i] X[j][c], which is
// (A X)[i][c] summed over the ranges.  fp64 matrix cores
// (v_mfma_f64_16x16x4f64): lane l supplies the A operand Aop[l % 16][l / 16]
// and the B operand Bop[l / 16][l % 16]; slot e of lane l holds
// D[4 e + l / 16][l % 16].  Here Aop[m][k] = A[j + k][i + m] (A's symmetry:
// rows of A are read, coalesced) and Bop[k][n] = X[j + k][n].  Wave w of
// workgroup (b, s) owns columns 256 b + 64 w .. + 63 of A; A is read from
// memory once, X (a few MB) from L2.  A's fp32 values are exact in fp64.
typedef double double4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int LP>
__global__ void __launch_bounds__(256) k_aq(const float* __restrict__ A, int d, const double* __restrict__ X,
                                            int jrows, double* __restrict__ part) {
  constexpr int NT = LP / 16;    // output column tiles
  constexpr int KB = 6;          // 4-row k-steps per block (24 rows; 4 and 8 measured slower)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lk = lane >> 4;
  const int i0 = blockIdx.x * kAqCols + wave * 64;
  const int j0 = blockIdx.y * jrows;
  const int j1 = min(d, j0 + jrows);
  int ic[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) ic[mt] = min(i0 + 16 * mt + lm, d - 1);   // clamped: loads stay in bounds
  double4v acc[4][NT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (double4v){0.0, 0.0, 0.0, 0.0};
  struct Blk {
    float a[KB][4];
    double b[KB][NT];
  };
  auto load = [&](int jb, Blk& t) {
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) {
      const int jr = min(jb + 4 * ks + lk, d - 1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) t.a[ks][mt] = A[(int64_t)jr * d + ic[mt]];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) t.b[ks][nt] = X[(int64_t)jr * LP + 16 * nt + lm];
    }
  };
  auto compute = [&](int jb, const Blk& t) {
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) {
      const bool in = jb + 4 * ks + lk < j1;   // rows past the range contribute zero
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const double av = in ? (double)t.a[ks][mt] : 0.0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, t.b[ks][nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };
  Blk cur, nxt;
  load(j0, cur);
  for (int jb = j0; jb < j1; jb += 4 * KB) {
    if (jb + 4 * KB < j1) load(jb + 4 * KB, nxt);   // in flight while this block computes
    compute(jb, cur);
    cur = nxt;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = i0 + 16 * mt + 4 * e + lk;
        if (row < d) part[((int64_t)blockIdx.y * d + row) * LP + 16 * nt + lm] = acc[mt][nt][e];
      }
}

// The same product on the fp32 matrix cores (v_mfma_f32_16x16x4f32, twice
// the fp64 rate) for the products of the subspace iteration, whose errors
// only perturb the basis that the next product and orthonormalisation
// carry on (the Rayleigh-Ritz product keeps fp64).  X is rounded to fp32 on
// load; A's fp32 values are exact; sums are fp32.  Workgroup (b, s) owns 64
// columns of A and row range s; its 4 waves take a quarter of the range
// each and their accumulators are added in LDS in wave order.  Slot e of
// lane l holds D[4 (l / 16) + e][l % 16].  The partials of the ranges are
// fp32 and summed in fp64 by k_sum_parts32.
template <int LP>
__global__ void __launch_bounds__(256) k_aq32(const float* __restrict__ A, int d, const double* __restrict__ X,
                                              int jrows, float* __restrict__ part) {
  constexpr int NT = LP / 16;
  constexpr int KB = 4;   // 4-row k-steps per block (16 rows)
  __shared__ floatx4 red[3][4][NT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lk = lane >> 4;
  const int i0 = blockIdx.x * 64;
  const int js = blockIdx.y * jrows, je = min(d, js + jrows);
  const int qr = jrows / 4;
  const int j0 = min(je, js + wave * qr), j1 = min(je, j0 + qr);
  int ic[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) ic[mt] = min(i0 + 16 * mt + lm, d - 1);   // clamped: loads stay in bounds
  floatx4 acc[4][NT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (floatx4){0.f, 0.f, 0.f, 0.f};
  struct Blk {
    float a[KB][4];
    double b[KB][NT];
  };
  auto load = [&](int jb, Blk& t) {
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) {
      const int jr = min(jb + 4 * ks + lk, d - 1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) t.a[ks][mt] = A[(int64_t)jr * d + ic[mt]];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) t.b[ks][nt] = X[(int64_t)jr * LP + 16 * nt + lm];
    }
  };
  auto compute = [&](int jb, const Blk& t) {
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) {
      const bool in = jb + 4 * ks + lk < j1;   // rows past the range contribute zero
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float av = in ? t.a[ks][mt] : 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, (float)t.b[ks][nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };
  if (j0 < j1) {
    Blk cur, nxt;
    load(j0, cur);
    for (int jb = j0; jb < j1; jb += 4 * KB) {
      if (jb + 4 * KB < j1) load(jb + 4 * KB, nxt);   // in flight while this block computes
      compute(jb, cur);
      cur = nxt;
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[wave - 1][mt][nt][lane] = acc[mt][nt];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        floatx4 v = acc[mt][nt];
#pragma unroll
        for (int w = 0; w < 3; ++w) v += red[w][mt][nt][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = i0 + 16 * mt + 4 * lk + e;
          if (row < d) part[((int64_t)blockIdx.y * d + row) * LP + 16 * nt + lm] = v[e];
        }
      }
  }
}

// out[e] = sum_p part[p][e] in fp64, in order p = 0, 1, ... (deterministic)
__global__ void __launch_bounds__(256) k_sum_parts32(const float* __restrict__ part, int nparts, int64_t n,
                                                     double* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  double s = 0.0;
  for (int p = 0; p < nparts; ++p) s += (double)part[(int64_t)p * n + e];
  out[e] = s;
}

// out[e] = sum_{p < nparts} part[p][e], in order p = 0, 1, ... (deterministic).
// Sixteen independent loads in flight per thread, added in order: the l x l
// Gram sums have few elements (2304 threads) and many partials, so the
// load latency, not the bytes, sets their time.
__global__ void __launch_bounds__(256) k_sum_parts(const double* __restrict__ part, int nparts, int64_t n,
                                                   double* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  constexpr int U = 16;
  double s = 0.0;
  int p = 0;
  for (; p + U <= nparts; p += U) {
    double v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = part[(int64_t)(p + u) * n + e];
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u];
  }
  for (; p < nparts; ++p) s += part[(int64_t)p * n + e];
  out[e] = s;
}

// part[ch][a][b] = sum_{i in rows of chunk ch} X[i][a] Y[i][b]  (fp64, LP a
// multiple of 16, at most 64), each entry summed over the chunk's rows in
// order.  Thread (ta, tb) of the 16 x 16 grid owns the BS x BS block of
// entries a = BS ta + u, b = BS tb + v (BS = LP / 16): per row it reads BS
// values of X and BS of Y from LDS for BS^2 products.
template <int LP>
__global__ void __launch_bounds__(256) k_gram_parts(const double* __restrict__ X, const double* __restrict__ Y,
                                                    int d, double* __restrict__ part) {
  static_assert(LP % 16 == 0 && LP <= 64, "16 x 16 thread blocks");
  constexpr int BS = LP / 16;
  __shared__ double Xs[32][LP];
  __shared__ double Ys[32][LP];
  const int ta = threadIdx.x >> 4, tb = threadIdx.x & 15;
  double acc[BS][BS];
#pragma unroll
  for (int u = 0; u < BS; ++u)
#pragma unroll
    for (int v = 0; v < BS; ++v) acc[u][v] = 0.0;
  const int r0 = blockIdx.x * kGramRows;
  for (int s0 = r0; s0 < min(d, r0 + kGramRows); s0 += 32) {
    for (int e = threadIdx.x; e < 32 * LP; e += 256) {
      int rr = e / LP, c = e % LP;
      bool ok = s0 + rr < d && s0 + rr < r0 + kGramRows;
      Xs[rr][c] = ok ? X[(int64_t)(s0 + rr) * LP + c] : 0.0;
      Ys[rr][c] = ok ? Y[(int64_t)(s0 + rr) * LP + c] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < 32; ++rr) {
      double xa[BS], yb[BS];
#pragma unroll
      for (int u = 0; u < BS; ++u) xa[u] = Xs[rr][BS * ta + u];
#pragma unroll
      for (int v = 0; v < BS; ++v) yb[v] = Ys[rr][BS * tb + v];
#pragma unroll
      for (int u = 0; u < BS; ++u)
#pragma unroll
        for (int v = 0; v < BS; ++v) acc[u][v] += xa[u] * yb[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < BS; ++u)
#pragma unroll
    for (int v = 0; v < BS; ++v)
      part[(int64_t)blockIdx.x * LP * LP + (BS * ta + u) * LP + BS * tb + v] = acc[u][v];
}

// v of lane j (j uniform) in every lane, through two v_readlane (no LDS
// round trip).
__device__ __forceinline__ double lane_bcast(double v, int j) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, j), hi = __builtin_amdgcn_readlane((int)(b >> 32), j);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// 1 / sqrt(x) from the hardware estimate and two Newton steps (about one
// ulp: the rotations stay orthogonal to rounding).
__device__ __forceinline__ double rsq_nr(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * (1.5 - 0.5 * x * y * y);
  return y * (1.5 - 0.5 * x * y * y);
}

// One wave: G (LP x LP, leading l x l used) = L L^T, writes M = L^-T (upper
// triangular, zero outside l x l) into small[kSmM].  Lane i keeps row i of
// L in registers (left-looking: at step j it forms L[i][j] from its own row
// and row j of L, read from LDS where each lane stores its new element), and
// then column i of L^-1 (forward substitution against the rows of L in
// LDS).  Both loops are unrolled over the compile-time size, so every
// register index is a constant and the LDS reads of a step are broadcasts
// issued together.  One wave keeps its LDS accesses in program order, so no
// barrier is needed.  Rows and columns past l are the identity.
template <int LP>
__global__ void __launch_bounds__(64) k_chol_inv_small(const double* __restrict__ G, int l,
                                                       double* __restrict__ small, uint32_t* __restrict__ flags) {
  static_assert(LP <= 64, "one lane per row");
  __shared__ __attribute__((aligned(16))) double Ls[LP][LP + 2];   // L, row-major, rows 16-byte aligned
  __shared__ double Dinv[LP];                                        // 1 / L[j][j]
  const int i = threadIdx.x;
  const bool own = i < LP;
  const int ir = own ? i : LP - 1;   // lanes past LP load a valid row and never store
  double row[LP];                    // G[i][q] for q >= j, L[i][q] for q < j
#pragma unroll
  for (int q = 0; q < LP; ++q) {
    const double g = G[ir * LP + q];
    row[q] = (i < l && q < l) ? g : (i == q ? 1.0 : 0.0);
  }
  bool bad = false;
#pragma unroll
  for (int j = 0; j < LP; ++j) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};   // four chains
#pragma unroll
    for (int q = 0; q < j; ++q) acc[q & 3] += row[q] * Ls[j][q];
    const double r = row[j] - ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    const double dj = lane_bcast(r, j);   // the pivot, from lane j
    double rs = rsq_nr(dj);               // 1 / L[j][j]
    if (!(dj > 0.0)) {
      bad = true;
      rs = __longlong_as_double(0x7FF8000000000000LL);
    }
    row[j] = i > j ? r * rs : (i == j ? dj * rs : 0.0);
    if (own) Ls[i][j] = row[j];
    if (i == 0) Dinv[j] = rs;
  }
  double x[LP];   // column i of L^-1: x[q] = (L^-1)[q][i], zero above the diagonal
#pragma unroll
  for (int rr = 0; rr < LP; ++rr) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < rr; ++q) acc[q & 3] += Ls[rr][q] * x[q];
    const double v = (rr == i ? 1.0 : 0.0) - ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    x[rr] = rr >= i ? v * Dinv[rr] : 0.0;
  }
  if (own) {
#pragma unroll
    for (int c = 0; c < LP; ++c) small[kSmM + i * LP + c] = (i < l && c < l) ? x[c] : 0.0;
  }
  if (i == 0 && bad) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
}

// out[i][:NC] = X[i][:LP] * M[:LP][:NC] with M in small[kSmM] ([LP][ldm]).
// Thread (i, g) computes the 8 outputs of row i in column group g; the rows
// of X are read by the NC / 8 threads of a row together (one broadcast).
template <int LP, int NC, typename TO>
__global__ void __launch_bounds__(256) k_right_small(const double* __restrict__ X, int d,
                                                     const double* __restrict__ small, int ldm,
                                                     TO* __restrict__ out) {
  constexpr int CPT = 8, NG = NC / CPT;
  __shared__ double Ms[LP][NC];
  for (int o = threadIdx.x; o < LP * NC; o += 256) Ms[o / NC][o % NC] = small[kSmM + (o / NC) * ldm + (o % NC)];
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int i = t / NG, g = t % NG;
  if (i >= d) return;
  double acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.0;
  double xr[LP];   // the whole row in flight at once
#pragma unroll
  for (int a = 0; a < LP; ++a) xr[a] = X[(int64_t)i * LP + a];
#pragma unroll
  for (int a = 0; a < LP; ++a) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] += xr[a] * Ms[a][g * CPT + c];
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) out[(int64_t)i * NC + g * CPT + c] = (TO)acc[c];
}

// Outputs of the Rayleigh-Ritz step, shared by both solvers: order[t] is the
// t-th largest Ritz value's index, theta(a) its value, vec(r, a) component r
// of its eigenvector.  V_k into small[kSmM] as [LP][32], the sorted Ritz
// values into small[kSmTheta], and the coefficient vectors (c_enc, c_dec,
// rho^-1/2, rho^1/2, lambda, rho) into coef.  Called by every thread after
// a barrier that made order, theta and vec visible.
template <int LP, typename TF, typename VF>
__device__ __forceinline__ void store_factor(int l, int k, int d, float damping_rel, const int* order, TF theta,
                                             VF vec, double* __restrict__ small, float* __restrict__ coef,
                                             uint32_t* __restrict__ flags) {
  const int tid = threadIdx.x;
  for (int o = tid; o < LP * 32; o += 256) {
    int a = o / 32, t = o % 32;
    small[kSmM + o] = (a < l && t < k) ? vec(a, order[t]) : 0.0;
  }
  if (tid < LP) small[kSmTheta + tid] = tid < l ? theta(order[tid]) : 0.0;
  __syncthreads();
  if (tid == 0) {
    double tr = small[kSmTrace];
    double lam = (double)damping_rel * tr / (double)d;
    double sum = 0.0;
    for (int t = 0; t < k; ++t) sum += theta(order[t]);
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
        double th = theta(order[t]);
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

// Jacobi rotation annihilating B[p][q] (Golub & Van Loan, Alg. 8.5.1): with
// d = aqq - app and a = 2 apq, t = tan(theta) = sg a / (|d| + sqrt(d^2 + a^2))
// (sg = sign(d), t = sign(a) at d = 0: |t| = 1 there, either root
// annihilates), c = 1 / sqrt(1 + t^2), s = t c.  Taken without a division:
// with h = |d| + sqrt(d^2 + a^2), c = h / sqrt(h^2 + a^2) and
// s = sg a / sqrt(h^2 + a^2).  d and a are first scaled by one power of two
// so that no square overflows or underflows.  Caller: apq != 0.
__device__ __forceinline__ void jacobi_rot(double app, double aqq, double apq, double& c, double& s) {
  double d = aqq - app, a = 2.0 * apq;
  int e;
  (void)frexp(fmax(fabs(d), fabs(a)), &e);
  d = ldexp(d, -e);
  a = ldexp(a, -e);   // max(|d|, |a|) in [0.5, 1)
  const double h2 = fma(d, d, a * a);
  const double h = fabs(d) + h2 * rsq_nr(h2);
  const double num = d < 0.0 ? -a : a;
  const double r = rsq_nr(fma(h, h, num * num));
  c = h * r;
  s = num * r;
}

// One workgroup: B (Q^T A Q, LP x LP, leading l x l used) symmetrised;
// cyclic Jacobi; Ritz values sorted descending (ties: lower index first);
// V_k (the first k sorted eigenvectors) into small[kSmM] as [LP][32];
// coefficients into coef.  A round applies n / 2 disjoint rotations R_i
// (round-robin ordering).  With J their product, B <- J^T B J acts on every
// 2 x 2 block (pair i rows, pair j columns) independently,
// B_ij <- R_i^T B_ij R_j, and V <- V J on pairs of columns; so a round is one
// barrier-free pass over the blocks after the rotations are known.
template <int LP>
__global__ void __launch_bounds__(256) k_jacobi_coef(const double* __restrict__ B0, int l, int k, int d,
                                                     float damping_rel, double* __restrict__ small,
                                                     float* __restrict__ coef, uint32_t* __restrict__ flags,
                                                     int after_tridiagonal) {
  // behind the tridiagonal solver, this kernel only runs when that solver
  // met a cluster of Ritz values and left the factor to it
  if (after_tridiagonal && small[kSmSolved] == 1.0) return;
  constexpr int NP = LP / 2;
  __shared__ double B[LP][LP + 1];
  __shared__ double V[LP][LP + 1];
  __shared__ double cs[NP][2];
  __shared__ int pq[NP][2];
  __shared__ int order[LP];
  __shared__ double red2[256][2];
  const int tid = threadIdx.x;
  {
    constexpr int NE = (LP * LP + 255) / 256;
    double x[NE], y[NE];   // all loads in flight before the first store
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int o = min(tid + 256 * u, LP * LP - 1), a = o / LP, b = o % LP;
      x[u] = B0[a * LP + b];
      y[u] = B0[b * LP + a];
    }
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int o = tid + 256 * u, a = o / LP, b = o % LP;
      if (o < LP * LP) {
        B[a][b] = (a < l && b < l) ? 0.5 * (x[u] + y[u]) : 0.0;
        V[a][b] = a == b ? 1.0 : 0.0;
      }
    }
  }
  const int n = (l + 1) & ~1;   // players in the round-robin (a dummy if l is odd)
  const int npair = n / 2;
  __syncthreads();
  for (int sweep = 0; sweep < 30; ++sweep) {
    for (int round = 0; round < n - 1; ++round) {
      if (tid < npair) {
        // pair tid: players p < q (player 0 fixed, the rest rotate)
        int v = tid - 1 + round;
        if (v >= n - 1) v -= n - 1;
        int w = n - 2 - tid + round;
        if (w >= n - 1) w -= n - 1;
        int p = tid == 0 ? 0 : v + 1, q = w + 1;
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        double c = 1.0, sn = 0.0;
        if (q >= l) {
          q = p;   // the dummy player: identity rotation on row / column p alone
        } else if (B[p][q] != 0.0) {
          jacobi_rot(B[p][p], B[q][q], B[p][q], c, sn);
        }
        cs[tid][0] = c;
        cs[tid][1] = sn;
        pq[tid][0] = p;
        pq[tid][1] = q;
      }
      __syncthreads();
      // every operand is loaded before anything is stored (the blocks are
      // disjoint), so the loads of all of a thread's blocks are in flight
      // together
      constexpr int NB = (NP * NP + 255) / 256, NV = (LP * NP + 255) / 256;
      double bb[NB][4], rr[NB][4], vv[NV][2];
      int bi[NB][4], vi[NV][2];
      bool bok[NB], vok[NV];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int o = tid + 256 * u, i = o / NP, j = o % NP;
        bok[u] = o < NP * NP && i < npair && j < npair;
        const int ii = bok[u] ? i : 0, jj = bok[u] ? j : 0;
        const int pi = pq[ii][0], qi = pq[ii][1], pj = pq[jj][0], qj = pq[jj][1];
        bi[u][0] = pi * (LP + 1) + pj;
        bi[u][1] = pi * (LP + 1) + qj;
        bi[u][2] = qi * (LP + 1) + pj;
        bi[u][3] = qi * (LP + 1) + qj;
#pragma unroll
        for (int e = 0; e < 4; ++e) bb[u][e] = (&B[0][0])[bi[u][e]];
        const double ci = cs[ii][0], si = cs[ii][1], cj = cs[jj][0], sj = cs[jj][1];
        // rows (R_i^T), then columns (R_j)
        const double rpp = ci * bb[u][0] - si * bb[u][2], rpq = ci * bb[u][1] - si * bb[u][3];
        const double rqp = si * bb[u][0] + ci * bb[u][2], rqq = si * bb[u][1] + ci * bb[u][3];
        rr[u][0] = cj * rpp - sj * rpq;
        rr[u][1] = sj * rpp + cj * rpq;
        rr[u][2] = cj * rqp - sj * rqq;
        rr[u][3] = sj * rqp + cj * rqq;
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int o = tid + 256 * u, r = o / NP, j = o % NP;
        vok[u] = o < LP * NP && r < l && j < npair;
        const int jj = vok[u] ? j : 0, r0 = vok[u] ? r : 0;
        const int pj = pq[jj][0], qj = pq[jj][1];
        vi[u][0] = r0 * (LP + 1) + pj;
        vi[u][1] = r0 * (LP + 1) + qj;
        const double vp = (&V[0][0])[vi[u][0]], vq = (&V[0][0])[vi[u][1]];
        const double cj = cs[jj][0], sj = cs[jj][1];
        vv[u][0] = cj * vp - sj * vq;
        vv[u][1] = sj * vp + cj * vq;
      }
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (bok[u]) {
#pragma unroll
          for (int e = 0; e < 4; ++e) (&B[0][0])[bi[u][e]] = rr[u][e];
        }
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (vok[u]) {
          (&V[0][0])[vi[u][0]] = vv[u][0];
          (&V[0][0])[vi[u][1]] = vv[u][1];
        }
      __syncthreads();
    }
    // off-diagonal and total squared norms (fixed-order tree reduction)
    double off = 0.0, all = 0.0;
    for (int o = tid; o < l * l; o += 256) {
      const int a = o / l, b = o % l;
      const double v = B[a][b] * B[a][b];
      all += v;
      if (a != b) off += v;
    }
    red2[tid][0] = off;
    red2[tid][1] = all;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if (tid < h) {
        red2[tid][0] += red2[tid + h][0];
        red2[tid][1] += red2[tid + h][1];
      }
      __syncthreads();
    }
    const bool done = red2[0][0] <= 1e-26 * red2[0][1];   // off-norm below 1e-13 of the norm
    __syncthreads();
    if (done) break;
  }
  if (tid == 0) {   // sort Ritz values descending (stable) -- one thread, l <= 64
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
  store_factor<LP>(l, k, d, damping_rel, order, [&](int a) { return B[a][a]; },
                   [&](int r, int a) { return V[r][a]; }, small, coef, flags);
}

// Sum over the 64 lanes of a wave, the same value in every lane: rotations
// inside each 16-lane row (DPP row_ror 8, 4, 2, 1), then the row swaps
// (v_permlane16_swap, v_permlane32_swap), each on the two 32-bit halves;
// lane 0's total is broadcast (the lanes' rounding orders differ, so one
// lane decides).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double pair_d(unsigned lo0, unsigned hi0, unsigned lo1, unsigned hi1) {
  return __longlong_as_double(((long long)hi0 << 32) | lo0) + __longlong_as_double(((long long)hi1 << 32) | lo1);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0x128>(v);
  v += dpp_d<0x124>(v);
  v += dpp_d<0x122>(v);
  v += dpp_d<0x121>(v);
  {
    const long long b = __double_as_longlong(v);
    const auto pl = __builtin_amdgcn_permlane16_swap((unsigned)b, (unsigned)b, false, false);
    const auto ph = __builtin_amdgcn_permlane16_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);
    v = pair_d(pl[0], ph[0], pl[1], ph[1]);
  }
  {
    const long long b = __double_as_longlong(v);
    const auto pl = __builtin_amdgcn_permlane32_swap((unsigned)b, (unsigned)b, false, false);
    const auto ph = __builtin_amdgcn_permlane32_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);
    v = pair_d(pl[0], ph[0], pl[1], ph[1]);
  }
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, 0), hi = __builtin_amdgcn_readlane((int)(b >> 32), 0);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Rayleigh-Ritz step by a tridiagonal reduction (used for l <= 48; the
// Jacobi kernel above stays as the solver for clustered spectra and for
// larger l).  One workgroup of 256 threads:
//  1. Householder reduction of the symmetric B to tridiagonal T = H^T B H
//     (Golub & Van Loan, Alg. 8.3.1): step j reflects column j below the
//     diagonal onto its first entry with v = x - alpha e1, alpha =
//     -sign(x1) |x|, and updates the trailing block S <- S - v w^T - w v^T
//     with p = beta S v, w = p - (beta/2)(p^T v) v, beta = 2 / v^T v.
//  2. T is split where a coupling is below eps (|d_i| + |d_i+1|); the
//     eigenvalues of each unreduced block come from bisection on Sturm counts
//     (the sign changes of the leading principal minors of T - s I, GvL
//     8.4.1), five evaluation points per step on five lanes of a wave (the
//     interval shrinks six-fold per step).
//  3. If two neighbouring eigenvalues of one block, both among the k largest,
//     are closer than 1e-8 of |T|, the eigenvectors below would not be
//     reliably orthogonal (a computed vector's angle to the true one is
//     about its residual, O(eps |T|), over the gap to the next eigenvalue,
//     here kept below the factor's fp32 rounding): the kernel leaves the
//     step to the Jacobi kernel (small[kSmSolved] = 0).
//  4. Each eigenvector of T from one twisted factorisation at its eigenvalue
//     (Dhillon and Parlett's twisted factorisation of T - lambda I: the
//     forward LDL^T and backward UDU^T pivots D+ and D-, the twist index r
//     minimising |D+_r + D-_r - (d_r - lambda)|, then z_r = 1 and the two
//     one-sided recurrences), normalised.
//  5. The eigenvectors of B are H z (the reflections applied in reverse).
// Every sum runs in a fixed order, so the result is deterministic.
template <int LP>
__global__ void __launch_bounds__(256) k_tridiag_coef(const double* __restrict__ B0, int l, int k, int d,
                                                      float damping_rel, double* __restrict__ small,
                                                      float* __restrict__ coef, uint32_t* __restrict__ flags) {
  static_assert(LP <= 48, "slots: 12 per wave, five lanes each");
  __shared__ double Bm[LP][LP + 1];
  __shared__ double HV[LP][LP];          // HV[j][i]: component i of the reflection vector of step j
  __shared__ double Zc[LP][LP + 1];      // Zc[i][g]: component i of eigenvector g
  __shared__ double Fw[3][LP][LP];       // per eigenvector g: D+ [0][i][g], L [1][i][g], U [2][i][g]
  __shared__ double dd[LP], ee[LP], e2[LP], hb[LP], vv[LP], wv[LP], th[LP];
  __shared__ int blk0[LP], blk1[LP], rk[LP], order[LP];
  __shared__ double s_tn, s_pivmin, s_glo, s_ghi;
  __shared__ int s_cluster;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // scaled copies of the diagonal and squared couplings for the bisection,
  // in the eigenvector work area (free until then)
  auto hv_dr = [&](int i) -> double& { return Fw[0][i][0]; };
  auto hv_er = [&](int i) -> double& { return Fw[0][i][1]; };
  const int n = l;
  const double eps = 0x1p-52;
  for (int o = tid; o < LP * LP; o += 256) {
    const int a = o / LP, b = o % LP;
    Bm[a][b] = (a < n && b < n) ? 0.5 * (B0[a * LP + b] + B0[b * LP + a]) : 0.0;
    Zc[a][b] = 0.0;
    HV[a][b] = 0.0;
  }
  if (tid < LP) {
    dd[tid] = 0.0;
    ee[tid] = 0.0;
    e2[tid] = 0.0;
  }
  __syncthreads();
  // 1. Householder reduction by wave 0: lane r holds row r of the matrix in
  // registers (compile-time column indices, the steps unrolled); by symmetry
  // step j's column below the diagonal is entry j of each lane's row.  The
  // wave's LDS accesses complete in program order, so the steps need no
  // barrier.
  if (wave == 0) {
    double row[LP];
    const int rl = lane < LP ? lane : LP - 1;   // lanes past LP carry a copy and change nothing
#pragma unroll
    for (int c = 0; c < LP; ++c) row[c] = Bm[rl][c];
#pragma unroll
    for (int j = 0; j + 2 < LP; ++j) {
      if (j + 2 < n) {
        const bool act = lane > j && lane < n;   // rows j + 1 .. n - 1
        const double cj = row[j];
        const double x = act ? cj : 0.0;
        const double sig = wave_sum_d(x * x);
        const long long cb = __double_as_longlong(cj);
        const int x0l = __builtin_amdgcn_readlane((int)cb, j + 1), x0h = __builtin_amdgcn_readlane((int)(cb >> 32), j + 1);
        const double x0 = __longlong_as_double(((long long)x0h << 32) | (unsigned)x0l);
        double beta = 0.0, alpha = x0, v = 0.0;
        if (sig > 0.0) {
          alpha = -copysign(sqrt(sig), x0);
          const double v0 = x0 - alpha;
          v = act ? (lane == j + 1 ? v0 : x) : 0.0;
          beta = 2.0 / (sig - x0 * x0 + v0 * v0);
        }
        if (lane < LP) {
          vv[lane] = v;   // zero outside rows j + 1 .. n - 1
          HV[j][lane] = v;
        }
        if (lane == j) {
          hb[j] = beta;
          ee[j] = alpha;
          dd[j] = cj;
        }
        __builtin_amdgcn_wave_barrier();
        // p = beta S v, w = p - (beta/2)(p^T v) v (v_c and w_c read as LDS
        // broadcasts)
        double a4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int c = j + 1; c < LP; ++c) a4[(c - j - 1) & 3] += row[c] * vv[c];
        const double acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
        const double pr = act ? beta * acc : 0.0;
        const double K = 0.5 * beta * wave_sum_d(pr * v);
        const double wr = act ? pr - K * v : 0.0;
        if (lane < LP) wv[lane] = wr;
        __builtin_amdgcn_wave_barrier();
        // S <- S - v w^T - w v^T (rows outside the block have v = w = 0)
#pragma unroll
        for (int c = j + 1; c < LP; ++c) row[c] -= v * wv[c] + wr * vv[c];
        __builtin_amdgcn_wave_barrier();
      }
    }
    // the trailing 2 x 2 block for the entries below
    if (lane < LP) {
#pragma unroll
      for (int c = 0; c < LP; ++c) Bm[lane][c] = row[c];
    }
  }
  __syncthreads();
  // 2. the last diagonal and coupling entries; then by wave 0, lane i for
  // row i: the norm |T| (largest absolute row sum), the split, the squared
  // couplings and a Gershgorin interval of the split T (the union of its
  // blocks' intervals, so it holds every block's eigenvalues)
  if (tid == 0) {
    if (n >= 2) {
      dd[n - 2] = Bm[n - 2][n - 2];
      ee[n - 2] = Bm[n - 1][n - 2];
    }
    dd[n - 1] = Bm[n - 1][n - 1];
  }
  __syncthreads();
  if (wave == 0) {
    const bool in = lane < n, cpl = lane + 1 < n;
    // each lane reads and writes only its own coupling; its left neighbour's
    // comes by a shuffle, before and after the split
    const double di = in ? dd[lane] : 0.0, dn = cpl ? dd[lane + 1] : 0.0;
    double er = cpl ? ee[lane] : 0.0;
    const double el = __shfl_up(er, 1, 64);
    double tn = fabs(di) + (lane > 0 ? fabs(el) : 0.0) + fabs(er);
    if (cpl && fabs(er) <= eps * (fabs(di) + fabs(dn))) er = 0.0;
    double me2 = er * er;
    if (cpl) {
      ee[lane] = er;
      e2[lane] = er * er;
    }
    const double els = __shfl_up(er, 1, 64);
    const double r = (lane > 0 ? fabs(els) : 0.0) + fabs(er);
    double lo = in ? di - r : 0.0, hi = in ? di + r : 0.0;
    lo = in ? lo : __shfl(lo, 0, 64);
    hi = in ? hi : __shfl(hi, 0, 64);
    for (int o = 32; o > 0; o >>= 1) {
      tn = fmax(tn, __shfl_xor(tn, o, 64));
      me2 = fmax(me2, __shfl_xor(me2, o, 64));
      lo = fmin(lo, __shfl_xor(lo, o, 64));
      hi = fmax(hi, __shfl_xor(hi, o, 64));
    }
    if (lane == 0) {
      s_tn = tn > 0.0 ? tn : 0x1p-1022;
      s_pivmin = 0x1p-1022 * fmax(me2, 1.0);
      s_glo = lo;
      s_ghi = hi;
      s_cluster = 0;
    }
  }
  __syncthreads();
  const double tn = s_tn, pivmin = s_pivmin;
  // eigenvalue slot g: its unreduced block [blk0, blk1), from the mask of
  // zero couplings (bit i: rows i and i + 1 decoupled)
  {
    const unsigned long long zm = __ballot(lane + 1 < n && ee[lane < LP ? lane : 0] == 0.0);
    if (tid < n) {
      const unsigned long long below = zm & ((1ull << tid) - 1ull), above = zm >> tid;
      blk0[tid] = below ? 64 - __clzll((long long)below) : 0;
      blk1[tid] = above ? tid + __ffsll((long long)above) : n;
    }
  }
  // bisection: slot g on lanes 5 (g % 12) .. + 4 of wave g / 12.  The
  // Sturm count is taken as the sign changes of the sequence of leading
  // principal minors of T - s I, p_i = (d_i - s) p_i-1 - e_i-1^2 p_i-2 (one
  // fma on the critical path per term, no division), on T scaled by a power
  // of two to |T| < 1, the pair (p_i-1, p_i) rescaled by a power of two every
  // eight terms; a zero term takes the sign opposite to the one before it.
  // The scaled diagonal and squared couplings are read as LDS broadcasts
  // (their addresses are fixed, so the reads run ahead of the recurrence).
  int tex;
  (void)frexp(tn, &tex);
  if (tid < LP) {
    hv_dr(tid) = ldexp(dd[tid], -tex);
    hv_er(tid) = ldexp(e2[tid], -2 * tex);
  }
  __syncthreads();
  {
    const int g = 12 * wave + lane / 5, sp = lane % 5;
    if (lane < 60 && g < n) {
      const int a = blk0[g], b = blk1[g], idx = b - 1 - g;   // ascending index of the (g - a)-th largest
      double lam;
      if (b - a == 1) {
        lam = dd[g];
      } else {
        double lo = s_glo - 2.0 * eps * tn, hi = s_ghi + 2.0 * eps * tn;
        const int base = lane - sp;
        for (int it = 0; it < 64; ++it) {
          const double w = hi - lo;
          const double pt = lo + w * (double)(sp + 1) * (1.0 / 6.0);
          const double ps = ldexp(pt, -tex);
          int cnt = 0;
          double p0 = 1.0, p1 = 1.0;
          if (a == 0 && b == LP) {   // one unreduced block over all LP rows: no per-term test
            // (a zero term in the middle gives the same count whatever sign
            // it is given; only a zero last term, s an eigenvalue of T, can
            // move the count by one, which the bracketing tolerates)
#pragma unroll
            for (int i = 0; i < LP; ++i) {
              double pn = hv_dr(i) - ps;
              if (i > 0) pn = fma(pn, p1, -hv_er(i > 0 ? i - 1 : 0) * p0);
              cnt += (int)((uint32_t)(__double2hiint(pn) ^ __double2hiint(p1)) >> 31);
              p0 = p1;
              p1 = pn;
              if ((i & 7) == 7) {
                int ex;
                (void)frexp(p1, &ex);
                p1 = ldexp(p1, -ex);
                p0 = ldexp(p0, -ex);
              }
            }
          } else {
#pragma unroll
          for (int i = 0; i < LP; ++i) {
            if (i >= a && i < b) {
              double pn = hv_dr(i) - ps;
              if (i > a) pn = fma(pn, p1, -hv_er(i > 0 ? i - 1 : 0) * p0);
              if (pn == 0.0) pn = -copysign(0x1p-1000, p1);
              cnt += (pn < 0.0) != (p1 < 0.0);
              p0 = p1;
              p1 = pn;
              if ((i & 7) == 7) {
                int ex;
                (void)frexp(p1, &ex);
                p1 = ldexp(p1, -ex);
                p0 = ldexp(p0, -ex);
              }
            }
          }
          }
          double nlo = lo, nhi = hi;
#pragma unroll
          for (int t = 0; t < 5; ++t) {
            const int ct = __shfl(cnt, base + t, 64);
            const double ptt = lo + w * (double)(t + 1) * (1.0 / 6.0);
            if (ct <= idx) nlo = ptt;
          }
#pragma unroll
          for (int t = 4; t >= 0; --t) {
            const int ct = __shfl(cnt, base + t, 64);
            const double ptt = lo + w * (double)(t + 1) * (1.0 / 6.0);
            if (ct > idx) nhi = ptt;
          }
          // absolute tolerance 4 eps |T| (the k largest are far above it)
          const bool done = (nlo == lo && nhi == hi) || nhi - nlo <= 4.0 * eps * tn;
          lo = nlo;
          hi = nhi;
          if (done) break;
        }
        lam = 0.5 * (lo + hi);
      }
      if (sp == 0) th[g] = lam;
    }
  }
  __syncthreads();
  // ranks (descending, ties to the lower slot) and the cluster test
  if (tid < n) {
    int r = 0;
    const double t = th[tid];
#pragma unroll
    for (int h = 0; h < LP; ++h) r += h < n && ((th[h] > t) || (th[h] == t && h < tid));
    rk[tid] = r;
    order[r] = tid;
  }
  __syncthreads();
  if (tid + 1 < n && blk1[tid] > tid + 1 && rk[tid] < k && rk[tid + 1] < k &&
      fabs(th[tid] - th[tid + 1]) <= 1e-8 * tn)
    s_cluster = 1;
  __syncthreads();
  if (s_cluster) {
    if (tid == 0) small[kSmSolved] = 0.0;
    return;
  }
  // 4. eigenvectors of T, one thread each
  if (tid < n) {
    const int g = tid, a = blk0[g], b = blk1[g];
    const double lam = th[g];
    if (b - a == 1) {
      Zc[g][g] = 1.0;
    } else {
      double dp = dd[a] - lam;
      if (fabs(dp) < pivmin) dp = pivmin;
      Fw[0][a][g] = dp;
      // the divisions by a refined hardware reciprocal (one Newton step)
      auto rcp = [](double x) {
        const double r = __builtin_amdgcn_rcp(x);
        return fma(r, fma(-x, r, 1.0), r);
      };
      for (int i = a; i + 1 < b; ++i) {
        const double L = ee[i] * rcp(dp);
        dp = dd[i + 1] - lam - L * ee[i];
        if (fabs(dp) < pivmin) dp = pivmin;
        Fw[1][i][g] = L;
        Fw[0][i + 1][g] = dp;
      }
      double dm = dd[b - 1] - lam;
      if (fabs(dm) < pivmin) dm = pivmin;
      int r = b - 1;
      double best = fabs(Fw[0][b - 1][g] + dm - (dd[b - 1] - lam));
      for (int i = b - 2; i >= a; --i) {
        const double U = ee[i] * rcp(dm);
        dm = dd[i] - lam - U * ee[i];
        if (fabs(dm) < pivmin) dm = pivmin;
        Fw[2][i][g] = U;
        const double gam = fabs(Fw[0][i][g] + dm - (dd[i] - lam));
        if (gam < best) {
          best = gam;
          r = i;
        }
      }
      double z = 1.0, nrm = 1.0;
      Zc[r][g] = 1.0;
      for (int i = r - 1; i >= a; --i) {
        z = -Fw[1][i][g] * z;
        Zc[i][g] = z;
        nrm += z * z;
      }
      z = 1.0;
      for (int i = r; i + 1 < b; ++i) {
        z = -Fw[2][i][g] * z;
        Zc[i + 1][g] = z;
        nrm += z * z;
      }
      const double sc = 1.0 / sqrt(nrm);
      for (int i = a; i < b; ++i) Zc[i][g] *= sc;
    }
  }
  __syncthreads();
  // 5. back-transformation: thread g applies the reflections, last first,
  // to column g held in registers
  if (tid < n) {
    double z[LP];
#pragma unroll
    for (int i = 0; i < LP; ++i) z[i] = Zc[i][tid];
#pragma unroll
    for (int j = LP - 3; j >= 0; --j) {
      if (j + 2 < n) {
        double a4[4] = {0.0, 0.0, 0.0, 0.0};   // four chains
#pragma unroll
        for (int i = j + 1; i < LP; ++i) a4[(i - j - 1) & 3] += HV[j][i] * z[i];
        const double sj = hb[j] * ((a4[0] + a4[1]) + (a4[2] + a4[3]));
#pragma unroll
        for (int i = j + 1; i < LP; ++i) z[i] -= sj * HV[j][i];
      }
    }
#pragma unroll
    for (int i = 0; i < LP; ++i) Zc[i][tid] = z[i];
  }
  __syncthreads();
  store_factor<LP>(l, k, d, damping_rel, order, [&](int a) { return th[a]; }, [&](int r, int a) { return Zc[r][a]; },
                   small, coef, flags);
  if (tid == 0) small[kSmSolved] = 1.0;
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
  const int nchG = (int)cdiv(d, kGramRows);
  const unsigned eb = (unsigned)cdiv((int64_t)d * LP, 256);
  hipLaunchKernelGGL(k_trace, dim3(1), dim3(1024), 0, s, A, d, small + kSmTrace);
  hipLaunchKernelGGL(k_omega64, dim3(eb), dim3(256), 0, s, omega, d, l, LP, Q);
  double* apart = reinterpret_cast<double*>(work + w.apart);
  double* gsum = gpart + (int64_t)nchG * LP * LP;      // the summed l x l matrix
  const int jrows = aq_rows_per_split(d), nsplit = aq_splits(d);
  const int64_t ny = (int64_t)d * LP;
  auto product = [&](const double* X, double* out) {   // out = A X (fp64 matrix cores)
    hipLaunchKernelGGL((k_aq<LP>), dim3((unsigned)cdiv(d, kAqCols), (unsigned)nsplit), dim3(256), 0, s, A, d, X,
                       jrows, apart);
    hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)cdiv(ny, 256)), dim3(256), 0, s, apart, nsplit, ny, out);
  };
  const int jrows32 = aq32_rows_per_split(d), nsplit32 = aq32_splits(d);
  auto product32 = [&](const double* X, double* out) {   // out = A X (fp32 matrix cores, fp64 result)
    float* p32 = reinterpret_cast<float*>(apart);
    hipLaunchKernelGGL((k_aq32<LP>), dim3((unsigned)cdiv(d, 64), (unsigned)nsplit32), dim3(256), 0, s, A, d, X,
                       jrows32, p32);
    hipLaunchKernelGGL(k_sum_parts32, dim3((unsigned)cdiv(ny, 256)), dim3(256), 0, s, p32, nsplit32, ny, out);
  };
  auto gram = [&](const double* X, const double* Y2) {  // gsum = X^T Y2
    hipLaunchKernelGGL((k_gram_parts<LP>), dim3(nchG), dim3(256), 0, s, X, Y2, d, gpart);
    hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)cdiv(LP * LP, 256)), dim3(256), 0, s, gpart, nchG,
                       (int64_t)LP * LP, gsum);
  };
  // CholeskyQR with `passes` passes.  Between products only the span of
  // the basis matters (one pass; its orthogonality error, ~kappa^2 eps, is
  // removed by the next pass over the next product); the basis of the
  // Rayleigh-Ritz step takes two passes (CholeskyQR2).
  auto orth = [&](const double* X, double* out, int passes) {
    const double* src = X;
    for (int pass = 0; pass < passes; ++pass) {
      gram(src, src);
      hipLaunchKernelGGL((k_chol_inv_small<LP>), dim3(1), dim3(64), 0, s, gsum, l, small, flags);
      hipLaunchKernelGGL((k_right_small<LP, LP, double>), dim3((unsigned)cdiv((int64_t)d * (LP / 8), 256)),
                         dim3(256), 0, s, src, d, small, LP, out);
      src = out;
    }
  };
  // The products of the iteration but the last on the fp32 matrix cores:
  // their rounding only perturbs the span that the next (exact) product and
  // orthonormalisation carry on.  The last product before the Rayleigh-Ritz
  // basis and the Rayleigh-Ritz product stay fp64.  (Measured on the
  // heavy-tailed 4096 x 16384 stress layer against the oracle's whitening
  // with the factor of the same A: with every product of the iteration in
  // fp32, codes near zero moved by up to 9 E5M2 steps; with all but the last
  // in fp32 the codes agree exactly as with fp64 products after the first
  // two.)
  product32(Q, Y);                    // Y = A Omega
  for (int it = 0; it < q; ++it) {
    orth(Y, Q, 1);                    // Q = orth(Y)
    if (it + 1 < q)
      product32(Q, Y);                // Y = A Q
    else
      product(Q, Y);
  }
  orth(Y, Q, 2);                      // Q = orth(Y)
  product(Q, Z);                      // Z = A Q (fp64: the Rayleigh-Ritz matrix and the Ritz values)
  gram(Q, Z);
  if constexpr (LP <= 48)
    hipLaunchKernelGGL((k_tridiag_coef<LP>), dim3(1), dim3(256), 0, s, gsum, l, k, d, damping_rel, small, coef, flags);
  hipLaunchKernelGGL((k_jacobi_coef<LP>), dim3(1), dim3(256), 0, s, gsum, l, k, d, damping_rel, small, coef, flags,
                     LP <= 48 ? 1 : 0);
  hipLaunchKernelGGL((k_right_small<LP, 32, float>), dim3((unsigned)cdiv((int64_t)d * 4, 256)), dim3(256), 0, s, Q,
                     d, small, 32, U);
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
