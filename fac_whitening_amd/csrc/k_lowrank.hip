// Low-rank input-side transform (whiten / map back) and column scaling.
//
// GIFT 阅读笔记, §简化一 Eq. (16): W~ = W T_A; §简化二 Eq. (17): A ~ U Lam U^T
// with r = 32; Algorithm 1: U = W (L_A)^-T before, W^ = U L_A^T after the
// collective.  With the rank-k form T = U diag(c) U^T + alpha I the product
// is never formed densely:
//     P = X U            (m x k, a skinny contraction over d)
//     out = alpha X + (P diag(c)) U^T
// Encode uses (alpha, c) = (rho^-1/2, c_enc), decode (rho^1/2, c_dec).
// The projection is split over column chunks of kProjChunk and the partial
// products are summed in a fixed order (deterministic).
// Partials and their sum are float64: with d in the tens of thousands and
// heavy-tailed rows, P is a long sum whose float32 rounding, amplified by
// the cancellation between alpha X and the low-rank term, would reach the
// 1e-5 relative budget of the whitened tensor.
#include "gift_internal.hpp"

namespace gift {

// part[chunk][row][c] = sum_{j in chunk} x[row][j] * U[j][c] on the fp64
// matrix cores (v_mfma_f64_16x16x4f64): lane l supplies Aop[l % 16][l / 16]
// and Bop[l / 16][l % 16], and slot e of lane l holds D[4 e + l / 16][l % 16].
// A wave owns 32 rows x 32 columns of one chunk (2 x 2 output tiles).  In
// each 32-column step, lane l loads 8 consecutive values of its row starting
// at 8 (l / 16) (two 16-byte loads, 128 contiguous bytes per 4 lanes), and
// k-step s pairs x[row][j + 8 k + s] with U[j + 8 k + s][c] for k = l / 16:
// a permutation of the contraction index, applied to both operands.  The
// fp32 inputs are exact in fp64, so every product is exact and only the
// fp64 accumulation rounds.  x is read from memory once; U (d x 32 fp32)
// from L2.
typedef double pdouble4 __attribute__((ext_vector_type(4)));
constexpr int kProjRowsWave = 32;

__global__ void __launch_bounds__(256) k_project(const float* __restrict__ x, int64_t ldx, int m, int d,
                                                 const float* __restrict__ U, double* __restrict__ part) {
  constexpr int KP = 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const int row0 = ((int)blockIdx.y * 4 + wave) * kProjRowsWave;
  if (row0 >= m) return;   // whole wave; the kernel has no barrier
  const int chunk = blockIdx.x;
  const int jb = chunk * kProjChunk, je = min(d, jb + kProjChunk);
  // rows past m are clamped for the loads and not stored
  const float* xr0 = x + (int64_t)min(row0 + lr, m - 1) * ldx;
  const float* xr1 = x + (int64_t)min(row0 + 16 + lr, m - 1) * ldx;
  pdouble4 acc[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[h][c] = (pdouble4){0.0, 0.0, 0.0, 0.0};
  for (int j0 = jb; j0 < je; j0 += 32) {
    const int j = j0 + 8 * lk;   // d is a multiple of 8: all 8 in range or none
    float a0[8], a1[8], b0[8], b1[8];
    if (j < je) {
      const float4 p0 = *reinterpret_cast<const float4*>(xr0 + j);
      const float4 p1 = *reinterpret_cast<const float4*>(xr0 + j + 4);
      const float4 q0 = *reinterpret_cast<const float4*>(xr1 + j);
      const float4 q1 = *reinterpret_cast<const float4*>(xr1 + j + 4);
      a0[0] = p0.x; a0[1] = p0.y; a0[2] = p0.z; a0[3] = p0.w;
      a0[4] = p1.x; a0[5] = p1.y; a0[6] = p1.z; a0[7] = p1.w;
      a1[0] = q0.x; a1[1] = q0.y; a1[2] = q0.z; a1[3] = q0.w;
      a1[4] = q1.x; a1[5] = q1.y; a1[6] = q1.z; a1[7] = q1.w;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        b0[s] = U[(int64_t)(j + s) * KP + lr];
        b1[s] = U[(int64_t)(j + s) * KP + 16 + lr];
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) a0[s] = a1[s] = b0[s] = b1[s] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const double A0 = a0[s], A1 = a1[s], B0 = b0[s], B1 = b1[s];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(A0, B0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(A0, B1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(A1, B0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(A1, B1, acc[1][1], 0, 0, 0);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + 16 * h + 4 * e + lk;
      if (row < m) {
        double* dst = part + ((int64_t)chunk * m + row) * KP + lr;
        dst[0] = acc[h][0][e];
        dst[16] = acc[h][1][e];
      }
    }
}

hipError_t launch_lr_project(const float* x, int64_t ldx, int m, int d, const float* U, int k,
                             double* ppart, hipStream_t s) {
  (void)k;
  if (m == 0 || d == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(d, kProjChunk), (unsigned)cdiv(m, 4 * kProjRowsWave));
  hipLaunchKernelGGL(k_project, grid, dim3(256), 0, s, x, ldx, m, d, U, ppart);
  return hipGetLastError();
}

// pc[i][t] = fp32(c_t * sum_chunk part[chunk][i][t]): the projection
// partials summed once, in chunk order, in float64 (then scaled by c and
// rounded once).
__global__ void __launch_bounds__(256) k_lr_reduce(const double* __restrict__ part, int nchunk, int m,
                                                   const float* __restrict__ coef, int which,
                                                   float* __restrict__ pc) {
  constexpr int KP = 32;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)m * KP) return;
  const float* c = coef + (which == 0 ? 0 : KP);
  double acc = 0.0;
  for (int ch = 0; ch < nchunk; ++ch) acc += part[(int64_t)ch * m * KP + i];
  pc[i] = (float)(acc * (double)c[i % KP]);
}

// out[i][j] = alpha x[i][j] + sum_t pc[i][t] U[j][t]
// Tile: 128 rows x 256 columns (U's 256 rows staged once, transposed, in
// LDS), walked 16 rows at a time; wave w owns rows 4w..4w+3 of each step,
// lane l columns 4l..4l+3.  The next step's x is loaded while this step's
// products run.  Optionally the amax of |out| per 128 x 128 tile (or
// tensor): a tile covers whole amax blocks.
constexpr int kApplyRows = 128;
static_assert(kApplyRows == kBlock, "an apply tile covers one row of amax blocks");

__global__ void __launch_bounds__(256) k_lr_apply(const float* __restrict__ x, int64_t ldx, int m, int d,
                                                  const float* __restrict__ U, const float* __restrict__ pc,
                                                  const float* __restrict__ coef, int which,
                                                  float* __restrict__ out, int64_t ldo, int scaling,
                                                  uint32_t* __restrict__ slots) {
  constexpr int KP = 32, STEPS = kApplyRows / 16;
  __shared__ float UsT[KP][256 + 4];
  __shared__ float Pc[kApplyRows][KP + 4];
  __shared__ uint32_t red[4][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col0 = blockIdx.x * 256;
  const int row0 = blockIdx.y * kApplyRows;
  const float alpha = coef[2 * KP + which];
  const int col = col0 + lane * 4;
  const bool colok = col < d;   // d is a multiple of 8: all 4 columns or none
  auto load_x = [&](int step, float4* xv) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = row0 + 16 * step + wave * 4 + rr;
      xv[rr] = (colok && row < m) ? *reinterpret_cast<const float4*>(x + (int64_t)row * ldx + col)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float4 xcur[4], xnxt[4];
  load_x(0, xcur);
  // U rows of this column tile, transposed into LDS; the row block's pc.
  for (int i = tid; i < 256 * KP / 4; i += 256) {
    const int j = i / (KP / 4), t = (i % (KP / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col0 + j < d) v = *reinterpret_cast<const float4*>(U + (int64_t)(col0 + j) * KP + t);
    UsT[t][j] = v.x;
    UsT[t + 1][j] = v.y;
    UsT[t + 2][j] = v.z;
    UsT[t + 3][j] = v.w;
  }
  for (int i = tid; i < kApplyRows * KP / 4; i += 256) {
    const int r = i / (KP / 4), t = (i % (KP / 4)) * 4;
    *reinterpret_cast<float4*>(&Pc[r][t]) = row0 + r < m ? *reinterpret_cast<const float4*>(pc + (int64_t)(row0 + r) * KP + t)
                                                         : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  uint32_t mx = 0;
  for (int step = 0; step < STEPS; ++step) {
    if (row0 + 16 * step >= m) break;   // uniform over the workgroup
    if (step + 1 < STEPS) load_x(step + 1, xnxt);
    float acc[4][4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[rr][q] = 0.f;
    const int rb = 16 * step + wave * 4;
#pragma unroll 2
    for (int t = 0; t < KP; t += 4) {
      float4 u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = *reinterpret_cast<const float4*>(&UsT[t + q][lane * 4]);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 p = *reinterpret_cast<const float4*>(&Pc[rb + rr][t]);
        const float pv[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[rr][0] += pv[q] * u[q].x;
          acc[rr][1] += pv[q] * u[q].y;
          acc[rr][2] += pv[q] * u[q].z;
          acc[rr][3] += pv[q] * u[q].w;
        }
      }
    }
    if (colok) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = row0 + rb + rr;
        if (row < m) {
          const float4 v = xcur[rr];
          const float4 o = make_float4(alpha * v.x + acc[rr][0], alpha * v.y + acc[rr][1],
                                       alpha * v.z + acc[rr][2], alpha * v.w + acc[rr][3]);
          *reinterpret_cast<float4*>(out + (int64_t)row * ldo + col) = o;
          uint32_t a = __float_as_uint(o.x) & 0x7FFFFFFFu, b = __float_as_uint(o.y) & 0x7FFFFFFFu;
          uint32_t e = __float_as_uint(o.z) & 0x7FFFFFFFu, f = __float_as_uint(o.w) & 0x7FFFFFFFu;
          a = a > b ? a : b;
          e = e > f ? e : f;
          a = a > e ? a : e;
          mx = mx > a ? mx : a;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) xcur[rr] = xnxt[rr];
  }
  if (slots) {
    for (int o = 16; o > 0; o >>= 1) {
      uint32_t v = (uint32_t)__shfl_xor((int)mx, o, 64);
      mx = mx > v ? mx : v;
    }
    if ((lane & 31) == 0) red[wave][lane >> 5] = mx;
    __syncthreads();
    if (tid < 2) {
      uint32_t v = red[0][tid];
      for (int w = 1; w < 4; ++w) v = v > red[w][tid] ? v : red[w][tid];
      int cb = col0 + tid * 128;
      if (cb < d && v) {
        int slot = scaling == 0 ? 0 : (row0 / kBlock) * (int)cdiv(d, kBlock) + cb / kBlock;
        atomicMax(slots + slot, v);
      }
    }
  }
}

hipError_t launch_lr_apply(const float* x, int64_t ldx, int m, int d, const float* U, int k,
                           const double* ppart, float* pc, const float* coef, int which, float* out,
                           int64_t ldo, int scaling, uint32_t* amax_slots, hipStream_t s) {
  (void)k;
  if (m == 0 || d == 0) return hipSuccess;
  const int nchunk = (int)cdiv(d, kProjChunk);
  hipLaunchKernelGGL(k_lr_reduce, dim3((unsigned)cdiv((int64_t)m * 32, 256)), dim3(256), 0, s, ppart, nchunk, m,
                     coef, which, pc);
  dim3 grid((unsigned)cdiv(d, 256), (unsigned)cdiv(m, kApplyRows));
  hipLaunchKernelGGL(k_lr_apply, grid, dim3(256), 0, s, x, ldx, m, d, U, pc, coef, which, out, ldo, scaling,
                     amax_slots);
  return hipGetLastError();
}

// out[i][j] = x[i][j] * v[j], with the optional amax of |out|.
__global__ void __launch_bounds__(256) k_diag_apply(const float* __restrict__ x, int64_t ldx, int m, int d,
                                                    const float* __restrict__ v, float* __restrict__ out,
                                                    int64_t ldo, int scaling, uint32_t* __restrict__ slots) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * 256 + lane * 4;
  const int r0 = blockIdx.y * kBlock;
  const int r1 = min(m, r0 + kBlock);
  uint32_t mx = 0;
  if (col < d) {
    float4 s = *reinterpret_cast<const float4*>(v + col);
    for (int r = r0 + wave; r < r1; r += 4) {
      float4 a = *reinterpret_cast<const float4*>(x + (int64_t)r * ldx + col);
      float4 o = make_float4(a.x * s.x, a.y * s.y, a.z * s.z, a.w * s.w);
      *reinterpret_cast<float4*>(out + (int64_t)r * ldo + col) = o;
      uint32_t b0 = __float_as_uint(o.x) & 0x7FFFFFFFu, b1 = __float_as_uint(o.y) & 0x7FFFFFFFu;
      uint32_t b2 = __float_as_uint(o.z) & 0x7FFFFFFFu, b3 = __float_as_uint(o.w) & 0x7FFFFFFFu;
      b0 = b0 > b1 ? b0 : b1;
      b2 = b2 > b3 ? b2 : b3;
      b0 = b0 > b2 ? b0 : b2;
      mx = mx > b0 ? mx : b0;
    }
  }
  if (!slots) return;
  for (int o = 16; o > 0; o >>= 1) {
    uint32_t t = (uint32_t)__shfl_xor((int)mx, o, 64);
    mx = mx > t ? mx : t;
  }
  __shared__ uint32_t red[4][2];
  if ((lane & 31) == 0) red[wave][lane >> 5] = mx;
  __syncthreads();
  if (threadIdx.x < 2) {
    uint32_t t = red[0][threadIdx.x];
    for (int w = 1; w < 4; ++w) t = t > red[w][threadIdx.x] ? t : red[w][threadIdx.x];
    int cb = blockIdx.x * 256 + threadIdx.x * 128;
    if (cb < d && t) {
      int slot = scaling == 0 ? 0 : blockIdx.y * (int)cdiv(d, kBlock) + cb / kBlock;
      atomicMax(slots + slot, t);
    }
  }
}

hipError_t launch_diag_apply(const float* x, int64_t ldx, int m, int d, const float* v, float* out,
                             int64_t ldo, int scaling, uint32_t* amax_slots, hipStream_t s) {
  if (m == 0 || d == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(d, 256), (unsigned)cdiv(m, kBlock));
  hipLaunchKernelGGL(k_diag_apply, grid, dim3(256), 0, s, x, ldx, m, d, v, out, ldo, scaling, amax_slots);
  return hipGetLastError();
}

}  // namespace gift
