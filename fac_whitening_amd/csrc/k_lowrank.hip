// Low-rank input-side transform (whiten / map back) and column scaling.
//
// GIFT 阅读笔记, §简化一 Eq. (16): W~ = W T_A; §简化二 Eq. (17): A ~ U Lam U^T
// with r = 32; Algorithm 1: U = W (L_A)^-T before, W^ = U L_A^T after the
// collective.  With the rank-k form T = U diag(c) U^T + alpha I the product
// is never formed densely:
//     P = X U            (m x k, a skinny contraction over d)
//     out = alpha X + (P diag(c)) U^T
// Encode uses (alpha, c) = (rho^-1/2, c_enc), decode (rho^1/2, c_dec).
// The projection is split over column chunks of 256 and the partial
// products are summed in a fixed order by the consumer (deterministic).
// Partials and their sum are float64: with d in the tens of thousands and
// heavy-tailed rows, P is a long sum whose float32 rounding, amplified by
// the cancellation between alpha X and the low-rank term, would reach the
// 1e-5 relative budget of the whitened tensor.
#include "gift_internal.hpp"

namespace gift {

// part[chunk][row][c] = sum_{j in chunk} x[row][j] * U[j][c]
//   KP: padded columns of U; CG: column groups per row (CW = KP / CG columns
//   per thread); RB = 256 / CG rows per workgroup; KC: chunk length.
//   FULLK: one workgroup walks every chunk of its rows and writes the whole
//   sum (part has a single chunk); otherwise one chunk per workgroup.
template <int KP, int CG, int KC, bool FULLK, typename TU, typename TO>
__global__ void __launch_bounds__(256) k_project(const float* __restrict__ x, int64_t ldx, int m, int d,
                                                 const TU* __restrict__ U, TO* __restrict__ part) {
  constexpr int CW = KP / CG;
  constexpr int RB = 256 / CG;
  __shared__ TU Us[KC][KP];
  __shared__ float Xs[RB][KC + 1];
  const int tid = threadIdx.x;
  const int row0 = blockIdx.y * RB;
  const int r = tid / CG, cg = tid % CG;
  TO acc[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) acc[c] = TO(0);
  const int c_begin = FULLK ? 0 : (int)blockIdx.x;
  const int c_end = FULLK ? (int)cdiv(d, KC) : (int)blockIdx.x + 1;
  for (int chunk = c_begin; chunk < c_end; ++chunk) {
    const int j0 = chunk * KC;
    if (FULLK) __syncthreads();
    for (int i = tid; i < KC * KP; i += 256) {
      int j = i / KP, c = i % KP;
      Us[j][c] = (j0 + j < d) ? U[(int64_t)(j0 + j) * KP + c] : TU(0);
    }
    for (int i = tid; i < RB * KC / 4; i += 256) {
      int rr = i / (KC / 4), j = (i % (KC / 4)) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row0 + rr < m && j0 + j < d) v = *reinterpret_cast<const float4*>(x + (int64_t)(row0 + rr) * ldx + j0 + j);
      Xs[rr][j] = v.x;
      Xs[rr][j + 1] = v.y;
      Xs[rr][j + 2] = v.z;
      Xs[rr][j + 3] = v.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int j = 0; j < KC; ++j) {
      TO xv = (TO)Xs[r][j];
#pragma unroll
      for (int c = 0; c < CW; ++c) acc[c] += xv * (TO)Us[j][cg * CW + c];
    }
  }
  if (row0 + r < m) {
    const int slot = FULLK ? 0 : (int)blockIdx.x;
    TO* dst = part + ((int64_t)slot * m + row0 + r) * KP + cg * CW;
#pragma unroll
    for (int c = 0; c < CW; ++c) dst[c] = acc[c];
  }
}

hipError_t launch_lr_project(const float* x, int64_t ldx, int m, int d, const float* U, int k,
                             double* ppart, hipStream_t s) {
  (void)k;
  if (m == 0 || d == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(d, kProjChunk), (unsigned)cdiv(m, 32));
  hipLaunchKernelGGL((k_project<32, 8, kProjChunk, false, float, double>), grid, dim3(256), 0, s, x, ldx, m, d, U,
                     ppart);
  return hipGetLastError();
}

// out[i][j] = alpha x[i][j] + sum_t (c_t sum_chunk part[chunk][i][t]) U[j][t]
// Tile: 16 rows x 256 columns; wave w owns rows 4w..4w+3, lane l columns
// 4l..4l+3.  Optionally the amax of |out| per 128 x 128 tile (or tensor).
__global__ void __launch_bounds__(256) k_lr_apply(const float* __restrict__ x, int64_t ldx, int m, int d,
                                                  const float* __restrict__ U, const double* __restrict__ part,
                                                  int nchunk, const float* __restrict__ coef, int which,
                                                  float* __restrict__ out, int64_t ldo, int scaling,
                                                  uint32_t* __restrict__ slots) {
  constexpr int KP = 32;
  __shared__ float UsT[KP][256 + 4];
  __shared__ float Pc[16][KP];
  __shared__ uint32_t red[4][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col0 = blockIdx.x * 256;
  const int row0 = blockIdx.y * 16;
  const float* c = coef + (which == 0 ? 0 : KP);
  const float alpha = coef[2 * KP + which];
  // U rows of this column tile, transposed into LDS.
  for (int i = tid; i < 256 * KP / 4; i += 256) {
    int j = i / (KP / 4), t = (i % (KP / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col0 + j < d) v = *reinterpret_cast<const float4*>(U + (int64_t)(col0 + j) * KP + t);
    UsT[t][j] = v.x;
    UsT[t + 1][j] = v.y;
    UsT[t + 2][j] = v.z;
    UsT[t + 3][j] = v.w;
  }
  // Reduce the projection partials of these 16 rows (fixed chunk order).
  for (int i = tid; i < 16 * KP; i += 256) {
    int r = i / KP, t = i % KP;
    double acc = 0.0;
    if (row0 + r < m)
      for (int ch = 0; ch < nchunk; ++ch) acc += part[((int64_t)ch * m + row0 + r) * KP + t];
    Pc[r][t] = (float)(acc * (double)c[t]);
  }
  __syncthreads();
  const int col = col0 + lane * 4;
  float acc[4][4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[rr][q] = 0.f;
#pragma unroll 8
  for (int t = 0; t < KP; ++t) {
    float4 u = *reinterpret_cast<const float4*>(&UsT[t][lane * 4]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float p = Pc[wave * 4 + rr][t];
      acc[rr][0] += p * u.x;
      acc[rr][1] += p * u.y;
      acc[rr][2] += p * u.z;
      acc[rr][3] += p * u.w;
    }
  }
  uint32_t mx = 0;
  if (col < d) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      int row = row0 + wave * 4 + rr;
      if (row < m) {
        float4 v = *reinterpret_cast<const float4*>(x + (int64_t)row * ldx + col);
        float4 o = make_float4(alpha * v.x + acc[rr][0], alpha * v.y + acc[rr][1], alpha * v.z + acc[rr][2],
                               alpha * v.w + acc[rr][3]);
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
                           const double* ppart, const float* coef, int which, float* out,
                           int64_t ldo, int scaling, uint32_t* amax_slots, hipStream_t s) {
  (void)k;
  if (m == 0 || d == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(d, 256), (unsigned)cdiv(m, 16));
  int nchunk = (int)cdiv(d, kProjChunk);
  hipLaunchKernelGGL(k_lr_apply, grid, dim3(256), 0, s, x, ldx, m, d, U, ppart, nchunk, coef, which, out, ldo,
                     scaling, amax_slots);
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
