// FP4 payload: E2M1 elements in 16-element row blocks, each with an E4M3
// scale, under one fp32 scale per tensor (byte-bound passes).
//
// The pages name NVFP4 as a communication format (GIFT abstract; GIFT 阅读笔记,
// summary: the coordinate change is forward compatible with FP4) and leave
// the layout open.  Layout and arithmetic implemented here:
//   g     = fp32(amax_T / (6 * 448))   per tensor (amax_T local or shared)
//   sig_b = fp32(amax_b / (6 g)),  sc_b = E4M3(sig_b) (RNE, saturating)
//   S_b   = fp32(dec(sc_b) g),  r_b = fp32(1 / S_b) (0 when S_b = 0)
//   q     = E2M1(fp32(x r_b))  (RNE, ties to the even code, saturating at 6)
//   value = S_b dec(q)
// A NaN tensor amax gives g = NaN: every block scale 0x7F, codes 0.  A block
// whose scale is NaN gets codes 0.  Quotients are double divisions of float
// values rounded once (the correctly rounded float quotient).
//
// E2M1 (OCP 4-bit float): sign, 2 exponent bits (bias 1), 1 mantissa bit;
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no Inf or NaN.  Two codes per byte,
// the even column in the low nibble.
//
// Tiling: quantiser, 4 lanes per block (one float4 each, a quad reduces the
// block amax with two shuffles); dequant-sum, 2 lanes per block (8 codes,
// one 32-bit load per replica).  Consecutive lanes take consecutive columns
// of a row, so every load and store of a wave is contiguous.
#include "fp8_codec.hpp"
#include "gift_internal.hpp"

namespace gift {

constexpr int kFp4Block = 16;
constexpr double kFp4TscaleDiv = 6.0 * 448.0;

// E2M1 code of y: the magnitude is the number of decision points below |y|,
// with the midpoints 0.25, 1.25, 2.5, 5 going down (to the even codes 0, 2,
// 4, 6) and 0.75, 1.75, 3.5 going up (to 2, 4, 6).  +-Inf saturates to 7;
// NaN gives +0.
__device__ __forceinline__ uint32_t enc_e2m1(float y) {
  const float a = __builtin_fabsf(y);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  const uint32_t sign = (a == a) ? (__float_as_uint(y) >> 28) & 0x8u : 0u;
  return c | sign;
}

// Value of an E2M1 code: magnitudes 0 and 1 are 0 and 0.5; k >= 2 is
// (1 + (k & 1) / 2) 2^((k >> 1) - 1), built as a float bit pattern.
__device__ __forceinline__ float dec_e2m1(uint32_t c) {
  const uint32_t k = c & 7u;
  const float v = k < 2u ? 0.5f * (float)k : __uint_as_float((((k >> 1) + 126u) << 23) | ((k & 1u) << 22));
  return __uint_as_float(__float_as_uint(v) | ((c & 8u) << 28));
}

// g from the tensor amax (bit pattern of |x|): NaN for a non-finite amax.
__device__ __forceinline__ float fp4_tscale(uint32_t am) {
  if (am >= 0x7F800000u) return __uint_as_float(0x7FC00000u);
  if (am == 0u) return 0.0f;
  return (float)((double)__uint_as_float(am) / kFp4TscaleDiv);
}

template <bool EF>
__global__ void __launch_bounds__(256) k_quantize_fp4(const float* __restrict__ x, int64_t ld, int m, int d,
                                                      const uint32_t* __restrict__ slot,
                                                      const float* __restrict__ amax_in, float* __restrict__ amax_out,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales,
                                                      float* __restrict__ tscale, float* __restrict__ resid,
                                                      uint32_t* __restrict__ flags) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q4 = d >> 2;                                   // float4 groups per row
  const int64_t n4 = (int64_t)m * q4;
  const bool in = t < n4;                                  // n4 is a multiple of 4: quads are all in or all out
  const int row = in ? (int)(t / q4) : 0;
  const int col = in ? (int)(t % q4) * 4 : 0;
  const uint32_t am_t = amax_in ? (__float_as_uint(amax_in[0]) & 0x7FFFFFFFu) : slot[0];
  const float g = fp4_tscale(am_t);
  if (t == 0) {
    tscale[0] = g;
    if (amax_out) amax_out[0] = __uint_as_float(slot[0]);
    if (am_t >= 0x7F800000u) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (in) {
    v = *reinterpret_cast<const float4*>(x + (int64_t)row * ld + col);
    if constexpr (EF) {
      const float4 e = *reinterpret_cast<const float4*>(resid + (int64_t)row * d + col);
      v.x += e.x;
      v.y += e.y;
      v.z += e.z;
      v.w += e.w;
    }
  }
  // block amax over the quad (|x| bit patterns order like |x|, NaN on top)
  auto ab = [](float f) { return __float_as_uint(f) & 0x7FFFFFFFu; };
  uint32_t mx = max(max(ab(v.x), ab(v.y)), max(ab(v.z), ab(v.w)));
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, 64));
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, 64));
  if (!in) return;
  float sig;
  if (g != g) sig = __uint_as_float(0x7FC00000u);
  else if (g == 0.0f) sig = 0.0f;
  else sig = (float)((double)__uint_as_float(mx) / (6.0 * (double)g));
  const uint32_t sc = enc_e4m3(sig);
  const float S = dec_e4m3(sc) * g;
  const bool bad = S != S;
  const float r = S > 0.0f ? (float)(1.0 / (double)S) : 0.0f;
  uint32_t c0 = enc_e2m1(v.x * r), c1 = enc_e2m1(v.y * r), c2 = enc_e2m1(v.z * r), c3 = enc_e2m1(v.w * r);
  if (bad) c0 = c1 = c2 = c3 = 0u;
  *reinterpret_cast<uint16_t*>(codes + (int64_t)row * (d >> 1) + (col >> 1)) =
      (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
  if ((col & (kFp4Block - 1)) == 0) {
    bscales[(int64_t)row * (d / kFp4Block) + col / kFp4Block] = (uint8_t)sc;
    if (bad && g == g) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);   // a NaN block under a finite tensor scale
  }
  if constexpr (EF) {
    // new residual fp32(u - S dec(q)), the difference rounded once
    const float4 e = make_float4(__builtin_fmaf(-S, dec_e2m1(c0), v.x), __builtin_fmaf(-S, dec_e2m1(c1), v.y),
                                 __builtin_fmaf(-S, dec_e2m1(c2), v.z), __builtin_fmaf(-S, dec_e2m1(c3), v.w));
    *reinterpret_cast<float4*>(resid + (int64_t)row * d + col) = e;
  }
}

hipError_t launch_quantize_fp4(const float* x, int64_t ld, int m, int d, const uint32_t* slot, const float* amax_in,
                               float* amax_out, uint8_t* codes, uint8_t* bscales, float* tscale, float* resid,
                               uint32_t* flags, hipStream_t s) {
  const int64_t n4 = (int64_t)m * (d / 4);
  const unsigned blocks = (unsigned)cdiv(n4 > 0 ? n4 : 1, 256);   // one thread at least: it writes the tensor scale
  if (resid)
    hipLaunchKernelGGL(k_quantize_fp4<true>, dim3(blocks), dim3(256), 0, s, x, ld, m, d, slot, amax_in, amax_out,
                       codes, bscales, tscale, resid, flags);
  else
    hipLaunchKernelGGL(k_quantize_fp4<false>, dim3(blocks), dim3(256), 0, s, x, ld, m, d, slot, amax_in, amax_out,
                       codes, bscales, tscale, resid, flags);
  return hipGetLastError();
}

// U = (1/R) sum_r S_{b,r} dec(q_r), replicas in increasing r (the sum
// starts from replica 0's term, so a lone -0 stays -0).
__global__ void __launch_bounds__(256) k_dequant_sum_fp4(const uint8_t* __restrict__ codes, int64_t code_stride,
                                                         const uint8_t* __restrict__ bscales, int64_t bscale_stride,
                                                         const float* __restrict__ tscales, int R, int m, int d,
                                                         float* __restrict__ out, int64_t ldo, float invR) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q8 = d >> 3;
  if (t >= (int64_t)m * q8) return;
  const int row = (int)(t / q8), col = (int)(t % q8) * 8;
  const int64_t co = (int64_t)row * (d >> 1) + (col >> 1);
  const int64_t so = (int64_t)row * (d / kFp4Block) + col / kFp4Block;
  float acc[8];
  for (int r = 0; r < R; ++r) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + (int64_t)r * code_stride + co);
    const float S = dec_e4m3(bscales[(int64_t)r * bscale_stride + so]) * tscales[r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = dec_e2m1((w >> (4 * j)) & 0xFu);
      acc[j] = r == 0 ? S * v : __builtin_fmaf(S, v, acc[j]);
    }
  }
  float* o = out + (int64_t)row * ldo + col;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0] * invR, acc[1] * invR, acc[2] * invR, acc[3] * invR);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4] * invR, acc[5] * invR, acc[6] * invR, acc[7] * invR);
}

hipError_t launch_dequant_sum_fp4(const uint8_t* codes, int64_t code_stride, const uint8_t* bscales,
                                  int64_t bscale_stride, const float* tscales, int R, int m, int d, float* out,
                                  int64_t ldo, hipStream_t s) {
  const int64_t n8 = (int64_t)m * (d / 8);
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequant_sum_fp4, dim3((unsigned)cdiv(n8, 256)), dim3(256), 0, s, codes, code_stride, bscales,
                     bscale_stride, tscales, R, m, d, out, ldo, 1.0f / (float)R);
  return hipGetLastError();
}

}  // namespace gift
