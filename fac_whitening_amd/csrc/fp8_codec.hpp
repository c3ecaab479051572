// FP8 E4M3 / E5M2 encode and decode on the device, by integer operations on
// the float32 bit pattern.
//
// Formats: GIFT 阅读笔记, §前置知识 "FP8 到底是什么" -- E4M3 (4 exponent, 3
// mantissa bits, largest 448) and E5M2 (5 / 2, largest 57344), in the OCP
// layouts (E4M3: bias 7, no Inf, 0x7F NaN; E5M2: bias 15).
// Encoding contract: round to nearest, ties to the even code; |y| >= FMAX
// (and +-Inf) saturates to +-FMAX; NaN -> 0x7F | sign; the sign bit is kept
// (so -0 and negative underflow give 0x80).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gift {

constexpr float kFmaxE4M3 = 448.0f;
constexpr float kFmaxE5M2 = 57344.0f;

__host__ __device__ inline float fp8_fmax(int fmt) { return fmt == 0 ? kFmaxE4M3 : kFmaxE5M2; }

// E4M3.  Normal range |y| >= 2^-6: round the 23-bit mantissa to 3 bits at
// bit 20 (add half minus one plus the kept LSB, then truncate); a carry out of
// the mantissa moves to the next binade by itself.  The E4M3 biased exponent
// is the fp32 one minus 120, i.e. (bits >> 20) - (120 << 3).
// Subnormal range |y| < 2^-6: code = rint(|y| * 2^9) in 0..8 (8 is the
// smallest normal, code 0x08).  The product is exact.
__device__ __forceinline__ uint32_t enc_e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;                                   // NaN
  } else if (a >= 0x43E00000u) {
    code = 0x7Eu;                                   // >= 448 (and Inf): saturate
  } else if (a >= 0x3C800000u) {
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return code | sign;
}

// E5M2.  Normal range |y| >= 2^-14: round at bit 21; biased exponent is the
// fp32 one minus 112.  Subnormal: code = rint(|y| * 2^16) in 0..4.
__device__ __forceinline__ uint32_t enc_e5m2(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;
  } else if (a >= 0x47600000u) {
    code = 0x7Bu;                                   // >= 57344 (and Inf)
  } else if (a >= 0x38800000u) {
    uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
    code = (r >> 21) - (112u << 2);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f);
  }
  return code | sign;
}

template <int FMT>
__device__ __forceinline__ uint32_t enc_fp8(float y) {
  if constexpr (FMT == 0) return enc_e4m3(y);
  else return enc_e5m2(y);
}

// Decode.  Placing the 7 magnitude bits at the top of an fp32 mantissa /
// exponent field gives 2^(e - 127) (1 + m / 2^mb) for e > 0 and the fp32
// subnormal m 2^-(149 - shift) for e = 0; one multiply by 2^(127 - bias)
// rescales both to the FP8 value exactly.  Needs fp32 denormals (the default).
__device__ __forceinline__ float dec_e4m3(uint32_t c) {
  uint32_t em = c & 0x7Fu;
  float v = __uint_as_float(((c & 0x80u) << 24) | (em << 20)) * 0x1p120f;
  return em == 0x7Fu ? __uint_as_float(0x7FC00000u) : v;
}

__device__ __forceinline__ float dec_e5m2(uint32_t c) {
  uint32_t em = c & 0x7Fu;
  float v = __uint_as_float(((c & 0x80u) << 24) | (em << 21)) * 0x1p112f;
  if (em >= 0x7Cu) {
    v = em == 0x7Cu ? __uint_as_float(((c & 0x80u) << 24) | 0x7F800000u) : __uint_as_float(0x7FC00000u);
  }
  return v;
}

template <int FMT>
__device__ __forceinline__ float dec_fp8(uint32_t c) {
  if constexpr (FMT == 0) return dec_e4m3(c);
  else return dec_e5m2(c);
}

// The four codes of a 32-bit word (byte i -> v[i]) by the hardware OCP FP8
// conversion, two at a time; the same values as dec_fp8.
typedef float fp8_float2 __attribute__((ext_vector_type(2)));
template <int FMT>
__device__ __forceinline__ void dec4_fp8(uint32_t w, float* v) {
  fp8_float2 lo, hi;
  if constexpr (FMT == 0) {
    lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  } else {
    lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  }
  v[0] = lo[0];
  v[1] = lo[1];
  v[2] = hi[0];
  v[3] = hi[1];
}

// Scale pair from an amax (as the bit pattern of |x|, ordered as uint32 so
// NaN > Inf > finite): r = fp32(FMAX / amax) (double division rounded once:
// the correctly rounded float quotient), s = fp32(amax / FMAX).
// amax = 0 -> r = s = 0.  Non-finite amax -> r = s = NaN.
__device__ __forceinline__ void scale_pair(uint32_t amax_bits, float fmax, float& r, float& s) {
  if (amax_bits >= 0x7F800000u) {
    r = __uint_as_float(0x7FC00000u);
    s = r;
  } else if (amax_bits == 0u) {
    r = 0.0f;
    s = 0.0f;
  } else {
    double am = (double)__uint_as_float(amax_bits);
    r = (float)((double)fmax / am);
    s = (float)(am / (double)fmax);
  }
}

// FP4 payload (E2M1 elements in 16-element row blocks with E4M3 block scales
// under one fp32 tensor scale: the layout is described where the FP4
// quantiser is defined).
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

}  // namespace gift
