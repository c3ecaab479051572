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
// Tiling: quantiser, one lane per 16-element block (four float4 loads, the
// scale arithmetic once per block); dequant-sum, 32 codes per lane (two
// blocks, one 16-byte load per replica).  Consecutive lanes take
// consecutive blocks (or code runs) of a row, so a wave's accesses cover
// one contiguous range.
#include "fp8_codec.hpp"
#include "gift_internal.hpp"

namespace gift {

// One lane per 16-element block: four 16-byte loads, the block amax in
// registers, the scale arithmetic once per block, one 8-byte code store and
// one scale byte (consecutive lanes take consecutive blocks of a row).
template <bool EF>
__global__ void __launch_bounds__(256) k_quantize_fp4(const float* __restrict__ x, int64_t ld, int m, int d,
                                                      const uint32_t* __restrict__ slot,
                                                      const float* __restrict__ amax_in, float* __restrict__ amax_out,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales,
                                                      float* __restrict__ tscale, float* __restrict__ resid,
                                                      uint32_t* __restrict__ flags) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;   // block index, row-major
  const int bpr = d / kFp4Block;
  const int64_t nb = (int64_t)m * bpr;
  const uint32_t am_t = amax_in ? (__float_as_uint(amax_in[0]) & 0x7FFFFFFFu) : slot[0];
  const float g = fp4_tscale(am_t);
  if (b == 0) {
    tscale[0] = g;
    if (amax_out) amax_out[0] = __uint_as_float(slot[0]);
    if (am_t >= 0x7F800000u) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);
  }
  if (b >= nb) return;
  const int row = (int)(b / bpr), col = (int)(b % bpr) * kFp4Block;
  float v[16];
  const float* src = x + (int64_t)row * ld + col;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 q = *reinterpret_cast<const float4*>(src + 4 * k);
    v[4 * k] = q.x;
    v[4 * k + 1] = q.y;
    v[4 * k + 2] = q.z;
    v[4 * k + 3] = q.w;
  }
  float* rp = resid + (int64_t)row * d + col;
  if constexpr (EF) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 e = *reinterpret_cast<const float4*>(rp + 4 * k);
      v[4 * k] += e.x;
      v[4 * k + 1] += e.y;
      v[4 * k + 2] += e.z;
      v[4 * k + 3] += e.w;
    }
  }
  // block amax (|x| bit patterns order like |x|, NaN on top)
  uint32_t mx = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) mx = max(mx, __float_as_uint(v[k]) & 0x7FFFFFFFu);
  float sig;
  if (g != g) sig = __uint_as_float(0x7FC00000u);
  else if (g == 0.0f) sig = 0.0f;
  else sig = (float)((double)__uint_as_float(mx) / (6.0 * (double)g));
  const uint32_t sc = enc_e4m3(sig);
  const float S = dec_e4m3(sc) * g;
  const bool bad = S != S;
  const float r = S > 0.0f ? (float)(1.0 / (double)S) : 0.0f;
  uint32_t c[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) c[k] = bad ? 0u : enc_e2m1(v[k] * r);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    w0 |= c[k] << (4 * k);
    w1 |= c[8 + k] << (4 * k);
  }
  *reinterpret_cast<uint2*>(codes + (int64_t)row * (d >> 1) + (col >> 1)) = make_uint2(w0, w1);
  bscales[b] = (uint8_t)sc;
  if (bad && g == g) atomicOr(flags, (uint32_t)GIFT_FLAG_NONFINITE);   // a NaN block under a finite tensor scale
  if constexpr (EF) {
    // new residual fp32(u - S dec(q)), the difference rounded once
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<float4*>(rp + 4 * k) =
          make_float4(__builtin_fmaf(-S, dec_e2m1(c[4 * k]), v[4 * k]),
                      __builtin_fmaf(-S, dec_e2m1(c[4 * k + 1]), v[4 * k + 1]),
                      __builtin_fmaf(-S, dec_e2m1(c[4 * k + 2]), v[4 * k + 2]),
                      __builtin_fmaf(-S, dec_e2m1(c[4 * k + 3]), v[4 * k + 3]));
  }
}

hipError_t launch_quantize_fp4(const float* x, int64_t ld, int m, int d, const uint32_t* slot, const float* amax_in,
                               float* amax_out, uint8_t* codes, uint8_t* bscales, float* tscale, float* resid,
                               uint32_t* flags, hipStream_t s) {
  const int64_t nb = (int64_t)m * (d / kFp4Block);
  const unsigned blocks = (unsigned)cdiv(nb > 0 ? nb : 1, 256);   // one thread at least: it writes the tensor scale
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
// A lane owns V consecutive codes of a row (V = 32: one 16-byte load per
// replica, or 16 with 8-byte loads when code rows are not 16-byte
// aligned); a wave walks the rows of a 32-row band with four replicas'
// loads in flight.  Codes are decoded a byte (two codes) at a time by the
// hardware E2M1 conversion with a unit scale, which is exact.
constexpr int kDq4Rows = 32;
typedef float fp4_float2 __attribute__((ext_vector_type(2)));

template <int V>
struct Fp4Vec {
  uint32_t w[V / 8];
  uint32_t sc[V / 16];   // E4M3 block scale bytes
};

template <int V>
__device__ __forceinline__ Fp4Vec<V> load_fp4(const uint8_t* cp, const uint8_t* sp) {
  Fp4Vec<V> c;
  if constexpr (V == 32) {
    const uint4 q = *reinterpret_cast<const uint4*>(cp);
    c.w[0] = q.x;
    c.w[1] = q.y;
    c.w[2] = q.z;
    c.w[3] = q.w;
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(cp);
    c.w[0] = q.x;
    c.w[1] = q.y;
  }
#pragma unroll
  for (int b = 0; b < V / 16; ++b) c.sc[b] = sp[b];
  return c;
}

// a[j] (+)= S_b dec(q_j) for the V codes of one replica; FIRST: replica 0.
template <int V, bool FIRST>
__device__ __forceinline__ void acc_fp4(const Fp4Vec<V>& c, float tscale, float* a) {
#pragma unroll
  for (int b = 0; b < V / 16; ++b) {
    const float S = dec_e4m3(c.sc[b]) * tscale;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t w = c.w[2 * b + k];
      const fp4_float2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0),
                               __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1),
                               __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2),
                               __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3)};
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        const int j = 16 * b + 8 * k + 2 * by;
        if constexpr (FIRST) {
          a[j] = S * v[by][0];
          a[j + 1] = S * v[by][1];
        } else {
          a[j] = __builtin_fmaf(S, v[by][0], a[j]);
          a[j + 1] = __builtin_fmaf(S, v[by][1], a[j + 1]);
        }
      }
    }
  }
}

template <int V>
__global__ void __launch_bounds__(256) k_dequant_sum_fp4(const uint8_t* __restrict__ codes, int64_t code_stride,
                                                         const uint8_t* __restrict__ bscales, int64_t bscale_stride,
                                                         const float* __restrict__ tscales, int R, int m, int d,
                                                         float* __restrict__ out, int64_t ldo, float invR) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * (64 * V) + lane * V;
  const int r0 = blockIdx.y * kDq4Rows;
  const int r1 = min(m, r0 + kDq4Rows);
  if (col >= d) return;   // d is a multiple of V: a lane's codes are all in range
  for (int row = r0 + wave; row < r1; row += 4) {
    const uint8_t* cp = codes + (int64_t)row * (d >> 1) + (col >> 1);
    const uint8_t* sp = bscales + (int64_t)row * (d / kFp4Block) + col / kFp4Block;
    float a[V];
    acc_fp4<V, true>(load_fp4<V>(cp, sp), tscales[0], a);
    int r = 1;
    for (; r + 4 <= R; r += 4) {
      Fp4Vec<V> c[4];
      float t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        t[u] = tscales[r + u];
        c[u] = load_fp4<V>(cp + (int64_t)(r + u) * code_stride, sp + (int64_t)(r + u) * bscale_stride);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc_fp4<V, false>(c[u], t[u], a);
    }
    for (; r < R; ++r)
      acc_fp4<V, false>(load_fp4<V>(cp + (int64_t)r * code_stride, sp + (int64_t)r * bscale_stride), tscales[r], a);
    float* o = out + (int64_t)row * ldo + col;
#pragma unroll
    for (int k = 0; k < V / 4; ++k)
      *reinterpret_cast<float4*>(o + 4 * k) =
          make_float4(a[4 * k] * invR, a[4 * k + 1] * invR, a[4 * k + 2] * invR, a[4 * k + 3] * invR);
  }
}

// The same with a compile-time replica count RC: the RC replicas' codes and
// scale bytes of a row are all in flight together (not replica 0 alone,
// then groups of four), and the tensor scales are read once per band.  The
// sums are formed in the same order, so the results are identical.
template <int V, int RC>
__global__ void __launch_bounds__(256) k_dequant_sum_fp4_rc(const uint8_t* __restrict__ codes, int64_t code_stride,
                                                            const uint8_t* __restrict__ bscales, int64_t bscale_stride,
                                                            const float* __restrict__ tscales, int m, int d,
                                                            float* __restrict__ out, int64_t ldo, float invR) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * (64 * V) + lane * V;
  const int r0 = blockIdx.y * kDq4Rows;
  const int r1 = min(m, r0 + kDq4Rows);
  if (col >= d) return;   // d is a multiple of V: a lane's codes are all in range
  float ts[RC];
#pragma unroll
  for (int r = 0; r < RC; ++r) ts[r] = tscales[r];
  for (int row = r0 + wave; row < r1; row += 4) {
    const uint8_t* cp = codes + (int64_t)row * (d >> 1) + (col >> 1);
    const uint8_t* sp = bscales + (int64_t)row * (d / kFp4Block) + col / kFp4Block;
    Fp4Vec<V> c[RC];
#pragma unroll
    for (int r = 0; r < RC; ++r) c[r] = load_fp4<V>(cp + (int64_t)r * code_stride, sp + (int64_t)r * bscale_stride);
    float a[V];
    acc_fp4<V, true>(c[0], ts[0], a);
#pragma unroll
    for (int r = 1; r < RC; ++r) acc_fp4<V, false>(c[r], ts[r], a);
    float* o = out + (int64_t)row * ldo + col;
#pragma unroll
    for (int k = 0; k < V / 4; ++k)
      *reinterpret_cast<float4*>(o + 4 * k) =
          make_float4(a[4 * k] * invR, a[4 * k + 1] * invR, a[4 * k + 2] * invR, a[4 * k + 3] * invR);
  }
}

template <int V>
static void launch_dq4(const uint8_t* codes, int64_t code_stride, const uint8_t* bscales, int64_t bscale_stride,
                       const float* tscales, int R, int m, int d, float* out, int64_t ldo, float invR,
                       hipStream_t s) {
  dim3 grid((unsigned)cdiv(d, 64 * V), (unsigned)cdiv(m, kDq4Rows));
  switch (R) {
    case 4:
      hipLaunchKernelGGL((k_dequant_sum_fp4_rc<V, 4>), grid, dim3(256), 0, s, codes, code_stride, bscales,
                         bscale_stride, tscales, m, d, out, ldo, invR);
      break;
    case 8:
      hipLaunchKernelGGL((k_dequant_sum_fp4_rc<V, 8>), grid, dim3(256), 0, s, codes, code_stride, bscales,
                         bscale_stride, tscales, m, d, out, ldo, invR);
      break;
    case 16:
      hipLaunchKernelGGL((k_dequant_sum_fp4_rc<V, 16>), grid, dim3(256), 0, s, codes, code_stride, bscales,
                         bscale_stride, tscales, m, d, out, ldo, invR);
      break;
    default:
      hipLaunchKernelGGL(k_dequant_sum_fp4<V>, grid, dim3(256), 0, s, codes, code_stride, bscales, bscale_stride,
                         tscales, R, m, d, out, ldo, invR);
  }
}

hipError_t launch_dequant_sum_fp4(const uint8_t* codes, int64_t code_stride, const uint8_t* bscales,
                                  int64_t bscale_stride, const float* tscales, int R, int m, int d, float* out,
                                  int64_t ldo, hipStream_t s) {
  if (m == 0 || d == 0) return hipSuccess;
  if (d % 16 != 0) return hipErrorInvalidValue;
  const float invR = 1.0f / (float)R;
  // 16-byte loads need 16-byte aligned code rows in every replica
  const bool v32 = d % 32 == 0 && (reinterpret_cast<uintptr_t>(codes) & 15u) == 0 && (R == 1 || code_stride % 16 == 0);
  if (v32)
    launch_dq4<32>(codes, code_stride, bscales, bscale_stride, tscales, R, m, d, out, ldo, invR, s);
  else
    launch_dq4<16>(codes, code_stride, bscales, bscale_stride, tscales, R, m, d, out, ldo, invR, s);
  return hipGetLastError();
}

}  // namespace gift
