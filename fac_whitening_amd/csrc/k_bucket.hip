// Flat gradient buckets: the Euclidean FP8 codec over many tensors in one
// launch per phase (GIFT 阅读笔记, Algorithm 1 lines 3-8: Scale,
// AllReduceMax, Q, AllReduceSum, Dequantize / N for every layer outside the
// selected set).  Scales per tensor, or per 512 consecutive elements of a
// tensor (the per-block Euclidean baseline of the experiment setup, block
// size 512; blocks restart at every tensor and a tensor's last block may be
// shorter).
//
// The tensors lie one after another in one flat fp32 buffer (element
// counts multiples of 4); codes use the same offsets, scales are numbered
// tensor by tensor.  Work is cut into chunks of 2048 elements of one tensor
// (a tensor's last chunk may be partial); wave w of a 256-thread workgroup
// takes elements 512 w .. 512 w + 511 of the chunk, lane l the float4s at
// 4 l and 256 + 4 l, so one wave covers exactly one 512-element block and a
// wave's loads are contiguous.  Workgroups loop over the chunks (grid
// stride) and find a chunk's tensor by binary search in the prefix table.
#include "fp8_codec.hpp"
#include "gift_internal.hpp"

namespace gift {

constexpr int kBChunk = 2048;

__device__ __forceinline__ int bucket_tensor(const int64_t* __restrict__ cs, int n, int64_t c) {
  int lo = 0, hi = n;   // the largest i with cs[i] <= c (cs[0] = 0, cs[n] = chunks)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cs[mid] <= c) lo = mid;
    else hi = mid;
  }
  return lo;
}

struct BChunk {
  int tensor;
  int64_t e;         // this lane's first element within the tensor
  int64_t numel;     // the tensor's element count
  int64_t base;      // the tensor's first element in the flat buffer
  int64_t slot;      // scale index of this wave's block (or of the tensor)
  bool blk_live;     // this wave's block exists
};

__device__ __forceinline__ BChunk bucket_chunk(const BucketTable& t, int64_t c, int block512) {
  BChunk b;
  const int i = bucket_tensor(t.chunk_start, t.n, c);
  const int64_t k = c - t.chunk_start[i];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  b.tensor = i;
  b.base = t.elem_off[i];
  b.numel = t.elem_off[i + 1] - b.base;
  const int64_t e0 = k * kBChunk + 512 * wave;
  b.e = e0 + 4 * lane;
  b.blk_live = e0 < b.numel;
  b.slot = t.scale_off[i] + (block512 ? 4 * k + wave : 0);
  return b;
}

__device__ __forceinline__ uint32_t absb(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }
__device__ __forceinline__ uint32_t umax4(float4 v) {
  return max(max(absb(v.x), absb(v.y)), max(absb(v.z), absb(v.w)));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// amax (as |x| bit patterns) of every scale block into slots (zeroed before).
__global__ void __launch_bounds__(256) k_bucket_amax(BucketTable t, const float* __restrict__ g, int block512,
                                                     uint32_t* __restrict__ slots) {
  __shared__ uint32_t red[4];
  for (int64_t c = blockIdx.x; c < t.chunks; c += gridDim.x) {
    const BChunk b = bucket_chunk(t, c, block512);
    const float* x = g + b.base;
    uint32_t v = 0;
    if (b.e < b.numel) v = umax4(*reinterpret_cast<const float4*>(x + b.e));
    if (b.e + 256 < b.numel) v = max(v, umax4(*reinterpret_cast<const float4*>(x + b.e + 256)));
    v = wave_umax(v);
    if (block512) {
      if ((threadIdx.x & 63) == 0 && b.blk_live) slots[b.slot] = v;   // one wave per block
    } else {
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
        if (m) atomicMax(slots + b.slot, m);
      }
      __syncthreads();   // red is rewritten by the next chunk
    }
  }
}

// Four codes of one float4 with reciprocal scale r (finite amax): the
// hardware conversion (round to nearest even) after clamping to +-FMAX;
// an element that is itself non-finite takes the integer encoder.
template <int FMT>
__device__ __forceinline__ uint32_t codes4(float4 v, float r, float fmax) {
  if (umax4(v) >= 0x7F800000u)
    return enc_fp8<FMT>(v.x * r) | (enc_fp8<FMT>(v.y * r) << 8) | (enc_fp8<FMT>(v.z * r) << 16) |
           (enc_fp8<FMT>(v.w * r) << 24);
  const float y0 = __builtin_amdgcn_fmed3f(v.x * r, fmax, -fmax), y1 = __builtin_amdgcn_fmed3f(v.y * r, fmax, -fmax);
  const float y2 = __builtin_amdgcn_fmed3f(v.z * r, fmax, -fmax), y3 = __builtin_amdgcn_fmed3f(v.w * r, fmax, -fmax);
  uint32_t q;
  if constexpr (FMT == 0) {
    q = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    q = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)q, true);
  } else {
    q = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
    q = __builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, (int)q, true);
  }
  return q;
}

template <int FMT>
__global__ void __launch_bounds__(256) k_bucket_quantize(BucketTable t, const float* __restrict__ g, int block512,
                                                         const uint32_t* __restrict__ slots,
                                                         const float* __restrict__ amax_in,
                                                         float* __restrict__ amax_out, uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const float fmax = fp8_fmax(FMT);
  for (int64_t c = blockIdx.x; c < t.chunks; c += gridDim.x) {
    const BChunk b = bucket_chunk(t, c, block512);
    if (!b.blk_live) continue;   // wave-uniform
    const uint32_t am = amax_in ? absb(amax_in[b.slot]) : slots[b.slot];
    float r, sc;
    scale_pair(am, fmax, r, sc);
    const bool bad = am >= 0x7F800000u;
    const bool writer = (threadIdx.x & 63) == 0 && (block512 || (c == t.chunk_start[b.tensor] && threadIdx.x == 0));
    if (writer) {
      scales[b.slot] = sc;
      if (amax_out) amax_out[b.slot] = __uint_as_float(slots[b.slot]);
      if (bad) atomicOr(t.flags, (uint32_t)GIFT_FLAG_NONFINITE);
    }
    const float* x = g + b.base;
    uint8_t* q = codes + b.base;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t e = b.e + 256 * h;
      if (e >= b.numel) continue;
      const float4 v = *reinterpret_cast<const float4*>(x + e);
      *reinterpret_cast<uint32_t*>(q + e) = bad ? 0x7F7F7F7Fu : codes4<FMT>(v, r, fmax);
    }
  }
}

// U = (1/R) sum_r s_r dec(q_r), replicas in increasing r (from replica 0's
// term, so a lone -0 stays -0).
template <int FMT>
__global__ void __launch_bounds__(256) k_bucket_dequant_sum(BucketTable t, const uint8_t* __restrict__ codes,
                                                            int64_t code_stride, const float* __restrict__ scales,
                                                            int64_t scale_stride, int R, int block512,
                                                            float* __restrict__ out, float invR) {
  for (int64_t c = blockIdx.x; c < t.chunks; c += gridDim.x) {
    const BChunk b = bucket_chunk(t, c, block512);
    if (!b.blk_live) continue;
    float acc[8];
    const bool live1 = b.e + 256 < b.numel;
    for (int r = 0; r < R; ++r) {
      const uint8_t* q = codes + (int64_t)r * code_stride + b.base;
      const float s = scales[(int64_t)r * scale_stride + b.slot];
      const uint32_t w0 = b.e < b.numel ? *reinterpret_cast<const uint32_t*>(q + b.e) : 0u;
      const uint32_t w1 = live1 ? *reinterpret_cast<const uint32_t*>(q + b.e + 256) : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v0 = dec_fp8<FMT>((w0 >> (8 * j)) & 0xFFu), v1 = dec_fp8<FMT>((w1 >> (8 * j)) & 0xFFu);
        acc[j] = r == 0 ? s * v0 : __builtin_fmaf(s, v0, acc[j]);
        acc[4 + j] = r == 0 ? s * v1 : __builtin_fmaf(s, v1, acc[4 + j]);
      }
    }
    float* o = out + b.base;
    if (b.e < b.numel)
      *reinterpret_cast<float4*>(o + b.e) = make_float4(acc[0] * invR, acc[1] * invR, acc[2] * invR, acc[3] * invR);
    if (live1)
      *reinterpret_cast<float4*>(o + b.e + 256) =
          make_float4(acc[4] * invR, acc[5] * invR, acc[6] * invR, acc[7] * invR);
  }
}

static unsigned bucket_grid(const BucketTable& t, int cus) {
  const int64_t want = (int64_t)(cus > 0 ? cus : 256) * 8;
  return (unsigned)(t.chunks < want ? (t.chunks > 0 ? t.chunks : 1) : want);
}

hipError_t launch_bucket_amax(const BucketTable& t, const float* g, int block512, uint32_t* slots, int cus,
                              hipStream_t s) {
  if (t.chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bucket_amax, dim3(bucket_grid(t, cus)), dim3(256), 0, s, t, g, block512, slots);
  return hipGetLastError();
}

hipError_t launch_bucket_quantize(const BucketTable& t, const float* g, int fmt, int block512, const uint32_t* slots,
                                  const float* amax_in, float* amax_out, uint8_t* codes, float* scales, int cus,
                                  hipStream_t s) {
  if (t.chunks == 0) return hipSuccess;
  if (fmt == 0)
    hipLaunchKernelGGL(k_bucket_quantize<0>, dim3(bucket_grid(t, cus)), dim3(256), 0, s, t, g, block512, slots,
                       amax_in, amax_out, codes, scales);
  else
    hipLaunchKernelGGL(k_bucket_quantize<1>, dim3(bucket_grid(t, cus)), dim3(256), 0, s, t, g, block512, slots,
                       amax_in, amax_out, codes, scales);
  return hipGetLastError();
}

hipError_t launch_bucket_dequant_sum(const BucketTable& t, const uint8_t* codes, int64_t code_stride,
                                     const float* scales, int64_t scale_stride, int R, int fmt, int block512,
                                     float* out, int cus, hipStream_t s) {
  if (t.chunks == 0) return hipSuccess;
  const float invR = 1.0f / (float)R;
  if (fmt == 0)
    hipLaunchKernelGGL(k_bucket_dequant_sum<0>, dim3(bucket_grid(t, cus)), dim3(256), 0, s, t, codes, code_stride,
                       scales, scale_stride, R, block512, out, invR);
  else
    hipLaunchKernelGGL(k_bucket_dequant_sum<1>, dim3(bucket_grid(t, cus)), dim3(256), 0, s, t, codes, code_stride,
                       scales, scale_stride, R, block512, out, invR);
  return hipGetLastError();
}

}  // namespace gift
