// Flat gradient buckets: the Euclidean FP8 codec over many tensors in one
// launch per phase (GIFT 阅读笔记, Algorithm 1, the Euclidean branch: Scale,
// AllReduceMax, Q, AllReduceSum, Dequantize / N for every layer outside the
// selected set).  Scales per tensor, or per 512 consecutive elements of a
// tensor (the per-block Euclidean baseline of the experiment setup, block
// size 512; blocks restart at every tensor and a tensor's last block may be
// shorter).
//
// The tensors lie one after another in one flat fp32 buffer (element
// counts multiples of 4); codes use the same offsets, scales are numbered
// tensor by tensor.  Work is cut into chunks of 4096 elements of one tensor
// (a tensor's last chunk may be partial); wave w of a 256-thread workgroup
// takes elements 1024 w .. 1024 w + 1023 of the chunk (512-element blocks
// 2w and 2w + 1), lane l the float4s at 256 h + 4 l, h = 0..3, so a wave's
// loads are contiguous and h = 0, 1 (2, 3) cover one block.  Each
// workgroup takes one contiguous range of chunks and follows the tensor
// boundaries through the prefix table, so the chunk-to-tensor search runs
// once per workgroup.
#include "fp8_codec.hpp"
#include "gift_internal.hpp"

namespace gift {

constexpr int kBChunk = 4096;
constexpr int kBH = 4;   // float4 loads per lane per chunk
typedef int int32x4_b __attribute__((ext_vector_type(4)));

// Reads of the offset tables, the amax slots and the scales: wave-uniform
// indices (taken through readfirstlane) into memory that no launch writes
// while it runs, read through the constant address space so that the
// compiler issues scalar loads.  (As vector loads they would retire in
// order behind the next chunk's data loads, and the wait for them would
// also wait for those.)
template <class T>
__device__ __forceinline__ T cld(const T* p, int64_t i) {
  typedef const __attribute__((address_space(4))) T CT;
  return ((CT*)(uintptr_t)p)[i];
}
__device__ __forceinline__ int uidx(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uidx64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int bucket_tensor(const int64_t* __restrict__ cs, int n, int64_t c) {
  int lo = 0, hi = n;   // the largest i with cs[i] <= c (cs[0] = 0, cs[n] = chunks)
  while (hi - lo > 1) {
    const int mid = uidx((lo + hi) >> 1);
    if (cld(cs, mid) <= c) lo = mid;
    else hi = mid;
  }
  return uidx(lo);
}

// A workgroup's contiguous range of chunks and the tensor of the current one
// (all workgroup-uniform).
struct BRange {
  int64_t c, end;    // current chunk, one past the last
  int i;             // tensor of chunk c
  int64_t next;      // first chunk of tensor i + 1
  __device__ BRange(const BucketTable& t) {
    const int64_t per = (t.chunks + gridDim.x - 1) / gridDim.x;
    c = uidx64((int64_t)blockIdx.x * per);
    end = uidx64(min(c + per, t.chunks));
    i = c < end ? bucket_tensor(t.chunk_start, t.n, c) : 0;
    next = c < end ? cld(t.chunk_start, uidx(i + 1)) : 0;
  }
  // move to chunk c + 1; returns true when it starts a new tensor
  __device__ bool advance(const BucketTable& t) {
    ++c;
    if (c < end && c >= next) {
      do {
        i = uidx(i + 1);
        next = cld(t.chunk_start, uidx(i + 1));
      } while (c >= next);
      return true;
    }
    return false;
  }
};

// Buffer resource over [p, p + bytes): loads past it return zeros and
// stores past it are dropped, so the partial last chunk of a tensor needs
// no branches around its memory operations.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

// Chunk c of tensor i: kBChunk elements from element chunk_elem of the
// tensor (fewer in its last chunk).  Wave w takes elements 1024 w ..
// 1024 w + 1023 of the chunk (512-element blocks 2w and 2w + 1), lane l the
// float4s at 256 h + 4 l, h = 0..3.
struct BLane {
  int64_t base;      // first element of the tensor in the flat buffer
  int64_t k;         // chunk of the tensor
  int64_t first;     // first element of the chunk in the flat buffer
  int valid;         // elements of the chunk inside the tensor (<= kBChunk)
  int wave;          // wave-uniform
  int off;           // this lane's first element within the chunk (h = 0)
  __device__ BLane(const BucketTable& t, const BRange& r) {
    const int i = uidx(r.i);
    base = uidx64(cld(t.elem_off, i));
    const int64_t numel = uidx64(cld(t.elem_off, uidx(i + 1))) - base;
    k = uidx64(r.c - cld(t.chunk_start, i));
    first = base + k * kBChunk;
    const int64_t rest = numel - k * kBChunk;
    valid = (int)(rest < kBChunk ? rest : kBChunk);
    wave = uidx((int)(threadIdx.x >> 6));
    off = 1024 * wave + 4 * (int)(threadIdx.x & 63);
  }
  __device__ bool live(int h) const { return off + 256 * h < valid; }
  // block 2 wave + half holds an element of the tensor (wave-uniform)
  __device__ bool block_live(int half) const { return 1024 * wave + 512 * half < valid; }
};

__device__ __forceinline__ uint32_t absb(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }
__device__ __forceinline__ uint32_t umax4(float4 v) {
  return max(max(absb(v.x), absb(v.y)), max(absb(v.z), absb(v.w)));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// Workgroup max of v (every thread calls it), then one atomicMax.
__device__ __forceinline__ void flush_tensor_max(uint32_t v, uint32_t* slot, uint32_t* red) {
  v = wave_umax(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (m) atomicMax(slot, m);
  }
  __syncthreads();
}

// The kBH float4s of this lane in chunk L (zeros past the tensor's end).
__device__ __forceinline__ void load_lane(const float* __restrict__ g, const BLane& L, float4* v) {
  const auto rs = brsrc(g + L.first, (int64_t)L.valid * 4);
#pragma unroll
  for (int h = 0; h < kBH; ++h)
    v[h] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (L.off + 256 * h), 0, 0));
}

// Scale slot of half `half` of this wave's range (per tensor: the tensor's).
__device__ __forceinline__ int64_t slot_of(const BucketTable& t, const BRange& r, const BLane& L, int block512,
                                           int half) {
  return uidx64(cld(t.scale_off, uidx(r.i)) + (block512 ? 8 * L.k + 2 * L.wave + half : 0));
}

// amax (as |x| bit patterns) of every scale block into slots (zeroed
// before).  The next chunk's values are loaded while this chunk is reduced.
__global__ void __launch_bounds__(256) k_bucket_amax(BucketTable t, const float* __restrict__ g, int block512,
                                                     uint32_t* __restrict__ slots) {
  __shared__ uint32_t red[4];
  BRange r(t);
  if (r.c >= r.end) return;   // workgroup-uniform
  uint32_t run = 0;   // per tensor: this lane's max over the tensor's chunks so far
  BLane L(t, r);
  float4 v[kBH];
  load_lane(g, L, v);
  for (;;) {
    BRange rn = r;
    const bool newt = rn.advance(t);
    const bool more = rn.c < rn.end;   // workgroup-uniform
    BLane Ln = L;
    float4 vn[kBH];
    if (more) {
      Ln = BLane(t, rn);
      load_lane(g, Ln, vn);
    }
    if (block512) {
      const uint32_t b0 = wave_umax(max(umax4(v[0]), umax4(v[1])));
      const uint32_t b1 = wave_umax(max(umax4(v[2]), umax4(v[3])));
      const int64_t blk = slot_of(t, r, L, 1, 0);
      if ((threadIdx.x & 63) == 0) {
        if (L.block_live(0)) slots[blk] = b0;   // one wave per block: no other writer
        if (L.block_live(1)) slots[blk + 1] = b1;
      }
    } else {
#pragma unroll
      for (int h = 0; h < kBH; ++h) run = max(run, umax4(v[h]));
      if (newt || !more) {   // the tensor's last chunk in this range (workgroup-uniform)
        flush_tensor_max(run, slots + slot_of(t, r, L, 0, 0), red);
        run = 0;
      }
    }
    if (!more) break;
    r = rn;
    L = Ln;
#pragma unroll
    for (int h = 0; h < kBH; ++h) v[h] = vn[h];
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

// The amax bits the codes of half `half` use (shared or local) and the local
// ones (for amax_out), read as scalars.
struct BAmax {
  uint32_t use[2], local[2];
};
__device__ __forceinline__ void load_amax(const BucketTable& t, const BRange& r, const BLane& L, int block512,
                                          const uint32_t* __restrict__ slots, const float* __restrict__ amax_in,
                                          BAmax& a) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t slot = slot_of(t, r, L, block512, half);
    a.local[half] = slots ? cld(slots, slot) : 0u;
    a.use[half] = amax_in ? absb(cld(amax_in, slot)) : a.local[half];
  }
}

template <int FMT>
__global__ void __launch_bounds__(256) k_bucket_quantize(BucketTable t, const float* __restrict__ g, int block512,
                                                         const uint32_t* __restrict__ slots,
                                                         const float* __restrict__ amax_in,
                                                         float* __restrict__ amax_out, uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const float fmax = fp8_fmax(FMT);
  BRange r(t);
  if (r.c >= r.end) return;
  // the next chunk's values and amax words are loaded while this chunk is
  // encoded
  BLane L(t, r);
  float4 v[kBH];
  load_lane(g, L, v);
  BAmax am;
  load_amax(t, r, L, block512, slots, amax_in, am);
  for (;;) {
    BRange rn = r;
    rn.advance(t);
    const bool more = rn.c < rn.end;   // workgroup-uniform
    BLane Ln = L;
    float4 vn[kBH];
    BAmax amn = am;
    if (more) {
      Ln = BLane(t, rn);
      load_lane(g, Ln, vn);
      load_amax(t, rn, Ln, block512, slots, amax_in, amn);
    }
    const auto qs = brsrc(codes + L.first, L.valid);
    // the scale of each half of the wave's range (one block each; per
    // tensor both are the tensor's)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (!L.block_live(half)) continue;   // wave-uniform: the block is absent
      float rr, sc;
      scale_pair(am.use[half], fmax, rr, sc);
      const bool bad = am.use[half] >= 0x7F800000u;
      const bool writer = (threadIdx.x & 63) == 0 &&
                          (block512 || (L.k == 0 && threadIdx.x == 0 && half == 0));
      if (writer) {
        const int64_t slot = slot_of(t, r, L, block512, half);
        scales[slot] = sc;
        if (amax_out) amax_out[slot] = __uint_as_float(am.local[half]);
        if (bad) atomicOr(t.flags, (uint32_t)GIFT_FLAG_NONFINITE);
      }
#pragma unroll
      for (int h = 2 * half; h < 2 * half + 2; ++h)
        __builtin_amdgcn_raw_buffer_store_b32(bad ? 0x7F7F7F7Fu : codes4<FMT>(v[h], rr, fmax), qs,
                                              L.off + 256 * h, 0, 0);
    }
    if (!more) break;
    r = rn;
    L = Ln;
    am = amn;
#pragma unroll
    for (int h = 0; h < kBH; ++h) v[h] = vn[h];
  }
}

// U = (1/R) sum_r s_r dec(q_r), replicas in increasing r (from replica 0's
// term, so a lone -0 stays -0).  RC: the replica count when known at
// compile time (0: R at run time).  The code loads and the fp32 stores are
// non-temporal (each byte is touched once: 3.24 -> 3.16 ms for the 155
// tensors of the 600M-class bucket at R = 8).
constexpr int kNTb = 2;
template <int FMT, int RC>
__global__ void __launch_bounds__(256) k_bucket_dequant_sum(BucketTable t, const uint8_t* __restrict__ codes,
                                                            int64_t code_stride, const float* __restrict__ scales,
                                                            int64_t scale_stride, int Rrt, int block512,
                                                            float* __restrict__ out, float invR) {
  const int R = RC > 0 ? RC : Rrt;
  BRange rg(t);
  for (; rg.c < rg.end; rg.advance(t)) {
    const BLane L(t, rg);
    const int64_t s0 = slot_of(t, rg, L, block512, 0);
    const int64_t s1 = slot_of(t, rg, L, block512, 1);
    float acc[kBH][4];
#pragma unroll (RC > 0 ? RC : 1)
    for (int r = 0; r < R; ++r) {
      const auto qs = brsrc(codes + (int64_t)r * code_stride + L.first, L.valid);
      const float sa = cld(scales, uidx64((int64_t)r * scale_stride + s0));
      const float sb = L.block_live(1) ? cld(scales, uidx64((int64_t)r * scale_stride + s1)) : 0.0f;
      uint32_t w[kBH];
#pragma unroll
      for (int h = 0; h < kBH; ++h) w[h] = __builtin_amdgcn_raw_buffer_load_b32(qs, L.off + 256 * h, 0, kNTb);
#pragma unroll
      for (int h = 0; h < kBH; ++h) {
        const float s = h < 2 ? sa : sb;
        float v[4];
        dec4_fp8<FMT>(w[h], v);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[h][j] = r == 0 ? s * v[j] : __builtin_fmaf(s, v[j], acc[h][j]);
      }
    }
    const auto os = brsrc(out + L.first, (int64_t)L.valid * 4);
#pragma unroll
    for (int h = 0; h < kBH; ++h)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(int32x4_b, make_float4(acc[h][0] * invR, acc[h][1] * invR, acc[h][2] * invR,
                                                    acc[h][3] * invR)),
          os, 4 * (L.off + 256 * h), 0, kNTb);
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

template <int FMT>
static void launch_bds(const BucketTable& t, const uint8_t* codes, int64_t cst, const float* scales, int64_t sst,
                       int R, int block512, float* out, dim3 gd, hipStream_t s) {
  const float invR = 1.0f / (float)R;
  switch (R) {
    case 4:
      hipLaunchKernelGGL((k_bucket_dequant_sum<FMT, 4>), gd, dim3(256), 0, s, t, codes, cst, scales, sst, R, block512,
                         out, invR);
      break;
    case 8:
      hipLaunchKernelGGL((k_bucket_dequant_sum<FMT, 8>), gd, dim3(256), 0, s, t, codes, cst, scales, sst, R, block512,
                         out, invR);
      break;
    case 16:
      hipLaunchKernelGGL((k_bucket_dequant_sum<FMT, 16>), gd, dim3(256), 0, s, t, codes, cst, scales, sst, R,
                         block512, out, invR);
      break;
    default:
      hipLaunchKernelGGL((k_bucket_dequant_sum<FMT, 0>), gd, dim3(256), 0, s, t, codes, cst, scales, sst, R, block512,
                         out, invR);
  }
}

hipError_t launch_bucket_dequant_sum(const BucketTable& t, const uint8_t* codes, int64_t code_stride,
                                     const float* scales, int64_t scale_stride, int R, int fmt, int block512,
                                     float* out, int cus, hipStream_t s) {
  if (t.chunks == 0) return hipSuccess;
  const dim3 gd(bucket_grid(t, cus));
  if (fmt == 0)
    launch_bds<0>(t, codes, code_stride, scales, scale_stride, R, block512, out, gd, s);
  else
    launch_bds<1>(t, codes, code_stride, scales, scale_stride, R, block512, out, gd, s);
  return hipGetLastError();
}

}  // namespace gift
