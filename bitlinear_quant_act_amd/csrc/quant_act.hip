// Per-token absmax int8 activation quantisation.
//
// "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
// "The Mathematical Mechanism", item 2: x_q = Clip(Round(x * Q_b / a'),
// -Q_b, Q_b) with Q_b = 127 and one scale per token; a' = max(max|x|, 1e-8).
//
// One workgroup per token.  The token's bf16 row is read once with 16-byte
// loads and kept in registers; |x| is reduced as integer bit patterns (for
// finite non-negative floats the bit order is the numeric order), first
// across the wave with DPP row operations, then across the four waves in
// LDS.  The scale is one IEEE fp32 divide (127 / a'); every code is one fp32
// multiply followed by v_rndne_f32 (round half to even) and a clamp, so the
// result is bit-identical to any other evaluation of the same two roundings.
#include "bitlinear_internal.hpp"

namespace bitlinear {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t quant_code(uint32_t bits16, float s) {
  float r = rintf(bf16_to_f32(bits16) * s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu;
}

__device__ __forceinline__ uint32_t abs_max2(uint32_t word) {
  // two bf16 values in one 32-bit word; clear the sign bits and compare
  return max(word & 0x7fffu, (word >> 16) & 0x7fffu);
}

// max over a workgroup of T threads; every thread receives the result
template <int T = kThreads>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < T / 64; ++i) r = max(r, red[i]);
  return r;
}

// rows longer than kThreads chunks: a workgroup of kLongThreads per token,
// so each thread converts at most a few chunks
constexpr int kLongThreads = 1024;

// Vector path: k % 8 == 0, x 16-byte aligned, xq 8-byte aligned; the row
// (k / 8 chunks of 8 values) fits in CPT chunks per thread of T.
template <int CPT, int T = kThreads>
__global__ __launch_bounds__(T) void quant_act_vec(const uint16_t* __restrict__ x, int k,
                                                   int8_t* __restrict__ xq,
                                                   float* __restrict__ amax) {
  __shared__ uint32_t red[T / 64];
  const int64_t row = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * k);
  const int chunks = k >> 3;
  uint4 c[CPT];
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int idx = threadIdx.x + i * T;
    if (idx < chunks) {
      c[i] = xr[idx];
      mx = max(mx, max(max(abs_max2(c[i].x), abs_max2(c[i].y)), max(abs_max2(c[i].z), abs_max2(c[i].w))));
    }
  }
  mx = block_max<T>(mx, red);
  const float a = fmaxf(bf16_to_f32(mx), 1e-8f);
  const float s = 127.0f / a;
  uint2* out = reinterpret_cast<uint2*>(xq + row * k);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int idx = threadIdx.x + i * T;
    if (idx < chunks) {
      const uint32_t w[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        lo |= quant_code(w[j] & 0xffffu, s) << (16 * j);
        lo |= quant_code(w[j] >> 16, s) << (16 * j + 8);
        hi |= quant_code(w[j + 2] & 0xffffu, s) << (16 * j);
        hi |= quant_code(w[j + 2] >> 16, s) << (16 * j + 8);
      }
      out[idx] = make_uint2(lo, hi);
    }
  }
  if (threadIdx.x == 0) amax[row] = a;
}

// General path: any k and alignment; two passes over the row with 2-byte loads.
__global__ __launch_bounds__(kThreads) void quant_act_any(const uint16_t* __restrict__ x, int64_t k,
                                                          int8_t* __restrict__ xq,
                                                          float* __restrict__ amax) {
  __shared__ uint32_t red[kWaves];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * k;
  uint32_t mx = 0;
  for (int64_t i = threadIdx.x; i < k; i += kThreads) mx = max(mx, static_cast<uint32_t>(xr[i]) & 0x7fffu);
  mx = block_max(mx, red);
  const float a = fmaxf(bf16_to_f32(mx), 1e-8f);
  const float s = 127.0f / a;
  int8_t* out = xq + row * k;
  for (int64_t i = threadIdx.x; i < k; i += kThreads)
    out[i] = static_cast<int8_t>(quant_code(xr[i], s));
  if (threadIdx.x == 0) amax[row] = a;
}

// ---- per-tensor variant ("BitNet 1-bit LLM Inference Framework", "The Core
// Structure of BitNet b1.58": the BitLinear class's activation_quantize) --
// one g = max |x| over the whole [m][k] tensor, code = round(clamp((x * 128) /
// (g + 1e-8), -128, 127)): one fp32 multiply (exact), one IEEE divide, clamp,
// v_rndne.  Kernel 1 leaves one max (bf16 bit pattern without sign) per
// workgroup of a contiguous range; kernel 2 folds them in every workgroup and
// quantizes its range (at most 1024 ranges, so the partials take at most
// 4 KiB).  A tensor of at most kTensorOneGroup values is done by one
// workgroup in one launch.

constexpr int64_t kTensorChunk = 16384;     // least values per workgroup range
constexpr int64_t kTensorOneGroup = 16384;  // single-launch size
constexpr int kTensorMaxParts = 1024;       // ranges (workgroups) at most

// values per range: at least kTensorChunk, a multiple of 8, at most kTensorMaxParts ranges
inline int64_t tensor_range(int64_t total) {
  int64_t per = (total + kTensorMaxParts - 1) / kTensorMaxParts;
  per = per < kTensorChunk ? kTensorChunk : per;
  return (per + 7) & ~int64_t(7);
}

__device__ __forceinline__ uint32_t tensor_code(uint32_t bits16, float d) {
  float t = (bf16_to_f32(bits16) * 128.0f) / d;
  t = fminf(fmaxf(t, -128.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(rintf(t))) & 0xffu;
}

__device__ __forceinline__ uint32_t range_max(const uint16_t* __restrict__ x, int64_t begin, int64_t end, bool vec) {
  uint32_t mx = 0;
  if (vec) {  // begin, end multiples of 8 (end may be the tensor's end: tail below)
    const int64_t vend = begin + ((end - begin) & ~int64_t(7));
    for (int64_t i = begin / 8 + threadIdx.x; i < vend / 8; i += kThreads) {
      const uint4 c = reinterpret_cast<const uint4*>(x)[i];
      mx = max(mx, max(max(abs_max2(c.x), abs_max2(c.y)), max(abs_max2(c.z), abs_max2(c.w))));
    }
    for (int64_t i = vend + threadIdx.x; i < end; i += kThreads) mx = max(mx, static_cast<uint32_t>(x[i]) & 0x7fffu);
  } else {
    for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) mx = max(mx, static_cast<uint32_t>(x[i]) & 0x7fffu);
  }
  return mx;
}

__device__ __forceinline__ void range_quant(const uint16_t* __restrict__ x, int64_t begin, int64_t end, float d,
                                            int8_t* __restrict__ xq, bool vec) {
  if (vec) {
    const int64_t vend = begin + ((end - begin) & ~int64_t(7));
    for (int64_t i = begin / 8 + threadIdx.x; i < vend / 8; i += kThreads) {
      const uint4 c = reinterpret_cast<const uint4*>(x)[i];
      const uint32_t w[4] = {c.x, c.y, c.z, c.w};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        lo |= tensor_code(w[j] & 0xffffu, d) << (16 * j);
        lo |= tensor_code(w[j] >> 16, d) << (16 * j + 8);
        hi |= tensor_code(w[j + 2] & 0xffffu, d) << (16 * j);
        hi |= tensor_code(w[j + 2] >> 16, d) << (16 * j + 8);
      }
      reinterpret_cast<uint2*>(xq)[i] = make_uint2(lo, hi);
    }
    for (int64_t i = vend + threadIdx.x; i < end; i += kThreads) xq[i] = static_cast<int8_t>(tensor_code(x[i], d));
  } else {
    for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) xq[i] = static_cast<int8_t>(tensor_code(x[i], d));
  }
}

__global__ __launch_bounds__(kThreads) void tensor_max_partial(const uint16_t* __restrict__ x, int64_t total,
                                                               int64_t per, uint32_t* __restrict__ partials,
                                                               bool vec) {
  __shared__ uint32_t red[kWaves];
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t end = min(total, begin + per);
  const uint32_t mx = block_max(range_max(x, begin, end, vec), red);
  if (threadIdx.x == 0) partials[blockIdx.x] = mx;
}

// parts == 0: one workgroup, the max of the whole tensor computed here
__global__ __launch_bounds__(kThreads) void tensor_quant(const uint16_t* __restrict__ x, int64_t total, int64_t per,
                                                         const uint32_t* __restrict__ partials, int parts,
                                                         int8_t* __restrict__ xq, float* __restrict__ gx, bool vec) {
  __shared__ uint32_t red[kWaves];
  uint32_t mx = 0;
  int64_t begin = 0, end = total;
  if (parts == 0) {
    mx = range_max(x, 0, total, vec);
  } else {
    for (int i = threadIdx.x; i < parts; i += kThreads) mx = max(mx, partials[i]);
    begin = static_cast<int64_t>(blockIdx.x) * per;
    end = min(total, begin + per);
  }
  mx = block_max(mx, red);
  const float g = bf16_to_f32(mx);
  const float d = g + 1e-8f;
  range_quant(x, begin, end, d, xq, vec);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gx = g;
}

}  // namespace

int quant_tensor_partial_count(int64_t m, int64_t k) {
  const int64_t total = m * k;
  if (total <= kTensorOneGroup) return 0;
  const int64_t per = tensor_range(total);
  return static_cast<int>((total + per - 1) / per);
}

hipError_t launch_quant_act_tensor(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* gx,
                                   uint32_t* partials, hipStream_t s) {
  const int64_t total = m * k;
  const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 8 == 0);
  const int parts = quant_tensor_partial_count(m, k);
  if (parts > kTensorMaxParts) return hipErrorInvalidValue;
  if (parts == 0) {
    tensor_quant<<<1, kThreads, 0, s>>>(x, total, total, nullptr, 0, xq, gx, vec);
    return hipGetLastError();
  }
  const int64_t per = tensor_range(total);
  tensor_max_partial<<<parts, kThreads, 0, s>>>(x, total, per, partials, vec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tensor_quant<<<parts, kThreads, 0, s>>>(x, total, per, partials, parts, xq, gx, vec);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* amax,
                            hipStream_t s) {
  const bool vec = (k % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(xq) % 8 == 0);
  const int64_t chunks = k / 8;
  const int64_t per_thread = (chunks + kThreads - 1) / kThreads;
  const dim3 grid(static_cast<unsigned>(m));
  const int ki = static_cast<int>(k);
  const int64_t per_long = (chunks + kLongThreads - 1) / kLongThreads;
  if (vec && per_thread > 1 && per_long <= 8) {  // long rows: 1024 threads per token
    if (per_long <= 1)
      quant_act_vec<1, kLongThreads><<<grid, kLongThreads, 0, s>>>(x, ki, xq, amax);
    else if (per_long <= 2)
      quant_act_vec<2, kLongThreads><<<grid, kLongThreads, 0, s>>>(x, ki, xq, amax);
    else if (per_long <= 4)
      quant_act_vec<4, kLongThreads><<<grid, kLongThreads, 0, s>>>(x, ki, xq, amax);
    else
      quant_act_vec<8, kLongThreads><<<grid, kLongThreads, 0, s>>>(x, ki, xq, amax);
  } else if (vec && per_thread <= 1)
    quant_act_vec<1><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 2)
    quant_act_vec<2><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 4)
    quant_act_vec<4><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 8)
    quant_act_vec<8><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 16)
    quant_act_vec<16><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else
    quant_act_any<<<grid, kThreads, 0, s>>>(x, k, xq, amax);
  return hipGetLastError();
}

}  // namespace bitlinear
