// Activation quantisation variants on either side of the BitLinear
// contraction.
//
// RMSNorm then per-token quantisation: "BitNet b1.58 in Production: 1-Bit
// LLMs and Energy Benchmarks", listing "bit_linear.py" (the BitLinear input
// passes nn.RMSNorm before activation_quant).  RMSNorm multiplies token t by
// r_t = 1 / sqrt(mean_k x^2 + eps) and channel c by a gain w_c.  Per-token
// absmax quantisation is invariant under the positive factor r_t, so the
// codes are taken from v = x * w (one fp32 multiply per value) and r_t is
// folded into the de-quantisation scale: a'_t = max_c |v| * r_t, with the
// mean square accumulated in fp64 and the product rounded once to fp32
// (rmsnorm_scales, which also applies the 1e-8 floor of the normalised
// token).  The codes are those of the normalised token except where its
// scaled value lies within a few roundings of a tie.
//
// Quantisation from fp32: the same per-token rule as the bf16 kernel
// (section "The Mathematical Mechanism", item 2), for activations produced in
// fp32 on the GPU -- the SwiGLU output feeding the down projection.
//
// One workgroup per token; rows are read with 16-byte loads, the max is
// reduced as fp32 bit patterns (non-negative floats order like their bits)
// and the mean square as fp64, across the wave with shuffles and across the
// workgroup's waves in LDS (the in-wave steps on DPP row operations).
#include "bitlinear_internal.hpp"

namespace bitlinear {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t code_of(float v, float s) {
  float r = rintf(v * s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu;
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) { return wave_max_u32(v); }
__device__ __forceinline__ double wave_sum_d(double v) { return wave_sum_f64(v); }

// ---------------------------------------------------------------------------
// RMSNorm + quantisation
// ---------------------------------------------------------------------------

// 8 consecutive values of one token: x (one 16-byte bf16 chunk), gain (two
// float4, or none) -> v = x * gain
__device__ __forceinline__ void chunk_values(const uint4& xc, const float* __restrict__ gain8, float (&v)[8],
                                             float (&xv)[8]) {
  const uint32_t w[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    xv[2 * q] = bf16_lo(w[q]);
    xv[2 * q + 1] = bf16_hi(w[q]);
  }
  if (gain8) {
    const float4 g0 = *reinterpret_cast<const float4*>(gain8);
    const float4 g1 = *reinterpret_cast<const float4*>(gain8 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = xv[i] * g[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = xv[i];
  }
}

// True when a' = fl32(av * r), r = 1 / sqrt(ms), is certainly at least
// 1e-8, judged in fp32: ms inside the normal fp32 range, where the fp32
// estimate of av * r is within a few roundings of the exact one, and that
// estimate at least twice the floor.  Then the codes' scale is 127 / av
// (rmsnorm_scales) and no fp64 root is needed for them.
__device__ __forceinline__ bool floor_cannot_bind(float av, double ms) {
  if (!(ms >= 1.1754944e-38 && ms <= 3.4028235e+38)) return false;
  const float est = av * rsqrtf(static_cast<float>(ms));
  return est >= 2e-8f && est <= 3.0e+38f;
}

// Vector path: k % 8 == 0, x and gain 16-byte aligned, xq 8-byte aligned.
// 1024 threads per token; the row fits in CPT chunks per thread, and the
// products v = x * gain stay in registers between the two passes, so x and
// the gains are read once.
constexpr int kNormThreads = 1024;
constexpr int kNormWaves = kNormThreads / 64;

template <int CPT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_quant_vec(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ gain, float eps, int k,
                                                                  int8_t* __restrict__ xq, float* __restrict__ amax) {
  __shared__ uint32_t red_max[kNormWaves];
  __shared__ double red_ss[kNormWaves];
  const int64_t row = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * k);
  const int chunks = k >> 3;
  float vk[CPT][8];
  uint32_t mx = 0;
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int idx = threadIdx.x + i * kNormThreads;
    if (idx < chunks) {
      float xv[8];
      chunk_values(xr[idx], gain ? gain + idx * 8 : nullptr, vk[i], xv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ss += static_cast<double>(xv[j]) * static_cast<double>(xv[j]);
        mx = max(mx, __float_as_uint(fabsf(vk[i][j])));
      }
    }
  }
  mx = wave_max_u(mx);
  ss = wave_sum_d(ss);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_max[wave] = mx;
    red_ss[wave] = ss;
  }
  __syncthreads();
  uint32_t mall = red_max[0];
  double sall = red_ss[0];
#pragma unroll
  for (int w = 1; w < kNormWaves; ++w) {
    mall = max(mall, red_max[w]);
    sall += red_ss[w];
  }
  uint2* out = reinterpret_cast<uint2*>(xq + row * k);
  auto write_codes = [&](float s) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = threadIdx.x + i * kNormThreads;
      if (idx < chunks) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo |= code_of(vk[i][j], s) << (8 * j);
          hi |= code_of(vk[i][4 + j], s) << (8 * j);
        }
        out[idx] = make_uint2(lo, hi);
      }
    }
  };
  // The codes' scale 127 / max|v| needs no r unless the 1e-8 floor binds on
  // the normalised token (floor_cannot_bind).  Otherwise every thread takes
  // the exact fp64 path; only thread 0 forms the exact a' for the output.
  const float av = __uint_as_float(mall);
  const double ms = sall / static_cast<double>(k) + static_cast<double>(eps);
  if (floor_cannot_bind(av, ms)) {
    write_codes(127.0f / av);
    if (threadIdx.x == 0) {
      float ap, s;
      rmsnorm_scales(av, 1.0 / sqrt(ms), &ap, &s);
      amax[row] = ap;
    }
  } else {
    float ap, s;
    rmsnorm_scales(av, 1.0 / sqrt(ms), &ap, &s);
    write_codes(av > 0.0f ? s : 0.0f);  // all-zero v: every code is 0
    if (threadIdx.x == 0) amax[row] = ap;
  }
}

// General path: any k and alignment; two passes over the row with scalar loads.
__global__ __launch_bounds__(kThreads) void rmsnorm_quant_any(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ gain, float eps, int64_t k,
                                                              int8_t* __restrict__ xq, float* __restrict__ amax) {
  __shared__ uint32_t red_max[kWaves];
  __shared__ double red_ss[kWaves];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * k;
  uint32_t mx = 0;
  double ss = 0.0;
  for (int64_t i = threadIdx.x; i < k; i += kThreads) {
    const float xv = __uint_as_float(static_cast<uint32_t>(xr[i]) << 16);
    const float v = gain ? xv * gain[i] : xv;
    ss += static_cast<double>(xv) * static_cast<double>(xv);
    mx = max(mx, __float_as_uint(fabsf(v)));
  }
  mx = wave_max_u(mx);
  ss = wave_sum_d(ss);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_max[wave] = mx;
    red_ss[wave] = ss;
  }
  __syncthreads();
  uint32_t mall = red_max[0];
  double sall = red_ss[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    mall = max(mall, red_max[w]);
    sall += red_ss[w];
  }
  int8_t* out = xq + row * k;
  auto write_codes = [&](float s) {
    for (int64_t i = threadIdx.x; i < k; i += kThreads) {
      const float xv = __uint_as_float(static_cast<uint32_t>(xr[i]) << 16);
      const float v = gain ? xv * gain[i] : xv;
      out[i] = static_cast<int8_t>(code_of(v, s));
    }
  };
  // (as in rmsnorm_quant_vec)
  const float av = __uint_as_float(mall);
  const double ms = sall / static_cast<double>(k) + static_cast<double>(eps);
  float ap, s;
  if (floor_cannot_bind(av, ms)) {
    write_codes(127.0f / av);
    if (threadIdx.x == 0) {
      rmsnorm_scales(av, 1.0 / sqrt(ms), &ap, &s);
      amax[row] = ap;
    }
  } else {
    rmsnorm_scales(av, 1.0 / sqrt(ms), &ap, &s);
    write_codes(av > 0.0f ? s : 0.0f);
    if (threadIdx.x == 0) amax[row] = ap;
  }
}

// ---------------------------------------------------------------------------
// quantisation from fp32
// ---------------------------------------------------------------------------

// Vector path: k % 4 == 0, x 16-byte aligned, xq 4-byte aligned.
template <int CPT, int T = kThreads>
__global__ __launch_bounds__(T) void quant_f32_vec(const float* __restrict__ x, int k, int8_t* __restrict__ xq,
                                                   float* __restrict__ amax) {
  __shared__ uint32_t red_max[T / 64];
  const int64_t row = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + row * k);
  const int chunks = k >> 2;
  float4 c[CPT];
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int idx = threadIdx.x + i * T;
    if (idx < chunks) {
      c[i] = xr[idx];
      mx = max(max(mx, max(__float_as_uint(fabsf(c[i].x)), __float_as_uint(fabsf(c[i].y)))),
               max(__float_as_uint(fabsf(c[i].z)), __float_as_uint(fabsf(c[i].w))));
    }
  }
  mx = wave_max_u(mx);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red_max[wave] = mx;
  __syncthreads();
  uint32_t mall = red_max[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) mall = max(mall, red_max[w]);
  const float a = fmaxf(__uint_as_float(mall), 1e-8f);
  const float s = 127.0f / a;
  uint32_t* out = reinterpret_cast<uint32_t*>(xq + row * k);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int idx = threadIdx.x + i * T;
    if (idx < chunks)
      out[idx] = code_of(c[i].x, s) | (code_of(c[i].y, s) << 8) | (code_of(c[i].z, s) << 16) | (code_of(c[i].w, s) << 24);
  }
  if (threadIdx.x == 0) amax[row] = a;
}

__global__ __launch_bounds__(kThreads) void quant_f32_any(const float* __restrict__ x, int64_t k,
                                                          int8_t* __restrict__ xq, float* __restrict__ amax) {
  __shared__ uint32_t red_max[kWaves];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * k;
  uint32_t mx = 0;
  for (int64_t i = threadIdx.x; i < k; i += kThreads) mx = max(mx, __float_as_uint(fabsf(xr[i])));
  mx = wave_max_u(mx);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red_max[wave] = mx;
  __syncthreads();
  uint32_t mall = red_max[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) mall = max(mall, red_max[w]);
  const float a = fmaxf(__uint_as_float(mall), 1e-8f);
  const float s = 127.0f / a;
  int8_t* out = xq + row * k;
  for (int64_t i = threadIdx.x; i < k; i += kThreads) out[i] = static_cast<int8_t>(code_of(xr[i], s));
  if (threadIdx.x == 0) amax[row] = a;
}

}  // namespace

hipError_t launch_rmsnorm_quant_act(const uint16_t* x, const float* gain, float eps, int64_t m, int64_t k, int8_t* xq,
                                    float* amax, hipStream_t s) {
  const bool vec = (k % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (gain == nullptr || reinterpret_cast<uintptr_t>(gain) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(xq) % 8 == 0);
  const int64_t per_thread = (k / 8 + kNormThreads - 1) / kNormThreads;
  const dim3 grid(static_cast<unsigned>(m));
  const int ki = static_cast<int>(k);
  if (vec && per_thread <= 1)
    rmsnorm_quant_vec<1><<<grid, kNormThreads, 0, s>>>(x, gain, eps, ki, xq, amax);
  else if (vec && per_thread <= 2)
    rmsnorm_quant_vec<2><<<grid, kNormThreads, 0, s>>>(x, gain, eps, ki, xq, amax);
  else if (vec && per_thread <= 4)
    rmsnorm_quant_vec<4><<<grid, kNormThreads, 0, s>>>(x, gain, eps, ki, xq, amax);
  else if (vec && per_thread <= 8)
    rmsnorm_quant_vec<8><<<grid, kNormThreads, 0, s>>>(x, gain, eps, ki, xq, amax);
  else
    rmsnorm_quant_any<<<grid, kThreads, 0, s>>>(x, gain, eps, k, xq, amax);
  return hipGetLastError();
}

hipError_t launch_quant_act_f32(const float* x, int64_t m, int64_t k, int8_t* xq, float* amax, hipStream_t s) {
  const bool vec = (k % 4 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(xq) % 4 == 0);
  const int64_t per_thread = (k / 4 + kThreads - 1) / kThreads;
  const int64_t per_long = (k / 4 + kNormThreads - 1) / kNormThreads;
  const dim3 grid(static_cast<unsigned>(m));
  const int ki = static_cast<int>(k);
  if (vec && per_thread > 1 && per_long <= 8) {  // rows of more than 1024 values: 1024 threads per token
    if (per_long <= 1)
      quant_f32_vec<1, kNormThreads><<<grid, kNormThreads, 0, s>>>(x, ki, xq, amax);
    else if (per_long <= 2)
      quant_f32_vec<2, kNormThreads><<<grid, kNormThreads, 0, s>>>(x, ki, xq, amax);
    else if (per_long <= 4)
      quant_f32_vec<4, kNormThreads><<<grid, kNormThreads, 0, s>>>(x, ki, xq, amax);
    else
      quant_f32_vec<8, kNormThreads><<<grid, kNormThreads, 0, s>>>(x, ki, xq, amax);
  } else if (vec && per_thread <= 1)
    quant_f32_vec<1><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 2)
    quant_f32_vec<2><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 4)
    quant_f32_vec<4><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 8)
    quant_f32_vec<8><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else if (vec && per_thread <= 16)
    quant_f32_vec<16><<<grid, kThreads, 0, s>>>(x, ki, xq, amax);
  else
    quant_f32_any<<<grid, kThreads, 0, s>>>(x, k, xq, amax);
  return hipGetLastError();
}

}  // namespace bitlinear
