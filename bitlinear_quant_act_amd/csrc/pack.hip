// One-time weight preparation: absmean scale, ternary RoundClip, 2-bit pack.
//
// "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
// "The Mathematical Mechanism", item 1: gamma = (1/nm) sum |W_ij| and
// W_q = Clip(Round(W / (gamma + eps)), -1, 1); eps = 1e-5, Round = half to
// even.  Two bits per weight as in "BitNet 1-bit LLM Inference Framework",
// section "How the LUT Kernel Works", in this library's tiled order.
//
// Kernel 1 (absmean_partial) streams W once and leaves one fp64 partial sum
// of |W| per workgroup in the caller's workspace.  Kernel 2 (ternarize_pack)
// first folds those partials -- every workgroup in the same fixed order, so
// all of them hold the same bits of gamma -- then streams W again and writes
// the packed tiles.  gamma = fp32(fp64 sum / (n k)), one rounding to fp32.
// Both kernels read W with 16-byte loads, consecutive lanes on consecutive
// addresses; the 16x smaller packed output is scattered into 1 KiB tiles.
#include <mutex>

#include "bitlinear_internal.hpp"

namespace bitlinear {

// Scratch of the allocation-free pack (bitlinear_pack_weights_noalloc): the
// fp64 partial sums of |W| that the caller's workspace holds otherwise, at
// most kPackPartials of them (8 KiB).  Every GPU the library runs on holds
// its own copy until the process ends; each call overwrites every slot it
// reads, so nothing needs clearing, and calls that overlap on one GPU race
// on it.
static __device__ __align__(256) double scratch[kPackPartials];

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r += red[i];
  return r;
}

// Partition of the flat weight array into `parts` contiguous ranges, each a
// multiple of 4 floats (so 16-byte alignment of W carries over).
__host__ __device__ inline int64_t split_per_part(int64_t total, int parts) {
  int64_t p = (total + parts - 1) / parts;
  return (p + 3) & ~int64_t(3);
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) void absmean_partial(const float* __restrict__ w, int64_t total,
                                                            int64_t per_part,
                                                            double* __restrict__ partials) {
  __shared__ double red[kWaves];
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * per_part;
  const int64_t end = max(begin, min(total, begin + per_part));  // empty range past the end
  double s = 0.0;
  if (kVec) {
    const int64_t vend = begin + ((end - begin) & ~int64_t(3));
    const float4* w4 = reinterpret_cast<const float4*>(w);
    for (int64_t i = begin / 4 + threadIdx.x; i < vend / 4; i += kThreads) {
      const float4 v = w4[i];
      s += fabs(static_cast<double>(v.x)) + fabs(static_cast<double>(v.y)) +
           fabs(static_cast<double>(v.z)) + fabs(static_cast<double>(v.w));
    }
    for (int64_t i = vend + threadIdx.x; i < end; i += kThreads) s += fabs(static_cast<double>(w[i]));
  } else {
    for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) s += fabs(static_cast<double>(w[i]));
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__device__ __forceinline__ uint32_t ternary_field(float wv, float d) {
  float r = rintf(wv / d);  // one IEEE fp32 divide, round half to even
  r = fminf(fmaxf(r, -1.0f), 1.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 3u;  // two's complement in 2 bits
}

// position of column t (0..15) of a 16-column word
__device__ __forceinline__ int field_shift(int t) { return 8 * (t & 3) + 2 * (t >> 2); }

// Ternary words of the packed matrix, one thread per 16-column word (words of
// a padded row are consecutive).  The denominator is gamma + 1e-5 for every
// row, or, with row_scale set, the binary16 scale of the word's row + 1e-5.
template <bool kVec>
__device__ void pack_ternary_words(const float* __restrict__ w, int64_t n, int64_t k, int64_t kt_count, float d_all,
                                   const uint16_t* __restrict__ row_scale, uint32_t* __restrict__ packed) {
  const int64_t words_per_row = kt_count * 16;
  const int64_t rows = row_blocks(n) * kTileRows;
  const int64_t total = rows * words_per_row;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t row = idx / words_per_row;
    const int64_t cw = idx - row * words_per_row;
    const int64_t k0 = cw * 16;
    const float d = (row_scale && row < n) ? half_bits_to_float(row_scale[row]) + 1e-5f : d_all;
    uint32_t word = 0;
    if (row < n && k0 + 16 <= k) {
      const float* src = w + row * k + k0;
      if (kVec) {
        const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = s4[q];
          word |= ternary_field(v.x, d) << field_shift(4 * q + 0);
          word |= ternary_field(v.y, d) << field_shift(4 * q + 1);
          word |= ternary_field(v.z, d) << field_shift(4 * q + 2);
          word |= ternary_field(v.w, d) << field_shift(4 * q + 3);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) word |= ternary_field(src[t], d) << field_shift(t);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t f = (row < n && k0 + t < k) ? ternary_field(w[row * k + k0 + t], d) : kZeroCode;
        word |= f << field_shift(t);
      }
    }
    // destination: tile (row / 16, cw / 16), slot (row % 16) + 16 * ((cw % 16) / 4), word cw % 4
    const int64_t kt = cw >> 4;
    const int64_t slot = (row & 15) + 16 * ((cw & 15) >> 2);
    packed[((row >> 4) * kt_count + kt) * 256 + slot * 4 + (cw & 3)] = word;
  }
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) void ternarize_pack(const float* __restrict__ w, int64_t n,
                                                           int64_t k, int64_t kt_count,
                                                           const double* __restrict__ partials,
                                                           int parts, float* __restrict__ gamma_out,
                                                           uint32_t* __restrict__ packed) {
  __shared__ double red[kWaves];
  double s = 0.0;
  for (int i = threadIdx.x; i < parts; i += kThreads) s += partials[i];
  s = block_sum(s, red);
  const float gamma = static_cast<float>(s / (static_cast<double>(n) * static_cast<double>(k)));
  if (blockIdx.x == 0 && threadIdx.x == 0) *gamma_out = gamma;
  pack_ternary_words<kVec>(w, n, k, kt_count, gamma + 1e-5f, nullptr, packed);
}

// ---- per-output-channel binary16 scales ("BitNet-2B-4T: Inside the
// 2B-Parameter, 4T-Token 1-Bit LLM", "Weight Representation: Ternary + Scale,
// Not Pure Binary"): the scale of row r is its absmean -- fp64 sum of |W|,
// divided by k, rounded to fp32, then to binary16 (round to nearest even) --
// and the row is ternarized with that stored value.  One wave per row.
__global__ __launch_bounds__(kThreads) void row_scale_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                             uint16_t* __restrict__ scales) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= n) return;
  const int lane = threadIdx.x & 63;
  const float* r = w + row * k;
  double s = 0.0;
  for (int64_t c = lane; c < k; c += 64) s += fabs(static_cast<double>(r[c]));
  s = wave_sum_f64(s);
  if (lane == 0) {
    const float mean = static_cast<float>(s / static_cast<double>(k));
    scales[row] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(mean));
  }
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) void ternarize_pack_rows(const float* __restrict__ w, int64_t n, int64_t k,
                                                                int64_t kt_count, const uint16_t* __restrict__ scales,
                                                                uint32_t* __restrict__ packed) {
  pack_ternary_words<kVec>(w, n, k, kt_count, 0.0f, scales, packed);
}

// ---- binary sign bits ("BitNet's 1-Bit Transformer: Architecture
// Breakdown", "Binary Weight Matrices with Learnable Scaling": W_bit =
// s * sign(W)); bit set for W < 0, so zero packs as +1.  One thread per
// 32-column word; word cw of a row is word cw % 4 of slot (row % 16) +
// 16 * ((cw % 16) / 4) in tile (row / 16, cw / 16).
__device__ __forceinline__ int sign_bit_pos(int c) { return 8 * (c & 3) + 7 - (c >> 2); }

__device__ __forceinline__ int64_t bin_word_index(int64_t row, int64_t cw, int64_t bt) {
  const int64_t slot = (row & 15) + 16 * ((cw & 15) >> 2);
  return ((row >> 4) * bt + (cw >> 4)) * 256 + slot * 4 + (cw & 3);
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) void pack_binary_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                               int64_t bt, uint32_t* __restrict__ packed) {
  const int64_t words_per_row = bt * 16;
  const int64_t total = row_blocks(n) * kTileRows * words_per_row;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t row = idx / words_per_row;
    const int64_t cw = idx - row * words_per_row;
    const int64_t k0 = cw * 32;
    uint32_t word = 0;
    if (row < n && kVec && k0 + 32 <= k) {
      const float4* s4 = reinterpret_cast<const float4*>(w + row * k + k0);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = s4[q];
        word |= static_cast<uint32_t>(v.x < 0.0f) << sign_bit_pos(4 * q + 0);
        word |= static_cast<uint32_t>(v.y < 0.0f) << sign_bit_pos(4 * q + 1);
        word |= static_cast<uint32_t>(v.z < 0.0f) << sign_bit_pos(4 * q + 2);
        word |= static_cast<uint32_t>(v.w < 0.0f) << sign_bit_pos(4 * q + 3);
      }
    } else if (row < n) {
      for (int c = 0; c < 32; ++c)
        if (k0 + c < k) word |= static_cast<uint32_t>(w[row * k + k0 + c] < 0.0f) << sign_bit_pos(c);
    }
    packed[bin_word_index(row, cw, bt)] = word;
  }
}

__global__ __launch_bounds__(kThreads) void unpack_binary_kernel(const uint32_t* __restrict__ packed, int64_t n,
                                                                 int64_t k, int64_t bt,
                                                                 int8_t* __restrict__ codes) {
  const int64_t words_per_row = bt * 16;
  const int64_t total = n * words_per_row;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t row = idx / words_per_row;
    const int64_t cw = idx - row * words_per_row;
    const uint32_t word = packed[bin_word_index(row, cw, bt)];
    const int64_t k0 = cw * 32;
    for (int c = 0; c < 32; ++c)
      if (k0 + c < k) codes[row * k + k0 + c] = ((word >> sign_bit_pos(c)) & 1u) ? int8_t(-1) : int8_t(1);
  }
}

__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint32_t* __restrict__ packed, int64_t n,
                                                          int64_t k, int64_t kt_count,
                                                          int8_t* __restrict__ codes) {
  const int64_t words_per_row = kt_count * 16;
  const int64_t total = n * words_per_row;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t row = idx / words_per_row;
    const int64_t cw = idx - row * words_per_row;
    const int64_t slot = (row & 15) + 16 * ((cw & 15) >> 2);
    const uint32_t word = packed[((row >> 4) * kt_count + (cw >> 4)) * 256 + slot * 4 + (cw & 3)];
    const int64_t k0 = cw * 16;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (k0 + t < k) {
        const int f = static_cast<int>((word >> field_shift(t)) & 3u);
        codes[row * k + k0 + t] = static_cast<int8_t>((f ^ 2) - 2);  // sign-extend (10, never written, -> -2)
      }
    }
  }
}

int grid_for(int64_t items) {
  const int64_t blocks = (items + kThreads - 1) / kThreads;
  return static_cast<int>(blocks < 2048 ? (blocks < 1 ? 1 : blocks) : 2048);
}

}  // namespace

int pack_partial_count(int64_t n, int64_t k) {
  const int64_t total = n * k;
  int64_t parts = (total + 16383) / 16384;
  if (parts < 1) parts = 1;
  if (parts > kPackPartials) parts = kPackPartials;
  return static_cast<int>(parts);
}

hipError_t launch_pack(const float* w, int64_t n, int64_t k, void* packed, float* gamma,
                       double* partials, hipStream_t s) {
  const int64_t total = n * k;
  const int parts = pack_partial_count(n, k);
  const int64_t per_part = split_per_part(total, parts);
  const bool vec = (reinterpret_cast<uintptr_t>(w) % 16 == 0);
  if (vec)
    absmean_partial<true><<<parts, kThreads, 0, s>>>(w, total, per_part, partials);
  else
    absmean_partial<false><<<parts, kThreads, 0, s>>>(w, total, per_part, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t kt = k_tiles(k);
  const int64_t words = row_blocks(n) * kTileRows * kt * 16;
  const bool vec2 = vec && (k % 4 == 0);
  if (vec2)
    ternarize_pack<true><<<grid_for(words), kThreads, 0, s>>>(w, n, k, kt, partials, parts, gamma,
                                                               static_cast<uint32_t*>(packed));
  else
    ternarize_pack<false><<<grid_for(words), kThreads, 0, s>>>(w, n, k, kt, partials, parts, gamma,
                                                                static_cast<uint32_t*>(packed));
  return hipGetLastError();
}

// Device address of `scratch` on each GPU, looked up once per device with
// that device current (the host-side name is not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};

hipError_t pack_scratch(double** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<double*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_pack_noalloc(const float* w, int64_t n, int64_t k, void* packed, float* gamma, hipStream_t s) {
  if (pack_partial_count(n, k) > kPackPartials) return hipErrorInvalidValue;  // never for accepted shapes
  double* partials = nullptr;
  const hipError_t e = pack_scratch(&partials);
  if (e != hipSuccess) return e;
  return launch_pack(w, n, k, packed, gamma, partials, s);
}

hipError_t launch_pack_rowscale(const float* w, int64_t n, int64_t k, void* packed, uint16_t* scales, hipStream_t s) {
  row_scale_kernel<<<static_cast<unsigned>((n + kWaves - 1) / kWaves), kThreads, 0, s>>>(w, n, k, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t kt = k_tiles(k);
  const int64_t words = row_blocks(n) * kTileRows * kt * 16;
  const bool vec = (reinterpret_cast<uintptr_t>(w) % 16 == 0) && (k % 4 == 0);
  if (vec)
    ternarize_pack_rows<true><<<grid_for(words), kThreads, 0, s>>>(w, n, k, kt, scales, static_cast<uint32_t*>(packed));
  else
    ternarize_pack_rows<false><<<grid_for(words), kThreads, 0, s>>>(w, n, k, kt, scales, static_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_pack_binary(const float* w, int64_t n, int64_t k, void* packed, hipStream_t s) {
  const int64_t bt = bin_tiles(k);
  const int64_t words = row_blocks(n) * kTileRows * bt * 16;
  const bool vec = (reinterpret_cast<uintptr_t>(w) % 16 == 0) && (k % 4 == 0);
  if (vec)
    pack_binary_kernel<true><<<grid_for(words), kThreads, 0, s>>>(w, n, k, bt, static_cast<uint32_t*>(packed));
  else
    pack_binary_kernel<false><<<grid_for(words), kThreads, 0, s>>>(w, n, k, bt, static_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack_binary(const void* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t s) {
  const int64_t bt = bin_tiles(k);
  unpack_binary_kernel<<<grid_for(n * bt * 16), kThreads, 0, s>>>(static_cast<const uint32_t*>(packed), n, k, bt,
                                                                  codes);
  return hipGetLastError();
}

hipError_t launch_unpack(const void* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t s) {
  const int64_t kt = k_tiles(k);
  unpack_kernel<<<grid_for(n * kt * 16), kThreads, 0, s>>>(static_cast<const uint32_t*>(packed), n, k, kt,
                                                          codes);
  return hipGetLastError();
}

}  // namespace bitlinear
