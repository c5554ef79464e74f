// Table-lookup decode forward: the lookup-table formulation of the ternary
// contraction ("BitNet 1-bit LLM Inference Framework", section "How the LUT
// Kernel Works": because every weight is -1, 0 or +1, the product with a
// group of activations takes one of a few values, which can be precomputed and
// looked up instead of multiplied), re-expressed for on-chip memory.
//
// Groups of two weights: the packed layout holds a weight pair in every 4-bit
// nibble (nibble j of a 32-bit word covers columns b + 8h and b + 8h + 4 of the
// word's 16, b = j / 2, h = j % 2), so each workgroup first builds, in LDS,
// the 16 signed partial sums
//   T[word][j][u] = w(u % 4) * x[c0] + w(u / 4) * x[c1],  w = two's-complement field
// for every 16-column word of its token's row (16 int16 per nibble, 16 * K
// bytes in all), then streams the packed weights in the same order as the
// matrix-core kernel and adds one table entry per nibble.  The sums are exact
// integers, so the result equals the matrix-core kernel's bit for bit.
//
// Workgroups are persistent (as many as the table lets reside on the chip),
// so each table is built once and serves many 16-row blocks.  Token t of m is
// handled by grid row t, which builds its own table and streams the weights
// again: the variant is meant for m = 1.
//
// Cost per two weights: a nibble extract, an LDS address, an LDS read and an
// add -- against about 0.44 ALU operations per weight for the register
// expansion feeding the matrix cores.  It is kept as the measured comparison
// of the two formulations.
#include <algorithm>

#include "bitlinear_internal.hpp"

namespace bitlinear {
namespace {

constexpr int kLutWaves = 8;
constexpr int kLutThreads = kLutWaves * 64;

__device__ __forceinline__ int sext2(uint32_t f) { return static_cast<int>(f << 30) >> 30; }

template <int U>
__global__ __launch_bounds__(kLutThreads) void gemv_lut_kernel(const uint4* __restrict__ packed,
                                                               const float* __restrict__ gamma_p, int64_t n, int k,
                                                               int kt_count, int64_t rb_count,
                                                               const int8_t* __restrict__ xq,
                                                               const float* __restrict__ amax, float* __restrict__ y,
                                                               int32_t* __restrict__ acc_out) {
  extern __shared__ __attribute__((aligned(16))) int16_t table[];  // [kt_count * 16 words][8 nibbles][16]
  __shared__ int red[kLutWaves * 64];  // per-lane sums at the end of a row block
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // the first weight tiles are requested before the table is built
  int64_t rb = blockIdx.x;
  uint4 wcur[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kt = wave + u * kLutWaves;
    wcur[u] = (rb < rb_count && kt < kt_count) ? load_weights_nt(packed + (rb * kt_count + kt) * 64 + lane)
                                               : make_uint4(0, 0, 0, 0);
  }

  // table: the 16 sums of nibble j of word `word` sit at entry
  // 128 * word + 16 * ((j + g) % 8), g = (word / 4) % 4 the 64-column group,
  // so the four groups a wave reads at once fall in different LDS banks;
  // columns past k read as 0
  const int8_t* xt = xq + static_cast<int64_t>(blockIdx.y) * k;
  for (int p = threadIdx.x; p < kt_count * 128; p += kLutThreads) {
    const int j = p & 7, word = p >> 3;
    const int col = (word >> 4) * kTileCols + ((word >> 2) & 3) * 64 + (word & 3) * 16 + (j >> 1) + 8 * (j & 1);
    const int x0 = col < k ? xt[col] : 0;
    const int x1 = col + 4 < k ? xt[col + 4] : 0;
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u0 = 2 * i, u1 = 2 * i + 1;
      const int t0 = sext2(u0 & 3) * x0 + sext2(u0 >> 2) * x1;
      const int t1 = sext2(u1 & 3) * x0 + sext2(u1 >> 2) * x1;
      v[i] = (static_cast<uint32_t>(t0) & 0xFFFFu) | (static_cast<uint32_t>(t1) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(table + word * 128 + ((j + ((word >> 2) & 3)) & 7) * 16);
    dst[0] = make_uint4(v[0], v[1], v[2], v[3]);
    dst[1] = make_uint4(v[4], v[5], v[6], v[7]);
  }
  lds_barrier();

  const float scale = *gamma_p * amax[blockIdx.y] / 127.0f;
  const int g = lane >> 4;  // 64-column group of the lane's slot
  int seg[8];               // entry offset of nibble j inside a word's 128
#pragma unroll
  for (int j = 0; j < 8; ++j) seg[j] = ((j + g) & 7) * 16;
  const int nchunks = (kt_count + U * kLutWaves - 1) / (U * kLutWaves);
  int c = 0;
  int acc = 0;
  while (rb < rb_count) {
    int64_t rbn = rb;
    int cn = c + 1;
    if (cn == nchunks) {
      cn = 0;
      rbn = rb + gridDim.x;
    }
    uint4 wnext[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = cn * U * kLutWaves + wave + u * kLutWaves;
      wnext[u] = (rbn < rb_count && kt < kt_count) ? load_weights_nt(packed + (rbn * kt_count + kt) * 64 + lane)
                                                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = c * U * kLutWaves + wave + u * kLutWaves;
      if (kt < kt_count) {
        const uint32_t words[4] = {wcur[u].x, wcur[u].y, wcur[u].z, wcur[u].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int16_t* t = table + (kt * 16 + g * 4 + s) * 128;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc += t[seg[j] + ((words[s] >> (4 * j)) & 15)];
        }
      }
    }
    if (c == nchunks - 1) {
      // lanes l, l + 16, l + 32, l + 48 hold parts of row 16 rb + l % 16
      red[wave * 64 + lane] = acc;
      lds_barrier();
      if (wave == 0 && lane < 16) {
        int v = 0;
#pragma unroll
        for (int w = 0; w < kLutWaves; ++w)
#pragma unroll
          for (int q = 0; q < 4; ++q) v += red[w * 64 + q * 16 + lane];
        const int64_t row = rb * kTileRows + lane;
        if (row < n) {
          const int64_t o = static_cast<int64_t>(blockIdx.y) * n + row;
          y[o] = static_cast<float>(v) * scale;
          if (acc_out) acc_out[o] = v;
        }
      }
      lds_barrier();
      acc = 0;
    }
    rb = rbn;
    c = cn;
#pragma unroll
    for (int u = 0; u < U; ++u) wcur[u] = wnext[u];
  }
}

constexpr int kLdsBytes = 160 * 1024;
constexpr int kStaticLds = kLutWaves * 64 * 4;
constexpr int kMaxLutBytes = kLdsBytes - kStaticLds;
constexpr int kCus = 256;

__host__ inline size_t lut_bytes(int64_t k) { return static_cast<size_t>(k_tiles(k)) * 128 * sizeof(int16_t) * 16; }

template <int U>
hipError_t launch_lut(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq, const float* amax,
                      int64_t m, float* y, int32_t* acc, hipStream_t s) {
  const int kt = static_cast<int>(k_tiles(k));
  const int64_t rbs = row_blocks(n);
  const size_t lds = lut_bytes(k);
  // workgroups that fit one compute unit's LDS, at most 2 (16 waves)
  const int64_t per_cu = std::min<int64_t>(2, kLdsBytes / static_cast<int64_t>(lds + kStaticLds));
  const int64_t groups = std::min<int64_t>(rbs, kCus * std::max<int64_t>(1, per_cu));
  static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_lut_kernel<U>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLutBytes) == hipSuccess;
  if (!attr) return hipErrorInvalidConfiguration;
  gemv_lut_kernel<U><<<dim3(static_cast<unsigned>(groups), static_cast<unsigned>(m)), kLutThreads, lds, s>>>(
      static_cast<const uint4*>(packed), gamma, n, static_cast<int>(k), kt, rbs, xq, amax, y, acc);
  return hipGetLastError();
}

}  // namespace

bool gemv_lut_supported(int64_t k) { return lut_bytes(k) <= static_cast<size_t>(kMaxLutBytes); }

hipError_t launch_gemv_lut(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                           const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  const int64_t kt = k_tiles(k);
  if (kt <= kLutWaves) return launch_lut<1>(packed, gamma, n, k, xq, amax, m, y, acc, s);
  if (kt <= 2 * kLutWaves) return launch_lut<2>(packed, gamma, n, k, xq, amax, m, y, acc, s);
  return launch_lut<4>(packed, gamma, n, k, xq, amax, m, y, acc, s);
}

}  // namespace bitlinear
