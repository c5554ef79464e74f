// Decode-path BitLinear forward for 1..16 tokens.
//
// "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
// "The Mathematical Mechanism", items 3-4: acc = sum_k x_q * W_q with
// W_q in {-1, 0, +1} (adds and subtracts only), then y = acc * gamma * a' / 127.
// "BitNet 1-bit LLM Inference Framework", section "Scalability with Thread
// Count": generation is bound by memory bandwidth, so the kernel is built to
// stream the 2-bit weights from HBM exactly once at full width.
//
// Work split: one workgroup per 16-row block of W; its waves take the block's
// 256-column tiles round-robin (wave w: tiles w, w + WAVES, ...), so at any
// moment the workgroup reads consecutive KiB of one contiguous stream.  Each
// wave issues U tile loads (16 B per lane, fully coalesced 1 KiB per wave)
// before it consumes any, to keep enough bytes in flight.
//
// Contraction on the matrix cores, not a dot-product loop: one
// v_mfma_i32_16x16x64_i8 takes 16 tokens x 64 columns of int8 activations
// (A; rows >= m are zero) and 64 columns x 16 weight rows (B).  The B operand
// of a lane is exactly one 32-bit word of its packed slot expanded with one
// shift and one mask per 4 weights: (word >> 2j) & 0x03030303 gives the
// stored values w + 1 in {0, 1, 2} as int8.  The offset is removed exactly
// with a second MFMA against an all-ones B (sum_k x), which runs on the
// otherwise idle matrix pipe:  acc = sum (w + 1) x - sum x.  Both sums are
// exact int32.  The activation operand of a lane is the 16 bytes of its own
// token at the same 16 columns, so the k order inside the instruction is the
// same for A and B and needs no shuffling.
//
// Epilogue: the waves' int32 partials are summed through LDS and scaled by
// gamma * a'[m] / 127 in fp32; lanes 0..15 of a result row write 16
// consecutive floats.
#include "bitlinear_internal.hpp"

namespace bitlinear {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i load_x16(const int8_t* __restrict__ row, int64_t col, int64_t k, bool valid,
                                        bool vec) {
  v4i r = {0, 0, 0, 0};
  if (!valid) return r;
  if (vec) {
    if (col < k) r = *reinterpret_cast<const v4i*>(row + col);
  } else {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 16; ++b)
      if (col + b < k) w[b >> 2] |= (static_cast<uint32_t>(static_cast<uint8_t>(row[col + b]))) << (8 * (b & 3));
    r = v4i{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]), static_cast<int>(w[3])};
  }
  return r;
}

__device__ __forceinline__ v4i expand(uint32_t word) {
  return v4i{static_cast<int>(word & 0x03030303u), static_cast<int>((word >> 2) & 0x03030303u),
             static_cast<int>((word >> 4) & 0x03030303u), static_cast<int>((word >> 6) & 0x03030303u)};
}

template <int WAVES, int U, bool VEC>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(const uint4* __restrict__ packed,
                                                          const float* __restrict__ gamma_p, int64_t n,
                                                          int64_t k, int kt_count,
                                                          const int8_t* __restrict__ xq,
                                                          const float* __restrict__ amax, int m,
                                                          float* __restrict__ y, int32_t* __restrict__ acc_out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t rb = blockIdx.x;
  const int g = lane >> 4;    // 64-column group of the lane inside a tile
  const int tok = lane & 15;  // token row of the lane's A operand
  const bool has_tok = tok < m;
  const uint4* tiles = packed + rb * kt_count * 64 + lane;
  const int8_t* xrow = xq + static_cast<int64_t>(has_tok ? tok : 0) * k;
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  v4i acc = {0, 0, 0, 0};
  v4i sum = {0, 0, 0, 0};
  for (int kt0 = wave; kt0 < kt_count; kt0 += WAVES * U) {
    uint4 wv[U];
    v4i xv[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = kt0 + u * WAVES;
      const bool in = kt < kt_count;
      wv[u] = in ? tiles[static_cast<int64_t>(kt) * 64] : make_uint4(kZeroWord, kZeroWord, kZeroWord, kZeroWord);
      const int64_t c0 = static_cast<int64_t>(kt) * kTileCols + g * 64;
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[u][s] = load_x16(xrow, c0 + 16 * s, k, in && has_tok, VEC);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t words[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(xv[u][s], expand(words[s]), acc, 0, 0, 0);
        sum = __builtin_amdgcn_mfma_i32_16x16x64_i8(xv[u][s], ones, sum, 0, 0, 0);
      }
    }
  }
  // lane holds tokens 4g + r (r = 0..3) for weight row 16 rb + (lane % 16)
  v4i res = acc - sum;

  const int64_t row = rb * kTileRows + tok;
  const float gamma = *gamma_p;
  if (WAVES == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * g + r;
      if (t < m && row < n) {
        const float scale = gamma * amax[t] / 127.0f;
        y[t * n + row] = static_cast<float>(res[r]) * scale;
        if (acc_out) acc_out[t * n + row] = res[r];
      }
    }
    return;
  }
  __shared__ int red[WAVES][4][64];
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = res[r];
  __syncthreads();
  for (int r = wave; r < 4; r += WAVES) {
    int v = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][r][lane];
    const int t = 4 * g + r;
    if (t < m && row < n) {
      const float scale = gamma * amax[t] / 127.0f;
      y[t * n + row] = static_cast<float>(v) * scale;
      if (acc_out) acc_out[t * n + row] = v;
    }
  }
}

template <int WAVES, int U>
hipError_t launch(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                  const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s, bool vec) {
  const int kt = static_cast<int>(k_tiles(k));
  const dim3 grid(static_cast<unsigned>(row_blocks(n)));
  const uint4* p = static_cast<const uint4*>(packed);
  if (vec)
    gemv_kernel<WAVES, U, true><<<grid, WAVES * 64, 0, s>>>(p, gamma, n, k, kt, xq, amax, static_cast<int>(m), y, acc);
  else
    gemv_kernel<WAVES, U, false><<<grid, WAVES * 64, 0, s>>>(p, gamma, n, k, kt, xq, amax, static_cast<int>(m), y, acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                       const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  const bool vec = (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
  const int64_t kt = k_tiles(k);
  if (kt <= 1) return launch<1, 1>(packed, gamma, n, k, xq, amax, m, y, acc, s, vec);
  if (kt <= 4) return launch<4, 1>(packed, gamma, n, k, xq, amax, m, y, acc, s, vec);
  return launch<4, 4>(packed, gamma, n, k, xq, amax, m, y, acc, s, vec);
}

}  // namespace bitlinear
