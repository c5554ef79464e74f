// Batched (prefill) BitLinear forward for any token count.
//
// "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
// "The Mathematical Mechanism", items 3-4 (ternary x int8 contraction in
// int32, de-quantisation by gamma * a' / 127).  With many tokens per weight
// the contraction is dense and compute-bound ("BitNet 1-bit LLM Inference
// Framework", section "Scalability with Thread Count": prompt processing is
// compute-intensive), so it runs on the int8 matrix cores.
//
// Tiling: a workgroup of 4 waves (2 x 2) owns a BM x BN output tile (tokens x
// weight rows) and walks k in 256-column steps.  Per step it copies the BM x
// 256 int8 activation tile and the BN/16 packed weight tiles (1 KiB each,
// copied verbatim -- still 2 bits per weight) into LDS; the next step's
// global loads are issued into registers before the current step's math, so
// HBM/L2 latency overlaps the matrix-core work.  Each wave expands its packed
// weight slots to int8 in registers -- one shift and one mask per 4 weights,
// done once per slot and reused by every token block of the wave -- and runs
// v_mfma_i32_16x16x64_i8 on (16 tokens x 64 cols) x (64 cols x 16 rows).
// The stored weight is w + 1; the per-token sum of x_q that this offset adds
// is accumulated exactly with v_dot4 while the activation tile passes
// through registers on its way to LDS, and subtracted in the epilogue.
#include "bitlinear_internal.hpp"

namespace bitlinear {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kAStride = kTileCols + 16;  // LDS row pitch of the activation tile (bytes)

__device__ __forceinline__ v4i expand(uint32_t word) {
  return v4i{static_cast<int>(word & 0x03030303u), static_cast<int>((word >> 2) & 0x03030303u),
             static_cast<int>((word >> 4) & 0x03030303u), static_cast<int>((word >> 6) & 0x03030303u)};
}

__device__ __forceinline__ uint4 load_a16(const int8_t* __restrict__ xq, int64_t row, int64_t col, int64_t m,
                                          int64_t k, bool vec) {
  uint4 r = make_uint4(0, 0, 0, 0);
  if (row >= m) return r;
  const int8_t* p = xq + row * k + col;
  if (vec) {
    if (col < k) r = *reinterpret_cast<const uint4*>(p);
  } else {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 16; ++b)
      if (col + b < k) w[b >> 2] |= static_cast<uint32_t>(static_cast<uint8_t>(p[b])) << (8 * (b & 3));
    r = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return r;
}

template <int BM, int BN, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const uint4* __restrict__ packed,
                                                           const float* __restrict__ gamma_p, int64_t n,
                                                           int64_t k, int kt_count,
                                                           const int8_t* __restrict__ xq,
                                                           const float* __restrict__ amax, int64_t m,
                                                           float* __restrict__ y, int32_t* __restrict__ acc_out) {
  constexpr int MB = BM / 32;                 // 16-token blocks per wave
  constexpr int NB = BN / 32;                 // 16-row blocks per wave
  constexpr int A_PER_THREAD = BM * 16 / kThreads;
  constexpr int B_CHUNKS = (BN / 16) * 64;
  constexpr int B_PER_THREAD = B_CHUNKS / kThreads;
  static_assert(A_PER_THREAD >= 1 && B_PER_THREAD >= 1, "tile too small for the workgroup");

  __shared__ __attribute__((aligned(16))) int8_t As[BM * kAStride];
  __shared__ uint4 Bs[B_CHUNKS];
  __shared__ int rowsum_s[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t rb0 = n0 / kTileRows;
  const int64_t rb_count = row_blocks(n);

  uint4 areg[A_PER_THREAD];
  uint4 breg[B_PER_THREAD];
  int rsum[A_PER_THREAD];
#pragma unroll
  for (int i = 0; i < A_PER_THREAD; ++i) rsum[i] = 0;

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) {
      const int c = tid + kThreads * i;
      areg[i] = load_a16(xq, m0 + (c >> 4), static_cast<int64_t>(kt) * kTileCols + (c & 15) * 16, m, k, VEC);
    }
#pragma unroll
    for (int i = 0; i < B_PER_THREAD; ++i) {
      const int c = tid + kThreads * i;
      const int64_t rbg = rb0 + (c >> 6);
      breg[i] = rbg < rb_count ? packed[(rbg * kt_count + kt) * 64 + (c & 63)]
                               : make_uint4(kZeroWord, kZeroWord, kZeroWord, kZeroWord);
    }
  };

  v4i acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  load_tile(0);
  for (int kt = 0; kt < kt_count; ++kt) {
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<uint4*>(As + (c >> 4) * kAStride + (c & 15) * 16) = areg[i];
      int s = rsum[i];
      s = __builtin_amdgcn_sdot4(static_cast<int>(areg[i].x), 0x01010101, s, false);
      s = __builtin_amdgcn_sdot4(static_cast<int>(areg[i].y), 0x01010101, s, false);
      s = __builtin_amdgcn_sdot4(static_cast<int>(areg[i].z), 0x01010101, s, false);
      s = __builtin_amdgcn_sdot4(static_cast<int>(areg[i].w), 0x01010101, s, false);
      rsum[i] = s;
    }
#pragma unroll
    for (int i = 0; i < B_PER_THREAD; ++i) Bs[tid + kThreads * i] = breg[i];
    __syncthreads();
    if (kt + 1 < kt_count) load_tile(kt + 1);

    v4i b[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint4 w = Bs[(wn * NB + nb) * 64 + lane];
      b[nb][0] = expand(w.x);
      b[nb][1] = expand(w.y);
      b[nb][2] = expand(w.z);
      b[nb][3] = expand(w.w);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const v4i a = *reinterpret_cast<const v4i*>(As + (wm * (BM / 2) + mb * 16 + l16) * kAStride + g * 64 + s * 16);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[nb][s], acc[mb][nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // per-token sums of x_q: the 16 threads of one token row are 16 consecutive lanes
#pragma unroll
  for (int i = 0; i < A_PER_THREAD; ++i) {
    int v = rsum[i];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    if ((tid & 15) == 0) rowsum_s[(tid >> 4) + 16 * i] = v;
  }
  __syncthreads();

  const float gamma = *gamma_p;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = wm * (BM / 2) + mb * 16 + 4 * g + r;
      const int64_t t = m0 + tl;
      if (t >= m) continue;
      const float scale = gamma * amax[t] / 127.0f;
      const int rs = rowsum_s[tl];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t j = n0 + wn * (BN / 2) + nb * 16 + l16;
        if (j < n) {
          const int v = acc[mb][nb][r] - rs;
          y[t * n + j] = static_cast<float>(v) * scale;
          if (acc_out) acc_out[t * n + j] = v;
        }
      }
    }
  }
}

template <int BM, int BN>
hipError_t launch(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                  const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s, bool vec) {
  const int kt = static_cast<int>(k_tiles(k));
  const dim3 grid(static_cast<unsigned>((n + BN - 1) / BN), static_cast<unsigned>((m + BM - 1) / BM));
  const uint4* p = static_cast<const uint4*>(packed);
  if (vec)
    gemm_kernel<BM, BN, true><<<grid, kThreads, 0, s>>>(p, gamma, n, k, kt, xq, amax, m, y, acc);
  else
    gemm_kernel<BM, BN, false><<<grid, kThreads, 0, s>>>(p, gamma, n, k, kt, xq, amax, m, y, acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                       const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  const bool vec = (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
  if (m <= 64) {
    const int64_t tiles128 = (n + 127) / 128;
    if (tiles128 >= 512) return launch<64, 128>(packed, gamma, n, k, xq, amax, m, y, acc, s, vec);
    return launch<64, 64>(packed, gamma, n, k, xq, amax, m, y, acc, s, vec);
  }
  const int64_t mt = (m + 127) / 128;
  if (((n + 127) / 128) * mt >= 512) return launch<128, 128>(packed, gamma, n, k, xq, amax, m, y, acc, s, vec);
  return launch<128, 64>(packed, gamma, n, k, xq, amax, m, y, acc, s, vec);
}

}  // namespace bitlinear
