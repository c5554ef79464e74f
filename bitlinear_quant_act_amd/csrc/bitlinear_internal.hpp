// Internal declarations of libbitlinear.so: device layout constants and the
// kernel launchers the C ABI (api.hip) dispatches to.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitlinear {

// ---- packed ternary layout, version 2 -------------------------------------
// A tile is 16 weight rows x 256 columns = 1024 bytes: 64 slots of 16 bytes,
// one per lane of a wave64, so a wave reads a tile with one fully coalesced
// 16-byte-per-lane load.  Slot l: row (l % 16), columns 64*(l/16) + [0, 64).
// Word s of a slot: 16 columns, column t at bits 8*(t%4) + 2*(t/4).  Each
// 2-bit field holds w in two's complement (00 = 0, 01 = +1, 11 = -1; 10 is
// never written), so (word << (6 - 2j)) & 0xC0C0C0C0 yields columns
// 4j..4j+3 in order as four int8 bytes equal to 64 * w.
constexpr int kTileRows = 16;
constexpr int kTileCols = 256;
constexpr int kTileBytes = 1024;
constexpr uint32_t kZeroCode = 0u;  // w = 0
constexpr uint32_t kZeroWord = 0u;  // sixteen zero weights
constexpr int kWeightShift = 6;     // expanded weight bytes are 64 * w

// ---- packed binary layout (sign bits, one per weight) ----------------------
// A binary tile is 16 rows x 512 columns = 1024 bytes: 64 slots of 16 bytes,
// one per lane, so a wave reads a tile with one coalesced 16-byte-per-lane
// load, as for the ternary tiles.  Slot l: row (l % 16), columns
// 128*(l/16) + [0, 128); word s (0..3) of a slot covers 32 of them, column c
// at bit 8*(c%4) + 7 - c/4, set for -1 and clear for +1.  Then
// ((word << i) & 0x80808080) | 0x40404040 yields columns 4i..4i+3 in order as
// four int8 bytes equal to 64 * w, the ternary expansion's scale.  The
// 256-column halves of a tile are contiguous (slots 0-31, then 32-63), so a
// matrix-core k-step of 256 columns reads 512 bytes per row block.
constexpr int kBinTileCols = 512;
constexpr int kBinTileBytes = 1024;
constexpr int kBinStepBytes = 512;  // one 256-column half of a binary tile

__host__ __device__ inline int64_t bin_tiles(int64_t k) { return (k + kBinTileCols - 1) / kBinTileCols; }

__host__ __device__ inline int64_t row_blocks(int64_t n) { return (n + kTileRows - 1) / kTileRows; }
__host__ __device__ inline int64_t k_tiles(int64_t k) { return (k + kTileCols - 1) / kTileCols; }

// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// accesses (lgkmcnt), not for its outstanding global loads.  __syncthreads()
// carries a release fence that also drains every vector-memory load, which
// would stall a kernel that keeps weight tiles in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-wide reductions on DPP row operations (register moves, no trip through
// the LDS unit): an inclusive scan inside each row of 16 lanes (row_shr 1, 2,
// 4, 8), then the row totals carried across rows (row_bcast 15 into rows 1
// and 3, row_bcast 31 into rows 2 and 3); lane 63 ends with the result, which
// is returned to every lane.  Lanes without a source keep the identity.
#define BITLINEAR_DPP_MAX(V, CTRL, ROWS) \
  V = max(V, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(V), static_cast<int>(V), CTRL, ROWS, 0xf, false)))

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  BITLINEAR_DPP_MAX(v, 0x111, 0xf);  // row_shr:1
  BITLINEAR_DPP_MAX(v, 0x112, 0xf);  // row_shr:2
  BITLINEAR_DPP_MAX(v, 0x114, 0xf);  // row_shr:4
  BITLINEAR_DPP_MAX(v, 0x118, 0xf);  // row_shr:8
  BITLINEAR_DPP_MAX(v, 0x142, 0xa);  // row_bcast:15 into rows 1, 3
  BITLINEAR_DPP_MAX(v, 0x143, 0xc);  // row_bcast:31 into rows 2, 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
#undef BITLINEAR_DPP_MAX

// one scan step of a 64-bit value: lanes without a source add 0
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_add_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, ROWS, 0xf, false);
  return v + __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                                        static_cast<uint32_t>(lo)));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v = dpp_add_f64<0x111, 0xf>(v);
  v = dpp_add_f64<0x112, 0xf>(v);
  v = dpp_add_f64<0x114, 0xf>(v);
  v = dpp_add_f64<0x118, 0xf>(v);
  v = dpp_add_f64<0x142, 0xa>(v);
  v = dpp_add_f64<0x143, 0xc>(v);
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), 63));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// 16-byte streaming load of packed weights: read once, so marked
// non-temporal to keep them from displacing reused data in the caches.
__device__ __forceinline__ uint4 load_weights_nt(const uint4* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// One packed word (16 weights) -> the 16-byte int8 operand 64 * w of one
// 16x16x64 MFMA, columns in order: three shifts and four masks.
typedef int expand_v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ expand_v4i expand_ternary(uint32_t word) {
  const uint32_t m = 0xC0C0C0C0u;
  return expand_v4i{static_cast<int>((word << 6) & m), static_cast<int>((word << 4) & m),
                    static_cast<int>((word << 2) & m), static_cast<int>(word & m)};
}

// Half o (columns 16o .. 16o+15) of a binary word -> the 16-byte int8
// operand 64 * w, columns in order: one shift and one and-or per 4 weights.
__device__ __forceinline__ expand_v4i expand_binary(uint32_t word, int o) {
  const int i0 = 4 * o;
  return expand_v4i{static_cast<int>(((word << i0) & 0x80808080u) | 0x40404040u),
                    static_cast<int>(((word << (i0 + 1)) & 0x80808080u) | 0x40404040u),
                    static_cast<int>(((word << (i0 + 2)) & 0x80808080u) | 0x40404040u),
                    static_cast<int>(((word << (i0 + 3)) & 0x80808080u) | 0x40404040u)};
}

// Scales of one token for RMSNorm folded into the absmax quantisation.
// RMSNorm scales the token by r = 1 / sqrt(mean x^2 + eps) and channel c by
// the gain w_c; the absmax rule is then applied to the normalised token,
// whose maximum is about av * r with av = max_c |x_c * w_c|.  Absmax
// quantisation is invariant under the positive factor r, so the codes are
// taken from v = x * w directly:
//   - max|x_norm| = fl32(av * r) at or above the 1e-8 floor: scale 127 / av
//     on v, and a' = fl32(av * r) for the de-quantisation;
//   - below the floor (a tiny token or gain): the floor is the token's
//     scale, so v is scaled by r * 127 / 1e-8 (binary64, rounded once, kept
//     finite) and a' = 1e-8.  An all-zero v gets codes 0.
// The codes equal those of the normalised token except where the value lies
// within a few roundings of a tie.
__device__ __forceinline__ void rmsnorm_scales(float av, double r, float* amax_dst, float* quant_dst) {
  const float ap = static_cast<float>(static_cast<double>(av) * r);
  if (ap >= 1e-8f) {  // false for NaN (av = 0 with r = inf)
    *amax_dst = ap;
    *quant_dst = 127.0f / av;
  } else {
    *amax_dst = 1e-8f;
    *quant_dst = fminf(static_cast<float>(r * (127.0 / static_cast<double>(1e-8f))), 3.40282347e+38f);
  }
}

// binary16 bit pattern -> binary32 (exact)
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// How the forward kernels turn an int32 accumulator into y:
//   y[t][j] = acc * (w_scale * a[t * astride] / qdiv)
// w_scale is the tensor's gamma, or the binary16 scale of row j when
// row_scale is set.  The main path: per-token a', qdiv 127.  The per-tensor
// activation variant: one a (astride 0), qdiv 128.
struct Dequant {
  const uint16_t* row_scale;
  float qdiv;
  int astride;
};
constexpr Dequant kTokenDequant = {nullptr, 127.0f, 1};

constexpr int kPackPartials = 1024;  // fp64 partial sums of |W| (max)

// ---- launchers (return the hipGetLastError of their launches) --------------
hipError_t launch_rmsnorm_quant_act(const uint16_t* x, const float* gain, float eps, int64_t m, int64_t k, int8_t* xq,
                                    float* amax, hipStream_t s);
hipError_t launch_quant_act_f32(const float* x, int64_t m, int64_t k, int8_t* xq, float* amax, hipStream_t s);
hipError_t launch_norm_quant_gemv(const void* packed, const float* gamma, int64_t n, int64_t k, const uint16_t* x,
                                  const float* gain, float eps, int64_t m, float* y, int32_t* acc, int8_t* xq_out,
                                  float* amax_out, hipStream_t s);
hipError_t launch_gemv_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u, const float* gamma_u,
                              int64_t f, int64_t k, const int8_t* xq, const float* amax, int64_t m, float* h,
                              int32_t* acc, hipStream_t s);
hipError_t launch_norm_quant_gemv_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u,
                                         const float* gamma_u, int64_t f, int64_t k, const uint16_t* x,
                                         const float* gain, float eps, int64_t m, float* h, int32_t* acc,
                                         int8_t* xq_out, float* amax_out, hipStream_t s);
hipError_t launch_quant_gemv_f32(const void* packed, const float* gamma, int64_t n, int64_t k, const float* x,
                                 int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out, hipStream_t s);
bool gemv_lut_supported(int64_t k);
hipError_t launch_gemv_lut(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                           const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s);
bool gemm_swiglu_supported(int64_t k, const int8_t* xq);
hipError_t launch_gemm_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u, const float* gamma_u,
                              int64_t f, int64_t k, const int8_t* xq, const float* amax, int64_t m, float* h,
                              int32_t* acc, hipStream_t s);
hipError_t launch_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* amax,
                            hipStream_t s);

int pack_partial_count(int64_t n, int64_t k);
hipError_t launch_pack(const float* w, int64_t n, int64_t k, void* packed, float* gamma,
                       double* partials, hipStream_t s);
hipError_t launch_pack_noalloc(const float* w, int64_t n, int64_t k, void* packed, float* gamma, hipStream_t s);
hipError_t launch_unpack(const void* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t s);

hipError_t launch_gemv(const void* packed, const float* gamma, int64_t n, int64_t k,
                       const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc,
                       hipStream_t s);
bool gemv_fits_lds(int64_t m, int64_t k);
hipError_t launch_quant_gemv(const void* packed, const float* gamma, int64_t n, int64_t k, const uint16_t* x,
                             int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out, hipStream_t s);
hipError_t launch_gemm(const void* packed, const float* gamma, int64_t n, int64_t k,
                       const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc,
                       hipStream_t s);

// ---- variant modes ------------------------------------------------------------
// forward with a de-quantization mode and a weight format (binary: sign-bit tiles)
hipError_t launch_gemv_ex(const void* packed, bool binary, const float* gamma, Dequant dq, int64_t n, int64_t k,
                          const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s);
hipError_t launch_quant_gemv_binary(const void* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                                    int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out, hipStream_t s);
bool gemv_binary_fits_lds(int64_t m, int64_t k);
hipError_t launch_gemm_ex(const void* packed, bool binary, const float* gamma, Dequant dq, int64_t n, int64_t k,
                          const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s);
int quant_tensor_partial_count(int64_t m, int64_t k);
hipError_t launch_quant_act_tensor(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* gx,
                                   uint32_t* partials, hipStream_t s);
hipError_t launch_pack_rowscale(const float* w, int64_t n, int64_t k, void* packed, uint16_t* scales, hipStream_t s);
hipError_t launch_pack_binary(const float* w, int64_t n, int64_t k, void* packed, hipStream_t s);
hipError_t launch_unpack_binary(const void* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t s);

}  // namespace bitlinear
