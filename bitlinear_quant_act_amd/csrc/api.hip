// C ABI of libbitlinear.so (declared in include/bitlinear.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so an argument error leaves outputs untouched and needs no
// device; then it enqueues its kernels on the caller's stream and returns
// without synchronising.  No device memory is allocated here.
#include "bitlinear.h"
#include <cmath>

#include "bitlinear_internal.hpp"

namespace {

constexpr int64_t kMaxK = int64_t(1) << 18;         // |64 acc| <= 64 * 127 k < 2^31
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxBatchedM = int64_t(1) << 21;  // token tiles fit a grid dimension

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? BITLINEAR_OK : BITLINEAR_E_HIP; }

int check_nk(int64_t n, int64_t k) {
  if (n < 1 || n > kMaxRows || k < 1 || k > kMaxK) return BITLINEAR_E_SHAPE;
  return BITLINEAR_OK;
}

int check_forward(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                  const float* amax, int64_t m, float* y, int32_t* acc) {
  if (!packed || !gamma || !xq || !amax || !y) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (m < 1 || m > kMaxRows) return BITLINEAR_E_SHAPE;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(amax, 4) || !aligned(y, 4) ||
      (acc && !aligned(acc, 4)))
    return BITLINEAR_E_ALIGN;
  return BITLINEAR_OK;
}

// decode kernel for m <= BITLINEAR_FORWARD_MAX_M, matrix-core kernel above
int forward_any(const void* packed, bool binary, const float* gamma, bitlinear::Dequant dq, int64_t n, int64_t k,
                const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc, void* stream) {
  if (m > kMaxBatchedM) return BITLINEAR_E_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (m <= BITLINEAR_FORWARD_MAX_M)
    return status_of(bitlinear::launch_gemv_ex(packed, binary, gamma, dq, n, k, xq, amax, m, y, acc, s));
  return status_of(bitlinear::launch_gemm_ex(packed, binary, gamma, dq, n, k, xq, amax, m, y, acc, s));
}

}  // namespace

extern "C" {

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

const char* bitlinear_status_string(int status) {
  switch (status) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_E_NULL: return "a required pointer is NULL";
    case BITLINEAR_E_SHAPE: return "a size is outside its allowed range";
    case BITLINEAR_E_ALIGN: return "a pointer does not meet its alignment requirement";
    case BITLINEAR_E_UNSUPPORTED: return "valid arguments not handled by this entry point";
    case BITLINEAR_E_SIZE: return "a caller-provided buffer is too small";
    case BITLINEAR_E_HIP: return "the HIP runtime reported a launch error";
    case BITLINEAR_E_VALUE: return "a scalar argument is outside its allowed range";
    default: return "unknown status";
  }
}

size_t bitlinear_packed_bytes(int64_t n, int64_t k) {
  if (check_nk(n, k)) return 0;
  return static_cast<size_t>(bitlinear::row_blocks(n) * bitlinear::k_tiles(k) * bitlinear::kTileBytes);
}

size_t bitlinear_pack_workspace_bytes(int64_t n, int64_t k) {
  if (check_nk(n, k)) return 0;
  return static_cast<size_t>(bitlinear::pack_partial_count(n, k)) * sizeof(double);
}

int bitlinear_pack_weights(const float* w, int64_t n, int64_t k, void* packed, size_t packed_bytes,
                           float* gamma, void* workspace, size_t workspace_bytes, void* stream) {
  if (!w || !packed || !gamma || !workspace) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (!aligned(w, 4) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(workspace, 8))
    return BITLINEAR_E_ALIGN;
  if (packed_bytes < bitlinear_packed_bytes(n, k) || workspace_bytes < bitlinear_pack_workspace_bytes(n, k))
    return BITLINEAR_E_SIZE;
  return status_of(bitlinear::launch_pack(w, n, k, packed, gamma, static_cast<double*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

int bitlinear_pack_weights_noalloc(const float* w, int64_t n, int64_t k, void* packed, size_t packed_bytes,
                                   float* gamma, void* stream) {
  if (!w || !packed || !gamma) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (!aligned(w, 4) || !aligned(packed, 16) || !aligned(gamma, 4)) return BITLINEAR_E_ALIGN;
  if (packed_bytes < bitlinear_packed_bytes(n, k)) return BITLINEAR_E_SIZE;
  if (bitlinear_pack_workspace_bytes(n, k) > BITLINEAR_PACK_NOALLOC_SCRATCH_BYTES) return BITLINEAR_E_SIZE;
  return status_of(bitlinear::launch_pack_noalloc(w, n, k, packed, gamma, static_cast<hipStream_t>(stream)));
}

int bitlinear_unpack_weights(const void* packed, int64_t n, int64_t k, int8_t* codes, void* stream) {
  if (!packed || !codes) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (!aligned(packed, 16)) return BITLINEAR_E_ALIGN;
  return status_of(bitlinear::launch_unpack(packed, n, k, codes, static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* x_absmax, void* stream) {
  if (!x || !xq || !x_absmax) return BITLINEAR_E_NULL;
  if (m < 1 || m > kMaxRows || k < 1 || k > kMaxK) return BITLINEAR_E_SHAPE;
  if (!aligned(x, 2) || !aligned(x_absmax, 4)) return BITLINEAR_E_ALIGN;
  return status_of(bitlinear::launch_quant_act(x, m, k, xq, x_absmax, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                      const float* x_absmax, int64_t m, float* y, int32_t* acc_or_null, void* stream) {
  if (int rc = check_forward(packed, gamma, n, k, xq, x_absmax, m, y, acc_or_null)) return rc;
  if (m > BITLINEAR_FORWARD_MAX_M) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_gemv(packed, gamma, n, k, xq, x_absmax, m, y, acc_or_null,
                                          static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_forward(const void* packed, const float* gamma, int64_t n, int64_t k, const uint16_t* x,
                            int64_t m, float* y, int32_t* acc_or_null, int8_t* xq_or_null, float* x_absmax_or_null,
                            void* stream) {
  if (!packed || !gamma || !x || !y) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (m < 1 || m > kMaxRows) return BITLINEAR_E_SHAPE;
  if ((xq_or_null == nullptr) != (x_absmax_or_null == nullptr)) return BITLINEAR_E_NULL;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(x, 2) || !aligned(y, 4) ||
      (acc_or_null && !aligned(acc_or_null, 4)) || (x_absmax_or_null && !aligned(x_absmax_or_null, 4)))
    return BITLINEAR_E_ALIGN;
  if (m > BITLINEAR_FORWARD_MAX_M || !bitlinear::gemv_fits_lds(m, k)) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_quant_gemv(packed, gamma, n, k, x, m, y, acc_or_null, xq_or_null,
                                                x_absmax_or_null, static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_forward_supported(int64_t m, int64_t k) {
  if (m < 1 || m > BITLINEAR_FORWARD_MAX_M || k < 1 || k > kMaxK) return 0;
  return bitlinear::gemv_fits_lds(m, k) ? 1 : 0;
}

// ---- variant modes ------------------------------------------------------------

size_t bitlinear_quant_act_tensor_workspace_bytes(int64_t m, int64_t k) {
  if (m < 1 || m > kMaxRows || k < 1 || k > kMaxK) return 0;
  const int parts = bitlinear::quant_tensor_partial_count(m, k);
  return static_cast<size_t>(parts > 0 ? parts : 1) * sizeof(uint32_t);
}

int bitlinear_quant_act_tensor(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* x_scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!x || !xq || !x_scale || !workspace) return BITLINEAR_E_NULL;
  if (m < 1 || m > kMaxRows || k < 1 || k > kMaxK) return BITLINEAR_E_SHAPE;
  if (m > (int64_t(1) << 40) / k) return BITLINEAR_E_SHAPE;
  if (!aligned(x, 2) || !aligned(x_scale, 4) || !aligned(workspace, 4)) return BITLINEAR_E_ALIGN;
  if (workspace_bytes < bitlinear_quant_act_tensor_workspace_bytes(m, k)) return BITLINEAR_E_SIZE;
  return status_of(bitlinear::launch_quant_act_tensor(x, m, k, xq, x_scale, static_cast<uint32_t*>(workspace),
                                                      static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_tensor_act(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                                 const float* x_scale, int64_t m, float* y, int32_t* acc_or_null, void* stream) {
  if (int rc = check_forward(packed, gamma, n, k, xq, x_scale, m, y, acc_or_null)) return rc;
  if (k >= kMaxK) return BITLINEAR_E_SHAPE;  // |64 acc| <= 64 * 128 k < 2^31
  const bitlinear::Dequant dq = {nullptr, 128.0f, 0};
  return forward_any(packed, false, gamma, dq, n, k, xq, x_scale, m, y, acc_or_null, stream);
}

int bitlinear_pack_weights_rowscale(const float* w, int64_t n, int64_t k, void* packed, size_t packed_bytes,
                                    uint16_t* scales, void* stream) {
  if (!w || !packed || !scales) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (!aligned(w, 4) || !aligned(packed, 16) || !aligned(scales, 2)) return BITLINEAR_E_ALIGN;
  if (packed_bytes < bitlinear_packed_bytes(n, k)) return BITLINEAR_E_SIZE;
  return status_of(bitlinear::launch_pack_rowscale(w, n, k, packed, scales, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_rowscale(const void* packed, const uint16_t* scales, int64_t n, int64_t k, const int8_t* xq,
                               const float* x_absmax, int64_t m, float* y, int32_t* acc_or_null, void* stream) {
  if (!packed || !scales || !xq || !x_absmax || !y) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (m < 1 || m > kMaxRows) return BITLINEAR_E_SHAPE;
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(x_absmax, 4) || !aligned(y, 4) ||
      (acc_or_null && !aligned(acc_or_null, 4)))
    return BITLINEAR_E_ALIGN;
  const bitlinear::Dequant dq = {scales, 127.0f, 1};
  return forward_any(packed, false, nullptr, dq, n, k, xq, x_absmax, m, y, acc_or_null, stream);
}

size_t bitlinear_packed_bytes_binary(int64_t n, int64_t k) {
  if (check_nk(n, k)) return 0;
  return static_cast<size_t>(bitlinear::row_blocks(n) * bitlinear::bin_tiles(k) * bitlinear::kBinTileBytes);
}

int bitlinear_pack_binary(const float* w, int64_t n, int64_t k, void* packed, size_t packed_bytes, void* stream) {
  if (!w || !packed) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (!aligned(w, 4) || !aligned(packed, 16)) return BITLINEAR_E_ALIGN;
  if (packed_bytes < bitlinear_packed_bytes_binary(n, k)) return BITLINEAR_E_SIZE;
  return status_of(bitlinear::launch_pack_binary(w, n, k, packed, static_cast<hipStream_t>(stream)));
}

int bitlinear_unpack_binary(const void* packed, int64_t n, int64_t k, int8_t* codes, void* stream) {
  if (!packed || !codes) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (!aligned(packed, 16)) return BITLINEAR_E_ALIGN;
  return status_of(bitlinear::launch_unpack_binary(packed, n, k, codes, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_binary(const void* packed, const float* scale, int64_t n, int64_t k, const int8_t* xq,
                             const float* x_absmax, int64_t m, float* y, int32_t* acc_or_null, void* stream) {
  if (int rc = check_forward(packed, scale, n, k, xq, x_absmax, m, y, acc_or_null)) return rc;
  return forward_any(packed, true, scale, bitlinear::kTokenDequant, n, k, xq, x_absmax, m, y, acc_or_null, stream);
}

int bitlinear_quant_forward_binary(const void* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                                   int64_t m, float* y, int32_t* acc_or_null, int8_t* xq_or_null,
                                   float* x_absmax_or_null, void* stream) {
  if (!packed || !scale || !x || !y) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (m < 1 || m > kMaxRows) return BITLINEAR_E_SHAPE;
  if ((xq_or_null == nullptr) != (x_absmax_or_null == nullptr)) return BITLINEAR_E_NULL;
  if (!aligned(packed, 16) || !aligned(scale, 4) || !aligned(x, 2) || !aligned(y, 4) ||
      (acc_or_null && !aligned(acc_or_null, 4)) || (x_absmax_or_null && !aligned(x_absmax_or_null, 4)))
    return BITLINEAR_E_ALIGN;
  if (m > BITLINEAR_FORWARD_MAX_M || !bitlinear::gemv_binary_fits_lds(m, k)) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_quant_gemv_binary(packed, scale, n, k, x, m, y, acc_or_null, xq_or_null,
                                                       x_absmax_or_null, static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_forward_binary_supported(int64_t m, int64_t k) {
  if (m < 1 || m > BITLINEAR_FORWARD_MAX_M || k < 1 || k > kMaxK) return 0;
  return bitlinear::gemv_binary_fits_lds(m, k) ? 1 : 0;
}

int bitlinear_forward_lut(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                          const float* x_absmax, int64_t m, float* y, int32_t* acc_or_null, void* stream) {
  if (int rc = check_forward(packed, gamma, n, k, xq, x_absmax, m, y, acc_or_null)) return rc;
  if (m > BITLINEAR_FORWARD_MAX_M || !bitlinear::gemv_lut_supported(k)) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_gemv_lut(packed, gamma, n, k, xq, x_absmax, m, y, acc_or_null,
                                              static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_lut_supported(int64_t k) {
  if (k < 1 || k > kMaxK) return 0;
  return bitlinear::gemv_lut_supported(k) ? 1 : 0;
}

int bitlinear_forward_batched(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                              const float* x_absmax, int64_t m, float* y, int32_t* acc_or_null, void* stream) {
  if (int rc = check_forward(packed, gamma, n, k, xq, x_absmax, m, y, acc_or_null)) return rc;
  if (m > kMaxBatchedM) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_gemm(packed, gamma, n, k, xq, x_absmax, m, y, acc_or_null,
                                          static_cast<hipStream_t>(stream)));
}

int bitlinear_rmsnorm_quant_act(const uint16_t* x, const float* gain_or_null, float eps, int64_t m, int64_t k,
                                int8_t* xq, float* x_absmax, void* stream) {
  if (!x || !xq || !x_absmax) return BITLINEAR_E_NULL;
  if (m < 1 || m > kMaxRows || k < 1 || k > kMaxK) return BITLINEAR_E_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return BITLINEAR_E_VALUE;
  if (!aligned(x, 2) || !aligned(x_absmax, 4) || (gain_or_null && !aligned(gain_or_null, 4))) return BITLINEAR_E_ALIGN;
  return status_of(bitlinear::launch_rmsnorm_quant_act(x, gain_or_null, eps, m, k, xq, x_absmax,
                                                       static_cast<hipStream_t>(stream)));
}

int bitlinear_rmsnorm_quant_forward(const void* packed, const float* gamma, int64_t n, int64_t k, const uint16_t* x,
                                    const float* gain_or_null, float eps, int64_t m, float* y, int32_t* acc_or_null,
                                    int8_t* xq_or_null, float* x_absmax_or_null, void* stream) {
  if (!packed || !gamma || !x || !y) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (m < 1 || m > kMaxRows) return BITLINEAR_E_SHAPE;
  if ((xq_or_null == nullptr) != (x_absmax_or_null == nullptr)) return BITLINEAR_E_NULL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return BITLINEAR_E_VALUE;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(x, 2) || !aligned(y, 4) ||
      (gain_or_null && !aligned(gain_or_null, 4)) || (acc_or_null && !aligned(acc_or_null, 4)) ||
      (x_absmax_or_null && !aligned(x_absmax_or_null, 4)))
    return BITLINEAR_E_ALIGN;
  if (m > BITLINEAR_FORWARD_MAX_M || !bitlinear::gemv_fits_lds(m, k)) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_norm_quant_gemv(packed, gamma, n, k, x, gain_or_null, eps, m, y, acc_or_null,
                                                     xq_or_null, x_absmax_or_null, static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_act_f32(const float* x, int64_t m, int64_t k, int8_t* xq, float* x_absmax, void* stream) {
  if (!x || !xq || !x_absmax) return BITLINEAR_E_NULL;
  if (m < 1 || m > kMaxRows || k < 1 || k > kMaxK) return BITLINEAR_E_SHAPE;
  if (!aligned(x, 4) || !aligned(x_absmax, 4)) return BITLINEAR_E_ALIGN;
  return status_of(bitlinear::launch_quant_act_f32(x, m, k, xq, x_absmax, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_swiglu(const void* packed_gate, const float* gamma_gate, const void* packed_up,
                             const float* gamma_up, int64_t f, int64_t k, const int8_t* xq, const float* x_absmax,
                             int64_t m, float* h, int32_t* acc_or_null, void* stream) {
  if (!packed_up || !gamma_up) return BITLINEAR_E_NULL;
  if (int rc = check_forward(packed_gate, gamma_gate, f, k, xq, x_absmax, m, h, acc_or_null)) return rc;
  if (!aligned(packed_up, 16) || !aligned(gamma_up, 4)) return BITLINEAR_E_ALIGN;
  if (m > kMaxBatchedM) return BITLINEAR_E_UNSUPPORTED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (m <= BITLINEAR_FORWARD_MAX_M && bitlinear::gemv_fits_lds(m, k))
    return status_of(bitlinear::launch_gemv_swiglu(packed_gate, gamma_gate, packed_up, gamma_up, f, k, xq, x_absmax, m,
                                                   h, acc_or_null, st));
  if (!bitlinear::gemm_swiglu_supported(k, xq)) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_gemm_swiglu(packed_gate, gamma_gate, packed_up, gamma_up, f, k, xq, x_absmax, m,
                                                 h, acc_or_null, st));
}

int bitlinear_rmsnorm_quant_forward_swiglu(const void* packed_gate, const float* gamma_gate, const void* packed_up,
                                           const float* gamma_up, int64_t f, int64_t k, const uint16_t* x,
                                           const float* gain_or_null, float eps, int64_t m, float* h,
                                           int32_t* acc_or_null, int8_t* xq_or_null, float* x_absmax_or_null,
                                           void* stream) {
  if (!packed_gate || !gamma_gate || !packed_up || !gamma_up || !x || !h) return BITLINEAR_E_NULL;
  if (int rc = check_nk(f, k)) return rc;
  if (m < 1 || m > kMaxRows) return BITLINEAR_E_SHAPE;
  if ((xq_or_null == nullptr) != (x_absmax_or_null == nullptr)) return BITLINEAR_E_NULL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return BITLINEAR_E_VALUE;
  if (!aligned(packed_gate, 16) || !aligned(packed_up, 16) || !aligned(gamma_gate, 4) || !aligned(gamma_up, 4) ||
      !aligned(x, 2) || !aligned(h, 4) || (gain_or_null && !aligned(gain_or_null, 4)) ||
      (acc_or_null && !aligned(acc_or_null, 4)) || (x_absmax_or_null && !aligned(x_absmax_or_null, 4)))
    return BITLINEAR_E_ALIGN;
  if (m > BITLINEAR_FORWARD_MAX_M || !bitlinear::gemv_fits_lds(m, k)) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_norm_quant_gemv_swiglu(packed_gate, gamma_gate, packed_up, gamma_up, f, k, x,
                                                            gain_or_null, eps, m, h, acc_or_null, xq_or_null,
                                                            x_absmax_or_null, static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_forward_f32(const void* packed, const float* gamma, int64_t n, int64_t k, const float* x, int64_t m,
                                float* y, int32_t* acc_or_null, int8_t* xq_or_null, float* x_absmax_or_null,
                                void* stream) {
  if (!packed || !gamma || !x || !y) return BITLINEAR_E_NULL;
  if (int rc = check_nk(n, k)) return rc;
  if (m < 1 || m > kMaxRows) return BITLINEAR_E_SHAPE;
  if ((xq_or_null == nullptr) != (x_absmax_or_null == nullptr)) return BITLINEAR_E_NULL;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(x, 4) || !aligned(y, 4) ||
      (acc_or_null && !aligned(acc_or_null, 4)) || (x_absmax_or_null && !aligned(x_absmax_or_null, 4)))
    return BITLINEAR_E_ALIGN;
  if (m > BITLINEAR_FORWARD_MAX_M || !bitlinear::gemv_fits_lds(m, k)) return BITLINEAR_E_UNSUPPORTED;
  return status_of(bitlinear::launch_quant_gemv_f32(packed, gamma, n, k, x, m, y, acc_or_null, xq_or_null,
                                                    x_absmax_or_null, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
