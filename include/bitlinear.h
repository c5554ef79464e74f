/*
 * bitlinear.h -- C ABI of libbitlinear.so, the BitNet b1.58 BitLinear forward
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (from "BitNet b1.58 in Production: 1-Bit LLMs and Energy
 * Benchmarks", section "The Mathematical Mechanism"):
 *   item 1  gamma = mean |W| over the whole [N][K] weight matrix;
 *           W_q = Clip(Round(W / (gamma + eps)), -1, 1), eps = 1e-5;
 *   item 2  per token (one row of K activations):
 *           x_q = Clip(Round(x * Q_b / a'), -Q_b, Q_b), Q_b = 127,
 *           a' = max(max_k |x|, 1e-8);
 *   item 3  acc[m][n] = sum_k x_q[m][k] * W_q[n][k] in int32 -- an add where
 *           the weight is +1, nothing where it is 0, a subtract where it is -1;
 *   item 4  y[m][n] = acc[m][n] * gamma * a'[m] / Q_b in fp32.
 * "Round" is round-half-to-even throughout.  The 2-bit storage of ternary
 * weights follows "BitNet 1-bit LLM Inference Framework: Running Large
 * Language Models on CPU", section "How the LUT Kernel Works" (four ternary
 * values per byte); the tiled order of those 2-bit fields on the device is
 * this library's own (see bitlinear_packed_bytes).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer on the current HIP device.  The
 *    caller allocates and frees every buffer; the library allocates nothing
 *    and keeps no mutable state, so calls on different streams may overlap
 *    as long as their output buffers do not.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it and the call returns without synchronising.
 *  - Row-major layouts: weights W fp32 [n][k]; activations bf16 [m][k] as raw
 *    uint16 bit patterns; activation codes int8 [m][k]; outputs fp32 [m][n].
 *  - Errors: arguments are validated on the host before any launch; on an
 *    argument error the call returns a negative status and leaves every
 *    output untouched.  A failed launch returns BITLINEAR_E_HIP.  Nothing is
 *    thrown and errno is not used.
 *  - Inputs containing NaN or Inf are outside the contract.
 *  - Sizes: 1 <= n, m <= 2^31 - 1 and 1 <= k <= 2^18 (the matrix cores
 *    accumulate 64 * acc, and |64 * acc| <= 64 * 127 * k stays inside int32).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 2

/* Largest token count accepted by bitlinear_forward (the decode path). */
#define BITLINEAR_FORWARD_MAX_M 16

typedef enum {
    BITLINEAR_OK = 0,
    BITLINEAR_E_NULL = -1,        /* a required pointer is NULL               */
    BITLINEAR_E_SHAPE = -2,       /* a size is outside its range              */
    BITLINEAR_E_ALIGN = -3,       /* a pointer breaks its alignment rule      */
    BITLINEAR_E_UNSUPPORTED = -4, /* valid, but not handled by this entry     */
    BITLINEAR_E_SIZE = -5,        /* a caller buffer is smaller than required */
    BITLINEAR_E_HIP = -6,         /* the HIP runtime reported a launch error  */
    BITLINEAR_E_VALUE = -7        /* a scalar argument is outside its range   */
} bitlinear_status;

/* Version of this ABI and of the device weight layout (BITLINEAR_ABI_VERSION). */
int bitlinear_abi_version(void);

/* Human-readable text of a status code (static storage, never NULL). */
const char *bitlinear_status_string(int status);

/*
 * Bytes of the packed ternary weights of an [n][k] matrix on the device.
 * Layout (version 2): the matrix is cut into tiles of 16 rows x 256 columns;
 * tile (rb, kt) is 1024 contiguous bytes at offset (rb * ceil(k/256) + kt) *
 * 1024, so one 16-row block is a contiguous stream along k.  Inside a tile,
 * 16-byte lane slot l (0..63) holds row 16*rb + (l % 16) and columns
 * 256*kt + 64*(l / 16) + [0, 64); its 32-bit word s covers 16 of those
 * columns, column t of the word in bits 8*(t % 4) + 2*(t / 4).  Each 2-bit
 * field holds w in two's complement (00 = 0, 01 = +1, 11 = -1; 10 unused);
 * rows >= n and columns >= k are padded with 00.  Pure host function;
 * returns 0 if n or k is out of range.
 */
size_t bitlinear_packed_bytes(int64_t n, int64_t k);

/* Bytes of device workspace bitlinear_pack_weights needs (at most 8 KiB). */
size_t bitlinear_pack_workspace_bytes(int64_t n, int64_t k);

/*
 * One-time weight preparation ("The Mathematical Mechanism", item 1):
 * gamma = mean |W| accumulated in fp64 and rounded once to fp32; every
 * weight is ternarised as Clip(Round(W / (gamma + 1e-5)), -1, 1) with one
 * IEEE fp32 divide and round-half-to-even, and written in the tiled 2-bit
 * layout above.
 *   w          in   fp32 [n][k], any 4-byte alignment
 *   packed     out  >= bitlinear_packed_bytes(n, k) bytes, 16-byte aligned
 *   gamma      out  1 fp32
 *   workspace  tmp  >= bitlinear_pack_workspace_bytes(n, k) bytes, 8-byte aligned
 * Two kernels; the gamma of one call never depends on another call.
 */
int bitlinear_pack_weights(const float *w, int64_t n, int64_t k,
                           void *packed, size_t packed_bytes,
                           float *gamma,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * bitlinear_pack_weights for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same result, bit for bit, from the same two kernels; the fp64
 * partial sums that the workspace argument holds otherwise live in a static
 * device array of BITLINEAR_PACK_NOALLOC_SCRATCH_BYTES inside the library
 * (one per GPU, held until the process ends, its address looked up on the
 * first call on each device).  Every accepted (n, k) needs at most that
 * much; a larger need returns BITLINEAR_E_SIZE.  The call allocates nothing.
 * Calls that overlap on one GPU (on different streams, or from different
 * threads) share the array and race: serialise them.
 *   w, packed, packed_bytes, gamma, stream   as bitlinear_pack_weights
 */
#define BITLINEAR_PACK_NOALLOC_SCRATCH_BYTES 8192
int bitlinear_pack_weights_noalloc(const float *w, int64_t n, int64_t k,
                                   void *packed, size_t packed_bytes,
                                   float *gamma, void *stream);

/*
 * Decode the packed layout back to ternary codes (for tests and inspection):
 * the W_q of "The Mathematical Mechanism", item 1, one int8 per weight, from
 * the 2-bit fields described at bitlinear_packed_bytes ("BitNet 1-bit LLM
 * Inference Framework", "How the LUT Kernel Works": four ternary values per
 * byte, here in this library's tiled order).
 *   packed  in   bitlinear_packed_bytes(n, k) bytes, 16-byte aligned
 *   codes   out  int8 [n][k] in {-1, 0, 1}
 */
int bitlinear_unpack_weights(const void *packed, int64_t n, int64_t k,
                             int8_t *codes, void *stream);

/*
 * Per-token absmax int8 activation quantisation ("The Mathematical
 * Mechanism", item 2): for each of the m tokens, a' = max(max_k |x|, 1e-8),
 * s = 127 / a' (one IEEE fp32 divide), x_q = Clip(Round(x * s), -127, 127)
 * (one fp32 multiply, round-half-to-even).
 *   x         in   bf16 bit patterns [m][k], 2-byte aligned
 *   xq        out  int8 [m][k]
 *   x_absmax  out  fp32 [m], receives a'
 */
int bitlinear_quant_act(const uint16_t *x, int64_t m, int64_t k,
                        int8_t *xq, float *x_absmax, void *stream);

/*
 * Decode-path forward for 1 <= m <= BITLINEAR_FORWARD_MAX_M tokens
 * ("The Mathematical Mechanism", items 3 and 4): streams the packed weights
 * once, accumulates acc = sum_k x_q * W_q exactly in int32 and writes
 * y = acc * gamma * a' / 127 in fp32.
 *   packed       in   from bitlinear_pack_weights(n, k), 16-byte aligned
 *   gamma        in   1 fp32 (device)
 *   xq, x_absmax in   from bitlinear_quant_act(m, k)
 *   y            out  fp32 [m][n], 4-byte aligned
 *   acc_or_null  out  optional int32 [m][n] copy of the exact accumulators
 * m > BITLINEAR_FORWARD_MAX_M returns BITLINEAR_E_UNSUPPORTED.
 */
int bitlinear_forward(const void *packed, const float *gamma, int64_t n, int64_t k,
                      const int8_t *xq, const float *x_absmax, int64_t m,
                      float *y, int32_t *acc_or_null, void *stream);

/*
 * Activation quantisation fused into the decode forward: one launch that
 * computes exactly bitlinear_quant_act followed by bitlinear_forward
 * ("The Mathematical Mechanism", items 2-4).  Every workgroup quantises the
 * m tokens into on-chip memory in its prologue while its first weight tiles
 * are in flight, so the int8 codes never round-trip through HBM.
 *   x                 in   bf16 bit patterns [m][k], 2-byte aligned
 *   y                 out  fp32 [m][n]
 *   acc_or_null       out  optional int32 [m][n] exact accumulators
 *   xq_or_null,       out  optional (both or neither): the int8 codes [m][k]
 *   x_absmax_or_null       and a' [m], identical to bitlinear_quant_act's
 * Supported when 1 <= m <= BITLINEAR_FORWARD_MAX_M and the m x k codes fit
 * the workgroup's on-chip budget (bitlinear_quant_forward_supported);
 * otherwise returns BITLINEAR_E_UNSUPPORTED.
 */
int bitlinear_quant_forward(const void *packed, const float *gamma, int64_t n, int64_t k,
                            const uint16_t *x, int64_t m,
                            float *y, int32_t *acc_or_null,
                            int8_t *xq_or_null, float *x_absmax_or_null, void *stream);

/* 1 if bitlinear_quant_forward accepts (m, k), else 0.  Pure host function. */
int bitlinear_quant_forward_supported(int64_t m, int64_t k);

/*
 * Batched (prefill) forward for 1 <= m <= 2^21 ("The Mathematical
 * Mechanism", items 3 and 4, for many tokens at once; "BitNet 1-bit LLM
 * Inference Framework", "Scalability with Thread Count": prompt processing is
 * compute-intensive): the same result as bitlinear_forward, computed as a
 * tiled int8 matrix-core contraction with the ternary tiles expanded on chip.  Larger m returns
 * BITLINEAR_E_UNSUPPORTED (split the tokens into several calls).
 * When the output tiles are too few to fill the device, the k extent is
 * split across workgroups: the exact int32 partial sums are added with
 * atomics in acc_or_null, or else in y's own memory (y is scratch until the
 * call's last kernel writes it), and a last pass scales them into y.  The
 * results are bit-identical either way; the call then enqueues three
 * kernels on the stream instead of one.
 */
int bitlinear_forward_batched(const void *packed, const float *gamma, int64_t n, int64_t k,
                              const int8_t *xq, const float *x_absmax, int64_t m,
                              float *y, int32_t *acc_or_null, void *stream);

/*
 * RMSNorm ahead of the activation quantisation ("BitNet b1.58 in
 * Production", listing "bit_linear.py": the BitLinear input passes
 * nn.RMSNorm, and activation_quant is applied to the normalised input).  Per
 * token r = 1 / sqrt(mean_k x^2 + eps) and x_norm = x * r * gain; then the
 * rule of bitlinear_quant_act on x_norm: a' = max(max_k |x_norm|, 1e-8),
 * x_q = Clip(Round(x_norm * 127 / a'), -127, 127).
 * Absmax quantisation is invariant under the positive per-token factor r, so
 * the codes are computed from v = x * gain (one fp32 multiply per value;
 * gain = 1 when NULL) and r is carried by the scale:
 *   s = 127 / max_k |v| (IEEE fp32 divide); x_q = Clip(Round(v * s), -127, 127);
 *   a' = max_k |v| * r (mean square in fp64, product rounded once);
 * when that a' is below 1e-8 the floor is the token's scale instead
 * (s = r * 127 / 1e-8 on v, a' = 1e-8), as the listing's clamp makes it.
 * The codes therefore equal Round(x_norm * 127 / a') except where that
 * value lies within a few fp32 roundings of a tie (2^-19 relative), where
 * they may be the other neighbour; a' agrees with max|x_norm| to within a
 * few ulps.  A token whose v is all zero gets codes 0 and a' = 1e-8.
 * y = acc * gamma * a' / 127 then de-quantises the normalised input.
 *   x             in   bf16 bit patterns [m][k], 2-byte aligned
 *   gain_or_null  in   fp32 [k] per-channel gain, 4-byte aligned, or NULL
 *   eps           in   finite and >= 0 (nn.RMSNorm's default for fp32 input
 *                      is FLT_EPSILON), else BITLINEAR_E_VALUE; with eps = 0
 *                      an all-zero token has no defined x_norm (0 / 0) and
 *                      is outside the contract
 *   xq, x_absmax  out  int8 [m][k] and fp32 [m] (a')
 */
int bitlinear_rmsnorm_quant_act(const uint16_t *x, const float *gain_or_null, float eps,
                                int64_t m, int64_t k, int8_t *xq, float *x_absmax, void *stream);

/*
 * RMSNorm and quantisation fused into the decode forward: one launch that
 * computes exactly bitlinear_rmsnorm_quant_act followed by bitlinear_forward.
 * Arguments as bitlinear_quant_forward plus gain_or_null and eps as above;
 * the same (m, k) support rule (bitlinear_quant_forward_supported).
 */
int bitlinear_rmsnorm_quant_forward(const void *packed, const float *gamma, int64_t n, int64_t k,
                                    const uint16_t *x, const float *gain_or_null, float eps, int64_t m,
                                    float *y, int32_t *acc_or_null,
                                    int8_t *xq_or_null, float *x_absmax_or_null, void *stream);

/*
 * Per-token quantisation of fp32 activations: the rule of bitlinear_quant_act
 * applied to binary32 inputs, for activations produced on the device in fp32
 * (such as the SwiGLU output of the feed-forward block, which feeds the down
 * projection).
 *   x             in   fp32 [m][k], 4-byte aligned
 *   xq, x_absmax  out  int8 [m][k] and fp32 [m] (a')
 */
int bitlinear_quant_act_f32(const float *x, int64_t m, int64_t k,
                            int8_t *xq, float *x_absmax, void *stream);

/*
 * Gate and up projections of the feed-forward block with the SwiGLU between
 * them fused into the epilogue ("BitNet 1-bit LLM Inference Framework",
 * section "A Deep Look at the BitNet Architecture": the block's ffn is
 * down_proj(silu(gate_proj(x)) * up_proj(x))).  For every token t and
 * feature j:
 *   y_g = acc_g * gamma_gate * a'[t] / 127,  y_u = acc_u * gamma_up * a'[t] / 127
 *   h[t][j] = y_g * y_u / (1 + exp(-y_g))     (fp32)
 * from one pass over the activation codes; the [m][2f] projections are never
 * written.  The gate and up matrices are packed separately (each with its own
 * gamma) or are the two halves of one packed [2f][k] matrix (f % 16 == 0:
 * the up half starts bitlinear_packed_bytes(f, k) bytes in).
 *   packed_gate, packed_up  in   from bitlinear_pack_weights(f, k), 16-byte aligned
 *   gamma_gate, gamma_up    in   1 fp32 each (device)
 *   xq, x_absmax            in   codes [m][k] and a' [m] of the block input
 *   h                       out  fp32 [m][f], 4-byte aligned
 *   acc_or_null             out  optional int32 [m][2f]: per token the f gate
 *                                accumulators, then the f up accumulators
 * 1 <= m <= 2^21.  Up to BITLINEAR_FORWARD_MAX_M tokens whose codes fit the
 * decode path's on-chip budget use the streaming decode kernel; otherwise the
 * matrix-core kernel, which needs k % 16 == 0 and 16-byte aligned codes
 * (else BITLINEAR_E_UNSUPPORTED).
 */
int bitlinear_forward_swiglu(const void *packed_gate, const float *gamma_gate,
                             const void *packed_up, const float *gamma_up,
                             int64_t f, int64_t k, const int8_t *xq, const float *x_absmax, int64_t m,
                             float *h, int32_t *acc_or_null, void *stream);

/*
 * The feed-forward block's first half in one launch for the decode path:
 * RMSNorm + quantisation of the block input (as bitlinear_rmsnorm_quant_act)
 * fused into the gate / up projections with the SwiGLU epilogue (as
 * bitlinear_forward_swiglu).  Arguments as those two entry points; xq_or_null
 * and x_absmax_or_null (both or neither) receive the codes and a'.  Supported
 * for the (m, k) of bitlinear_quant_forward_supported, else
 * BITLINEAR_E_UNSUPPORTED.
 */
int bitlinear_rmsnorm_quant_forward_swiglu(const void *packed_gate, const float *gamma_gate,
                                           const void *packed_up, const float *gamma_up,
                                           int64_t f, int64_t k, const uint16_t *x,
                                           const float *gain_or_null, float eps, int64_t m,
                                           float *h, int32_t *acc_or_null,
                                           int8_t *xq_or_null, float *x_absmax_or_null, void *stream);

/*
 * Quantisation of fp32 activations fused into the decode forward: exactly
 * bitlinear_quant_act_f32 followed by bitlinear_forward, in one launch (the
 * down projection fed by the SwiGLU output h).  x: fp32 [m][k], 4-byte
 * aligned; other arguments and the support rule as bitlinear_quant_forward.
 */
int bitlinear_quant_forward_f32(const void *packed, const float *gamma, int64_t n, int64_t k,
                                const float *x, int64_t m, float *y, int32_t *acc_or_null,
                                int8_t *xq_or_null, float *x_absmax_or_null, void *stream);

/*
 * Table-lookup decode forward ("BitNet 1-bit LLM Inference Framework",
 * "How the LUT Kernel Works": every ternary weight is -1, 0 or +1, so the
 * product of a weight group with the activations takes one of a few values
 * that can be looked up instead of multiplied).  Same arguments and the same
 * result, bit for bit, as bitlinear_forward: each workgroup builds in on-chip
 * memory the 16 partial sums of every pair of int8 codes that share a 4-bit
 * nibble of the packed layout and adds one table entry per weight pair.  The
 * table takes 16 bytes per activation column (k rounded up to 256), so
 * 1 <= m <= BITLINEAR_FORWARD_MAX_M and bitlinear_forward_lut_supported(k)
 * are required, else BITLINEAR_E_UNSUPPORTED.  Each token streams the weights
 * once: the entry is meant for m = 1 and is kept as the measured counterpart
 * of the matrix-core decode kernel.
 */
int bitlinear_forward_lut(const void *packed, const float *gamma, int64_t n, int64_t k,
                          const int8_t *xq, const float *x_absmax, int64_t m,
                          float *y, int32_t *acc_or_null, void *stream);

/* 1 if bitlinear_forward_lut's table for k fits on chip, else 0.  Pure host function. */
int bitlinear_forward_lut_supported(int64_t k);

/* ======================================================================
 * Variant modes described by the other pages.  Each keeps the main path's
 * contraction (int8 codes times +-1 / 0 weights, exact int32 accumulators)
 * and changes one side of it.
 * ====================================================================== */

/*
 * V1, activation side: one scale per tensor with Q_b = 128 ("BitNet 1-bit LLM
 * Inference Framework", "A Deep Look at the BitNet Architecture", "The Core
 * Structure of BitNet b1.58": the BitLinear class's activation_quantize).
 * g = max |x| over all m * k values; every code is
 * round_half_even(clamp((x * 128) / (g + 1e-8), -128, 127)) (fp32 multiply,
 * one IEEE fp32 divide, g + 1e-8 in fp32), so codes span [-128, 127].
 *   x          in   bf16 bit patterns [m][k], 2-byte aligned, finite
 *   xq         out  int8 [m][k]
 *   x_scale    out  1 fp32: g (without the 1e-8, the de-quantization scale)
 *   workspace  tmp  >= bitlinear_quant_act_tensor_workspace_bytes(m, k) bytes
 *                   (at most 4 KiB), 4-byte aligned
 * m * k above 2^40 returns BITLINEAR_E_SHAPE.  One launch for at most 16384
 * values, else two.
 */
size_t bitlinear_quant_act_tensor_workspace_bytes(int64_t m, int64_t k);
int bitlinear_quant_act_tensor(const uint16_t *x, int64_t m, int64_t k,
                               int8_t *xq, float *x_scale,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * V1 forward: the codes of bitlinear_quant_act_tensor against main-path
 * weights (bitlinear_pack_weights), y = acc * (gamma * g / 128) in fp32 (the
 * class's de-quantization by w_scale * x_scale / 2^7).  Any 1 <= m <= 2^21
 * (decode kernel up to BITLINEAR_FORWARD_MAX_M tokens, matrix cores above);
 * k must be below 2^18 (|acc| <= 128 k), else BITLINEAR_E_SHAPE.
 *   x_scale  in  1 fp32 (device), from bitlinear_quant_act_tensor
 *   other arguments as bitlinear_forward
 */
int bitlinear_forward_tensor_act(const void *packed, const float *gamma, int64_t n, int64_t k,
                                 const int8_t *xq, const float *x_scale, int64_t m,
                                 float *y, int32_t *acc_or_null, void *stream);

/*
 * V2, weight side: one binary16 scale per output channel ("BitNet-2B-4T:
 * Inside the 2B-Parameter, 4T-Token 1-Bit LLM", "Weight Representation:
 * Ternary + Scale, Not Pure Binary").  The page does not say how the scale
 * is found; here s_r = binary16(fp32(mean |W[r][:]|)) (fp64 sum, one rounding
 * to fp32, then round-to-nearest-even to binary16), and row r is ternarised
 * as Clip(Round(W / (s_r + 1e-5)), -1, 1) with that stored value, in the
 * same tiled 2-bit layout (bitlinear_packed_bytes).
 *   w       in   fp32 [n][k], 4-byte aligned, finite
 *   packed  out  >= bitlinear_packed_bytes(n, k) bytes, 16-byte aligned
 *   scales  out  binary16 bit patterns [n], 2-byte aligned
 * Rows whose absmean rounds above the binary16 range get an infinite scale.
 */
int bitlinear_pack_weights_rowscale(const float *w, int64_t n, int64_t k,
                                    void *packed, size_t packed_bytes,
                                    uint16_t *scales, void *stream);

/*
 * V2 forward: per-token codes (bitlinear_quant_act), y[t][j] = acc *
 * (s_j * a'_t / 127) in fp32 with s_j widened from binary16.  Any
 * 1 <= m <= 2^21 as bitlinear_forward_tensor_act.
 *   scales  in  binary16 [n] (device), from bitlinear_pack_weights_rowscale
 *   other arguments as bitlinear_forward
 */
int bitlinear_forward_rowscale(const void *packed, const uint16_t *scales, int64_t n, int64_t k,
                               const int8_t *xq, const float *x_absmax, int64_t m,
                               float *y, int32_t *acc_or_null, void *stream);

/*
 * V3, weight side: binary weights W_bit = s * sign(W) with one per-layer
 * scale s ("BitNet's 1-Bit Transformer: Architecture Breakdown", "Binary
 * Weight Matrices with Learnable Scaling"), one bit per weight.  sign(0) is
 * taken as +1 (one bit has no code for 0): the bit is set exactly where
 * W < 0.  s is learned, so it is an input of the forward, not computed here.
 * Layout: tiles of 16 rows x 512 columns, 1024 bytes each, tile (rb, kt) at
 * byte (rb * ceil(k/512) + kt) * 1024; 16-byte slot l (0..63) holds row
 * 16*rb + (l % 16) and columns 512*kt + 128*(l / 16) + [0, 128); its 32-bit
 * word s (0..3) covers 32 of those columns, column c of the word in bit
 * 8*(c % 4) + 7 - c/4 (set = -1, clear = +1).  Padding bits are clear.
 */
size_t bitlinear_packed_bytes_binary(int64_t n, int64_t k);
int bitlinear_pack_binary(const float *w, int64_t n, int64_t k,
                          void *packed, size_t packed_bytes, void *stream);

/* Decode the binary layout to int8 codes in {-1, +1} [n][k] (tests, inspection). */
int bitlinear_unpack_binary(const void *packed, int64_t n, int64_t k,
                            int8_t *codes, void *stream);

/*
 * V3 forward: per-token codes against the sign bits, y = acc * (s * a' / 127)
 * in fp32.  Any 1 <= m <= 2^21 as bitlinear_forward_tensor_act.
 *   packed  in  from bitlinear_pack_binary(n, k), 16-byte aligned
 *   scale   in  1 fp32 (device): the layer's scale s
 *   other arguments as bitlinear_forward
 */
int bitlinear_forward_binary(const void *packed, const float *scale, int64_t n, int64_t k,
                             const int8_t *xq, const float *x_absmax, int64_t m,
                             float *y, int32_t *acc_or_null, void *stream);

/*
 * V3 decode forward with the activation quantisation fused (as
 * bitlinear_quant_forward, binary weights).  Supported when
 * bitlinear_quant_forward_binary_supported(m, k), else BITLINEAR_E_UNSUPPORTED.
 */
int bitlinear_quant_forward_binary(const void *packed, const float *scale, int64_t n, int64_t k,
                                   const uint16_t *x, int64_t m, float *y, int32_t *acc_or_null,
                                   int8_t *xq_or_null, float *x_absmax_or_null, void *stream);
int bitlinear_quant_forward_binary_supported(int64_t m, int64_t k);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
