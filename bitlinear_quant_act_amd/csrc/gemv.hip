// Decode-path BitLinear forward for 1..16 tokens.
//
// "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
// "The Mathematical Mechanism", items 2-4: per-token int8 codes, acc =
// sum_k x_q * W_q with W_q in {-1, 0, +1} (adds and subtracts only), then
// y = acc * gamma * a' / 127.  "BitNet 1-bit LLM Inference Framework",
// section "Scalability with Thread Count": generation is bound by memory
// bandwidth, so the kernel streams the 2-bit weights from HBM exactly once,
// with as many bytes in flight as the chip can hold.
//
// Work split: a persistent grid (at most kMaxResidentGroups workgroups, each
// taking the same number of 16-row blocks of W).  The WAVES waves of a
// workgroup take a row block's 256-column tiles round-robin (wave w: tiles w,
// w + WAVES, ...), so the workgroup reads consecutive KiB of one contiguous
// stream; every tile is one fully coalesced 16-byte-per-lane load.  A wave
// requests all its tiles of the next row block before it consumes the
// current one (rows longer than U * WAVES tiles are walked in chunks).
//
// Activation codes live in LDS for the whole kernel (m rows, padded pitch so
// the 16 token rows of one operand read start in distinct banks).  They are
// staged once per workgroup by one of two prologues:
//   * kFromCodes: copied from the int8 codes of bitlinear_quant_act;
//   * kFromBf16:  computed from the bf16 activations -- the activation
//     quantisation fused into the GEMV: per-token max|x| as integer bit
//     patterns, a' = max(., 1e-8), s = 127 / a' (IEEE divide), code =
//     clamp(rint(x * s)), bit-identical to bitlinear_quant_act;
//   * kFromBf16Norm: RMSNorm fused as well ("bit_linear.py" listing: the
//     BitLinear input passes nn.RMSNorm first): codes of v = x * gain, and
//     a' = max|v| / sqrt(mean x^2 + eps) (the per-token factor cancels in
//     the codes; rmsnorm_scales), equal to bitlinear_rmsnorm_quant_act's
//     (a' within one ulp: the mean square is an fp64 sum in another order);
//   * kFromF32: computed from fp32 activations, bit-identical to
//     bitlinear_quant_act_f32.
// The activations are requested before the first weight tiles: vector-memory
// results are waited for in issue order, so the prologue then runs while the
// weights are still in flight.
//
// Contraction on the matrix cores: one v_mfma_i32_16x16x64_i8 multiplies 16
// tokens x 64 columns of codes (A; token rows >= m are zero) by 64 columns x
// 16 weight rows (B).  A lane's B operand is one 32-bit word of its packed
// slot, expanded with one shift and one mask per 4 weights (expand_ternary:
// each 2-bit two's-complement field lands in the top bits of its byte, the
// int8 value 64 * w).  The MFMA therefore accumulates 64 * acc exactly; the
// epilogue shifts it back.  A lane's A operand is the 16 codes of its own
// token at the same 16 columns, so A and B share the k order without any
// shuffling.
//
// Barriers are LDS-only (lds_barrier): a __syncthreads fence would wait for
// the weight tiles still in flight.
//
// Epilogue: the waves' int32 partials are summed through LDS and scaled by
// gamma * a'[m] / 127 in fp32; lanes 0..15 of a result row write 16
// consecutive floats.
//
// When m x k codes exceed the LDS budget, the global-operand variant reads
// each lane's 16-byte A operand straight from the codes in memory instead.
#include "bitlinear_internal.hpp"

namespace bitlinear {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Persistent grid: at most 256 workgroups of 16 waves (one per compute unit,
// which stages the activations once), or 512 of 8 waves; dispatch_lds picks
// the size per row length.
#ifndef BITLINEAR_GEMV_MAX_GROUPS
#define BITLINEAR_GEMV_MAX_GROUPS 256
#endif
#ifndef BITLINEAR_GEMV_WAVES
#define BITLINEAR_GEMV_WAVES 16
#endif
constexpr int64_t kMaxResidentGroups = BITLINEAR_GEMV_MAX_GROUPS;  // persistent grid cap
constexpr int kWaves = BITLINEAR_GEMV_WAVES;                        // waves per workgroup
// dynamic LDS budget for the staged codes: 140 KiB, which leaves the static
// reduction buffer (16 KiB at 16 waves) and the small arrays room inside the
// CU's 160 KiB.  The launch raises the kernel's dynamic-LDS limit to it.  The
// persistent grid holds one 16-wave workgroup per CU; the 8-wave kernels
// (two per CU) keep two resident while their codes take at most ~70 KiB.
constexpr int kMaxLdsBytes = 140 * 1024;
constexpr int kCachedChunks = 4;  // activation chunks per thread held in registers by the prologue

// Weight tiles are read as a raw buffer: a buffer resource names a base
// address and a byte extent, and a load past the extent returns zero without
// touching memory.  Every lane issues every tile load, with no branch around
// it, so on every path the loads complete in issue order and the prologue's
// waits for the activations (requested first) leave the weight tiles
// requested after them in flight.
constexpr int kRawBuffer = 0x00020000;  // descriptor word 3: untyped, 32-bit data format
constexpr int kLoadNonTemporal = 2;     // cache policy: read once

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_tile_nt(__amdgpu_buffer_rsrc_t r, int offset) {
  const v4u_t t = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, kLoadNonTemporal);
  return make_uint4(t.x, t.y, t.z, t.w);
}

enum Source { kFromCodes = 0, kFromBf16 = 1, kFromBf16Norm = 2, kFromF32 = 3 };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint32_t quant_code(uint32_t bits16, float s) {
  float r = rintf(bf16_to_f32(bits16) * s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu;
}

// The code of a value v of a token with scale s = 127 / a', a' >= max|x|,
// as the bit pattern of fl(fl(v s) + 1.5 * 2^23).  |fl(v s)| rounds to at
// most 127, so the clamp to [-127, 127] never binds; in [2^23, 2^24) floats
// are the integers, so the sum is 1.5 * 2^23 + rint(v s) (ties to even, the
// default rounding), and its low byte is rint(v s) in two's complement.
// Two operations per value instead of a round, a clamp and a conversion.
__device__ __forceinline__ uint32_t code_bits(float v, float s) {
  return __float_as_uint(__fadd_rn(__fmul_rn(v, s), 12582912.0f));
}

// the low bytes of four words, in order, as one word
__device__ __forceinline__ uint32_t low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);  // b0.byte0, b1.byte0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);               // lo.byte0-1, hi.byte0-1
}

// 8 bf16 values (one 16-byte chunk) -> 8 codes (two words); value 2q of a
// chunk is the low half of word q, value 2q + 1 its high half
__device__ __forceinline__ uint2 quant_chunk(const uint4& v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t b[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    b[2 * q] = code_bits(__uint_as_float(w[q] << 16), s);
    b[2 * q + 1] = code_bits(__uint_as_float(w[q] & 0xffff0000u), s);
  }
  return make_uint2(low_bytes(b[0], b[1], b[2], b[3]), low_bytes(b[4], b[5], b[6], b[7]));
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// max |x| of a chunk as a bf16 bit pattern (sign cleared: the patterns of
// non-negative values order like the values), two halves per packed 16-bit max
__device__ __forceinline__ unsigned chunk_absmax(const uint4& v) {
  const u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7fff7fffu);
  const u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7fff7fffu);
  const u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7fff7fffu);
  const u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7fff7fffu);
  const u16x2 mx = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max(static_cast<unsigned>(mx.x), static_cast<unsigned>(mx.y));
}

__device__ __forceinline__ unsigned wave_max(unsigned v) { return wave_max_u32(v); }

// LDS row pitch of the staged codes: the padded k extent plus 16 bytes, so
// consecutive token rows start 4 banks apart.
__host__ __device__ inline int64_t lds_pitch(int64_t kt_count) { return kt_count * kTileCols + 16; }

inline size_t lds_bytes(int64_t m, int64_t kt_count) { return static_cast<size_t>(m * lds_pitch(kt_count)); }

// chunk j of this thread held in registers (j is uniform per loop trip)
__device__ __forceinline__ uint4 cached(const uint4 (&cache)[kCachedChunks], int j) {
  uint4 v = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int q = 0; q < kCachedChunks; ++q)
    if (q == j) v = cache[q];
  return v;
}

// ---------------------------------------------------------------------------
// prologues: fill xs[t][0 .. kpad) for t < m (zero past k); a' to amax_s
// ---------------------------------------------------------------------------

// Vector paths, first step: request this thread's first kCachedChunks 16-byte
// chunks (chunk c = thread + j * blockDim.x) before anything else.
__device__ __forceinline__ void prefetch_codes(uint4 (&cache)[kCachedChunks], const int8_t* __restrict__ xq, int m,
                                               int64_t k, int kpad) {
  const int cpr = kpad / 16;
#pragma unroll
  for (int j = 0; j < kCachedChunks; ++j) {
    // every thread requests every chunk (a chunk past the codes reads chunk 0,
    // and stage_codes stores zeros for it), so later waits count exactly
    const int c = threadIdx.x + j * static_cast<int>(blockDim.x);
    const int t = c / cpr;
    const int64_t col = static_cast<int64_t>(c - t * cpr) * 16;
    const bool ok = c < m * cpr && col < k;
    cache[j] = *reinterpret_cast<const uint4*>(xq + (ok ? t * k + col : 0));
  }
}

// Waves per token when m tokens share a workgroup's waves: the largest power
// of two G with m * G <= WAVES (m <= WAVES).  Token t belongs to waves
// [t G, t G + G); inside them, thread tt = threadIdx.x - 64 t G takes the
// token's 16-byte chunks tt, tt + 64 G, ...  With m = 1 that is every thread
// over the whole row.
template <int WAVES>
__device__ __forceinline__ int token_group(int m) {
  int g = WAVES;
  while (g > 1 && g * m > WAVES) g >>= 1;
  return g;
}

// The wave's place in its token group, in scalar registers: every wave of a
// group runs the same prologue code, so its indices cost no vector
// instructions (each vector instruction of a prologue is paid by all waves
// of the workgroup, four to a SIMD).
struct TokenGroup {
  int G;     // waves per token
  int t;     // the wave's token
  int w0;    // the group's first wave, t * G
  int tt;    // the lane's thread index inside the group (vector)
};

template <int WAVES>
__device__ __forceinline__ TokenGroup token_group_of(int m) {
  TokenGroup g;
  g.G = token_group<WAVES>(m);
  const int lg = __builtin_ctz(static_cast<unsigned>(g.G));
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  g.t = wave >> lg;
  g.w0 = g.t << lg;
  g.tt = static_cast<int>(threadIdx.x) - 64 * g.w0;
  return g;
}

__device__ __forceinline__ unsigned max4(const uint4& v) { return max(max(v.x, v.y), max(v.z, v.w)); }

// max of the wave slots [w0, w0 + G) of one token group (G a power of two up
// to 16, w0 a multiple of G, both wave-uniform: one branch runs, with
// 16-byte slot reads)
__device__ __forceinline__ unsigned group_slot_max(const unsigned* slots, int w0, int G) {
  const uint4* p = reinterpret_cast<const uint4*>(slots + w0);
  if (G == 16) return max(max(max4(p[0]), max4(p[1])), max(max4(p[2]), max4(p[3])));
  if (G == 8) return max(max4(p[0]), max4(p[1]));
  if (G == 4) return max4(p[0]);
  if (G == 2) return max(slots[w0], slots[w0 + 1]);
  return slots[w0];
}

// sum of the wave slots [w0, w0 + G) in wave order (the same order for every
// token count), under the same conditions
__device__ __forceinline__ double group_slot_sum(const double* slots, int w0, int G) {
  const double* p = slots + w0;
  double r = p[0];
  if (G == 16) {
#pragma unroll
    for (int i = 1; i < 16; ++i) r += p[i];
  } else if (G == 8) {
#pragma unroll
    for (int i = 1; i < 8; ++i) r += p[i];
  } else if (G == 4) {
#pragma unroll
    for (int i = 1; i < 4; ++i) r += p[i];
  } else if (G == 2) {
    r += p[1];
  }
  return r;
}

__device__ __forceinline__ void prefetch_bf16(uint4 (&cache)[kCachedChunks], const uint16_t* __restrict__ x, int m,
                                              int64_t k) {
  const int total = m * static_cast<int>(k / 8);
#pragma unroll
  for (int j = 0; j < kCachedChunks; ++j) {
    const int c = threadIdx.x + j * static_cast<int>(blockDim.x);
    cache[j] = c < total ? *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 8) : make_uint4(0, 0, 0, 0);
  }
}

// m > 1 tokens (m <= WAVES): chunk order of stage_bf16_group
template <int WAVES>
__device__ __forceinline__ void prefetch_bf16_group(uint4 (&cache)[kCachedChunks], const uint16_t* __restrict__ x, int m,
                                                    int64_t k) {
  const TokenGroup g = token_group_of<WAVES>(m);
  const int cpr = static_cast<int>(k / 8);
  const uint4* row = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(g.t < m ? g.t : 0) * k);
#pragma unroll
  for (int j = 0; j < kCachedChunks; ++j) {
    const int c = g.tt + j * 64 * g.G;
    cache[j] = (g.t < m && c < cpr) ? row[c] : make_uint4(0, 0, 0, 0);
  }
}

__device__ void stage_codes(int8_t* xs, int pitch, const uint4 (&cache)[kCachedChunks],
                            const int8_t* __restrict__ xq, int m, int64_t k, int kpad, bool vec) {
  const int nthreads = blockDim.x;
  if (vec) {  // k % 16 == 0 and xq 16-byte aligned
    const int cpr = kpad / 16;
    const int total = m * cpr;
    // chunk c = threadIdx.x + j * nthreads: the first kCachedChunks are in
    // registers already and are stored on every path (so none of their
    // requests is moved behind the weight tiles); the rest are requested
    // kCachedChunks at a time and then stored, one wait per batch instead of
    // one per chunk
    auto store = [&](int j, const uint4& v) {
      const int c = threadIdx.x + j * nthreads;
      const int t = c / cpr, cc = c - t * cpr;
      const bool ok = c < total && static_cast<int64_t>(cc) * 16 < k;
      if (c < total) *reinterpret_cast<uint4*>(xs + t * pitch + cc * 16) = ok ? v : make_uint4(0, 0, 0, 0);
    };
#pragma unroll
    for (int q = 0; q < kCachedChunks; ++q) store(q, cache[q]);
    for (int j0 = kCachedChunks; j0 * nthreads < total; j0 += kCachedChunks) {
      uint4 v[kCachedChunks];
#pragma unroll
      for (int q = 0; q < kCachedChunks; ++q) {
        const int c = threadIdx.x + (j0 + q) * nthreads;
        const int t = c / cpr, cc = c - t * cpr;
        const int64_t col = static_cast<int64_t>(cc) * 16;
        v[q] = *reinterpret_cast<const uint4*>(xq + (c < total && col < k ? t * k + col : 0));
      }
#pragma unroll
      for (int q = 0; q < kCachedChunks; ++q) store(j0 + q, v[q]);
      // everything requested so far has landed (the batch came last); said
      // explicitly, so that the code after the loop need not assume a batch
      // request may still write its registers
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) only (gfx9 encoding)
    }
  } else {
    for (int c = threadIdx.x; c < m * kpad; c += nthreads) {
      const int t = c / kpad, col = c - t * kpad;
      xs[t * pitch + col] = col < k ? xq[t * k + col] : static_cast<int8_t>(0);
    }
  }
}

// Single token, vector path: wave shuffles + one LDS slot per wave, no atomics.
template <int WAVES>
__device__ void stage_bf16_single(int8_t* xs, float* amax_s, unsigned* wmax_s, const uint4 (&cache)[kCachedChunks],
                                  const uint16_t* __restrict__ x, int64_t k, int kpad, int8_t* __restrict__ xq_out,
                                  float* __restrict__ amax_out) {
  const int nthreads = blockDim.x;
  const bool write_out = xq_out != nullptr && blockIdx.x == 0;
  const int total = static_cast<int>(k / 8);
  unsigned mx = 0;
  int j = 0;
  for (int c = threadIdx.x; c < total; c += nthreads, ++j)
    mx = max(mx, chunk_absmax(j < kCachedChunks ? cached(cache, j)
                                                : *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 8)));
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) wmax_s[threadIdx.x >> 6] = mx;
  lds_barrier();
  unsigned mall = wmax_s[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) mall = max(mall, wmax_s[w]);
  const float a = fmaxf(bf16_to_f32(mall), 1e-8f);
  const float s = 127.0f / a;
  if (threadIdx.x == 0) {
    amax_s[0] = a;
    if (write_out) amax_out[0] = a;
  }
  j = 0;
  for (int c = threadIdx.x; c < total; c += nthreads, ++j) {
    const uint2 q = quant_chunk(j < kCachedChunks ? cached(cache, j)
                                                  : *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 8),
                                s);
    *reinterpret_cast<uint2*>(xs + c * 8) = q;
    if (write_out) *reinterpret_cast<uint2*>(xq_out + c * 8) = q;
  }
  for (int c = total + threadIdx.x; c < kpad / 8; c += nthreads) *reinterpret_cast<uint2*>(xs + c * 8) = make_uint2(0, 0);
}

// Vector path, 1 < m <= WAVES tokens: the waves of a token group
// (token_group) reduce max|x| over their chunks with DPP wave operations; with
// more than one wave per token the wave maxima meet through one LDS slot per
// wave and one barrier.  No atomics.  The chunk order is prefetch_bf16_group's.
template <int WAVES>
__device__ void stage_bf16_group(int8_t* xs, int pitch, float* amax_s, unsigned* wmax_s,
                                 const uint4 (&cache)[kCachedChunks], const uint16_t* __restrict__ x, int m, int64_t k,
                                 int kpad, int8_t* __restrict__ xq_out, float* __restrict__ amax_out) {
  const bool write_out = xq_out != nullptr && blockIdx.x == 0;
  const TokenGroup g = token_group_of<WAVES>(m);
  const int G = g.G, t = g.t, tt = g.tt;
  const int step = 64 * G;
  const bool active = t < m;
  const int cpr = static_cast<int>(k / 8);
  const uint4* row = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(active ? t : 0) * k);
  unsigned mx = 0;
  int j = 0;
  if (active)
    for (int c = tt; c < cpr; c += step, ++j) mx = max(mx, chunk_absmax(j < kCachedChunks ? cached(cache, j) : row[c]));
  mx = wave_max(mx);
  if (G > 1) {  // uniform: m is the same for the whole workgroup
    if ((threadIdx.x & 63) == 0) wmax_s[threadIdx.x >> 6] = mx;
    lds_barrier();
    mx = group_slot_max(wmax_s, g.w0, G);
  }
  if (!active) return;
  const float a = fmaxf(bf16_to_f32(mx), 1e-8f);
  const float s = 127.0f / a;
  if (tt == 0) {
    amax_s[t] = a;
    if (write_out) amax_out[t] = a;
  }
  int8_t* xrow = xs + t * pitch;
  j = 0;
  for (int c = tt; c < cpr; c += step, ++j) {
    const uint2 q = quant_chunk(j < kCachedChunks ? cached(cache, j) : row[c], s);
    *reinterpret_cast<uint2*>(xrow + c * 8) = q;
    if (write_out) *reinterpret_cast<uint2*>(xq_out + static_cast<int64_t>(t) * k + c * 8) = q;
  }
  for (int c = cpr + tt; c < kpad / 8; c += step) *reinterpret_cast<uint2*>(xrow + c * 8) = make_uint2(0, 0);
}

// Any token count: per-token max through LDS atomics (one per token change).
// Used where stage_bf16_group does not apply (unaligned rows, more tokens than
// waves, or a kernel built without it).  CACHED: cache holds prefetch_bf16's
// thread-major chunks; otherwise the activations are read here.
template <bool CACHED>
__device__ void stage_bf16(int8_t* xs, int pitch, float* amax_s, unsigned* max_s, const uint4 (&cache)[kCachedChunks],
                           const uint16_t* __restrict__ x, int m, int64_t k, int kpad, bool vec,
                           int8_t* __restrict__ xq_out, float* __restrict__ amax_out) {
  const int nthreads = blockDim.x;
  const bool write_out = xq_out != nullptr && blockIdx.x == 0;
  if (threadIdx.x < m) max_s[threadIdx.x] = 0u;
  lds_barrier();
  if (vec) {  // k % 8 == 0 and x 16-byte aligned: chunks of 8 values
    const int cpr = static_cast<int>(k / 8);
    const int total = m * cpr;
    int cur_t = -1;
    unsigned cur = 0;
    int j = 0;
    for (int c = threadIdx.x; c < total; c += nthreads, ++j) {
      const int t = c / cpr;
      if (t != cur_t) {
        if (cur_t >= 0) atomicMax(&max_s[cur_t], cur);
        cur_t = t;
        cur = 0;
      }
      cur = max(cur, chunk_absmax(CACHED && j < kCachedChunks ? cached(cache, j)
                                                    : *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 8)));
    }
    if (cur_t >= 0) atomicMax(&max_s[cur_t], cur);
    lds_barrier();
    if (threadIdx.x < m) amax_s[threadIdx.x] = fmaxf(bf16_to_f32(max_s[threadIdx.x]), 1e-8f);
    lds_barrier();
    j = 0;
    for (int c = threadIdx.x; c < total; c += nthreads, ++j) {
      const int t = c / cpr, cc = c - t * cpr;
      const uint2 q = quant_chunk(CACHED && j < kCachedChunks ? cached(cache, j)
                                                    : *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 8),
                                  127.0f / amax_s[t]);
      *reinterpret_cast<uint2*>(xs + t * pitch + cc * 8) = q;
      if (write_out) *reinterpret_cast<uint2*>(xq_out + t * k + cc * 8) = q;
    }
    const int padc = (kpad - static_cast<int>(k)) / 8;
    for (int c = threadIdx.x; c < m * padc; c += nthreads) {
      const int t = c / padc, cc = c - t * padc;
      *reinterpret_cast<uint2*>(xs + t * pitch + static_cast<int>(k) + cc * 8) = make_uint2(0, 0);
    }
  } else {
    for (int t = 0; t < m; ++t) {
      unsigned cur = 0;
      for (int64_t i = threadIdx.x; i < k; i += nthreads) cur = max(cur, static_cast<unsigned>(x[t * k + i]) & 0x7fffu);
      atomicMax(&max_s[t], cur);
    }
    lds_barrier();
    if (threadIdx.x < m) amax_s[threadIdx.x] = fmaxf(bf16_to_f32(max_s[threadIdx.x]), 1e-8f);
    lds_barrier();
    for (int c = threadIdx.x; c < m * kpad; c += nthreads) {
      const int t = c / kpad, col = c - t * kpad;
      int8_t q = 0;
      if (col < k) {
        q = static_cast<int8_t>(quant_code(x[t * k + col], 127.0f / amax_s[t]));
        if (write_out) xq_out[t * k + col] = q;
      }
      xs[t * pitch + col] = q;
    }
  }
  if (write_out && threadIdx.x < m) amax_out[threadIdx.x] = amax_s[threadIdx.x];
}

// RMSNorm + quantisation, any token count: per-token max|x * gain| (LDS
// atomics on the fp32 bit patterns) and fp64 sum of x^2 (LDS fp64 atomics);
// quant_s receives the quantisation scale 127 / max|v|, amax_s the
// de-quantisation a' = max|v| * r.
__device__ __forceinline__ void norm_values(const uint4& xc, const float* __restrict__ gain8, float (&v)[8],
                                            float (&xv)[8]) {
  const uint32_t w[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    xv[2 * q] = __uint_as_float(w[q] << 16);
    xv[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
  if (gain8) {
    const float4 g0 = *reinterpret_cast<const float4*>(gain8);
    const float4 g1 = *reinterpret_cast<const float4*>(gain8 + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = xv[i] * gv[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = xv[i];
  }
}

// the same from two float4 gains already in registers
__device__ __forceinline__ void norm_values_reg(const uint4& xc, const float4& g0, const float4& g1, bool has_gain,
                                                float (&v)[8], float (&xv)[8]) {
  const uint32_t w[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    xv[2 * q] = __uint_as_float(w[q] << 16);
    xv[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
  const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = has_gain ? xv[i] * gv[i] : xv[i];
}

// gains of the chunks whose activations prefetch_bf16 requests (single token)
__device__ __forceinline__ void prefetch_gain(float4 (&gc)[kCachedChunks][2], const float* __restrict__ gain,
                                              int64_t k) {
  const int total = static_cast<int>(k / 8);
#pragma unroll
  for (int j = 0; j < kCachedChunks; ++j) {
    const int c = threadIdx.x + j * static_cast<int>(blockDim.x);
    if (gain && c < total) {
      gc[j][0] = *reinterpret_cast<const float4*>(gain + c * 8);
      gc[j][1] = *reinterpret_cast<const float4*>(gain + c * 8 + 4);
    } else {
      gc[j][0] = gc[j][1] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    }
  }
}

// gains of the chunks whose activations prefetch_bf16_group requests
template <int WAVES>
__device__ __forceinline__ void prefetch_gain_group(float4 (&gc)[kCachedChunks][2], const float* __restrict__ gain, int m,
                                                    int64_t k) {
  const TokenGroup g = token_group_of<WAVES>(m);
  const int cpr = static_cast<int>(k / 8);
#pragma unroll
  for (int j = 0; j < kCachedChunks; ++j) {
    const int c = g.tt + j * 64 * g.G;
    if (gain && g.t < m && c < cpr) {
      gc[j][0] = *reinterpret_cast<const float4*>(gain + c * 8);
      gc[j][1] = *reinterpret_cast<const float4*>(gain + c * 8 + 4);
    } else {
      gc[j][0] = gc[j][1] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    }
  }
}

__device__ __forceinline__ float4 cached_gain(const float4 (&gc)[kCachedChunks][2], int j, int half) {
  float4 v = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
#pragma unroll
  for (int q = 0; q < kCachedChunks; ++q)
    if (q == j) v = gc[q][half];
  return v;
}

__device__ __forceinline__ uint32_t norm_code(float v, float s) {
  float r = rintf(v * s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu;
}

__device__ __forceinline__ double wave_sum_d(double v) { return wave_sum_f64(v); }

// a' and the quantisation scale of one token from max|v| and the sum of x^2
__device__ __forceinline__ void norm_scales(unsigned mx, double ss, int64_t k, float eps, float* amax_dst,
                                            float* quant_dst) {
  const double r = 1.0 / sqrt(ss / static_cast<double>(k) + static_cast<double>(eps));
  rmsnorm_scales(__uint_as_float(mx), r, amax_dst, quant_dst);
}

// Single token, vector path: wave shuffles and one LDS slot per wave for both
// reductions (no atomics, a fixed summation order).
template <int WAVES>
__device__ void stage_bf16_norm_single(int8_t* xs, float* amax_s, float* quant_s, unsigned* wmax_s, double* wss_s,
                                       const uint4 (&cache)[kCachedChunks], const float4 (&gcache)[kCachedChunks][2],
                                       const uint16_t* __restrict__ x, const float* __restrict__ gain, float eps,
                                       int64_t k, int kpad, int8_t* __restrict__ xq_out,
                                       float* __restrict__ amax_out) {
  const int nthreads = blockDim.x;
  const bool write_out = xq_out != nullptr && blockIdx.x == 0;
  const int total = static_cast<int>(k / 8);
  const bool has_gain = gain != nullptr;
  unsigned mx = 0;
  double ss = 0.0;
  int j = 0;
  // chunks j < kCachedChunks come from registers (activations and gains were
  // requested before the weight tiles); later ones are read here
  auto values = [&](int c, int jj, float (&v)[8], float (&xv)[8]) {
    if (jj < kCachedChunks)
      norm_values_reg(cached(cache, jj), cached_gain(gcache, jj, 0), cached_gain(gcache, jj, 1), has_gain, v, xv);
    else
      norm_values(*reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 8), gain ? gain + c * 8 : nullptr, v, xv);
  };
  for (int c = threadIdx.x; c < total; c += nthreads, ++j) {
    float v[8], xv[8];
    values(c, j, v, xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ss += static_cast<double>(xv[i]) * static_cast<double>(xv[i]);
      mx = max(mx, __float_as_uint(fabsf(v[i])));
    }
  }
  mx = wave_max(mx);
  ss = wave_sum_d(ss);
  if ((threadIdx.x & 63) == 0) {
    wmax_s[threadIdx.x >> 6] = mx;
    wss_s[threadIdx.x >> 6] = ss;
  }
  lds_barrier();
  unsigned mall = wmax_s[0];
  double sall = wss_s[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    mall = max(mall, wmax_s[w]);
    sall += wss_s[w];
  }
  float ap, qs;
  norm_scales(mall, sall, k, eps, &ap, &qs);
  if (threadIdx.x == 0) {
    amax_s[0] = ap;
    quant_s[0] = qs;
    if (write_out) amax_out[0] = ap;
  }
  j = 0;
  for (int c = threadIdx.x; c < total; c += nthreads, ++j) {
    float v[8], xv[8];
    values(c, j, v, xv);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= norm_code(v[i], qs) << (8 * i);
      hi |= norm_code(v[4 + i], qs) << (8 * i);
    }
    const uint2 q = make_uint2(lo, hi);
    *reinterpret_cast<uint2*>(xs + c * 8) = q;
    if (write_out) *reinterpret_cast<uint2*>(xq_out + c * 8) = q;
  }
  for (int c = total + threadIdx.x; c < kpad / 8; c += nthreads) *reinterpret_cast<uint2*>(xs + c * 8) = make_uint2(0, 0);
}

// Vector path, 1 < m <= WAVES tokens: the waves of a token group
// (token_group) reduce max|v| and the fp64 sum of x^2 over their chunks
// (per lane in chunk order, then across the wave with DPP), and the group's
// wave partials meet through one LDS slot per wave in wave order: a fixed
// summation order, no atomics.  The chunk order is prefetch_bf16_group's.
template <int WAVES>
__device__ void stage_bf16_norm_group(int8_t* xs, int pitch, float* amax_s, float* quant_s, unsigned* wmax_s,
                                      double* wss_s, const uint4 (&cache)[kCachedChunks],
                                      const float4 (&gcache)[kCachedChunks][2], const uint16_t* __restrict__ x,
                                      const float* __restrict__ gain, float eps, int m, int64_t k, int kpad,
                                      int8_t* __restrict__ xq_out, float* __restrict__ amax_out) {
  const bool write_out = xq_out != nullptr && blockIdx.x == 0;
  const TokenGroup g = token_group_of<WAVES>(m);
  const int G = g.G, t = g.t, tt = g.tt;
  const int step = 64 * G;
  const bool active = t < m;
  const int cpr = static_cast<int>(k / 8);
  const uint16_t* xr = x + static_cast<int64_t>(active ? t : 0) * k;
  const bool has_gain = gain != nullptr;
  auto values = [&](int c, int jj, float (&v)[8], float (&xv)[8]) {
    if (jj < kCachedChunks)
      norm_values_reg(cached(cache, jj), cached_gain(gcache, jj, 0), cached_gain(gcache, jj, 1), has_gain, v, xv);
    else
      norm_values(*reinterpret_cast<const uint4*>(xr + c * 8), gain ? gain + c * 8 : nullptr, v, xv);
  };
  unsigned mx = 0;
  double ss = 0.0;
  int j = 0;
  if (active)
    for (int c = tt; c < cpr; c += step, ++j) {
      float v[8], xv[8];
      values(c, j, v, xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss += static_cast<double>(xv[i]) * static_cast<double>(xv[i]);
        mx = max(mx, __float_as_uint(fabsf(v[i])));
      }
    }
  mx = wave_max(mx);
  ss = wave_sum_d(ss);
  if (G > 1) {  // uniform: m is the same for the whole workgroup
    if ((threadIdx.x & 63) == 0) {
      wmax_s[threadIdx.x >> 6] = mx;
      wss_s[threadIdx.x >> 6] = ss;
    }
    lds_barrier();
    // (w0 < WAVES for every wave, active or not)
    mx = group_slot_max(wmax_s, g.w0, G);
    ss = group_slot_sum(wss_s, g.w0, G);
  }
  if (!active) return;
  float ap, qs;
  norm_scales(mx, ss, k, eps, &ap, &qs);
  if (tt == 0) {
    amax_s[t] = ap;
    quant_s[t] = qs;
    if (write_out) amax_out[t] = ap;
  }
  int8_t* xrow = xs + t * pitch;
  j = 0;
  for (int c = tt; c < cpr; c += step, ++j) {
    float v[8], xv[8];
    values(c, j, v, xv);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= norm_code(v[i], qs) << (8 * i);
      hi |= norm_code(v[4 + i], qs) << (8 * i);
    }
    const uint2 q = make_uint2(lo, hi);
    *reinterpret_cast<uint2*>(xrow + c * 8) = q;
    if (write_out) *reinterpret_cast<uint2*>(xq_out + static_cast<int64_t>(t) * k + c * 8) = q;
  }
  for (int c = cpr + tt; c < kpad / 8; c += step) *reinterpret_cast<uint2*>(xrow + c * 8) = make_uint2(0, 0);
}

// Any token count: token t belongs to wave t % WAVES, whose lanes reduce it
// with shuffles (a fixed order, no atomics).  vec: k % 8 == 0, x and gain
// 16-byte aligned.
template <int WAVES>
__device__ void stage_bf16_norm(int8_t* xs, int pitch, float* amax_s, float* quant_s, const uint16_t* __restrict__ x,
                                const float* __restrict__ gain, float eps, int m, int64_t k, int kpad, bool vec,
                                int8_t* __restrict__ xq_out, float* __restrict__ amax_out) {
  const bool write_out = xq_out != nullptr && blockIdx.x == 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = wave; t < m; t += WAVES) {
    const uint16_t* xr = x + t * k;
    unsigned mx = 0;
    double ss = 0.0;
    if (vec) {
      for (int cc = lane; cc < k / 8; cc += 64) {
        float v[8], xv[8];
        norm_values(*reinterpret_cast<const uint4*>(xr + cc * 8), gain ? gain + cc * 8 : nullptr, v, xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ss += static_cast<double>(xv[i]) * static_cast<double>(xv[i]);
          mx = max(mx, __float_as_uint(fabsf(v[i])));
        }
      }
    } else {
      for (int64_t i = lane; i < k; i += 64) {
        const float xv = __uint_as_float(static_cast<uint32_t>(xr[i]) << 16);
        ss += static_cast<double>(xv) * static_cast<double>(xv);
        mx = max(mx, __float_as_uint(fabsf(gain ? xv * gain[i] : xv)));
      }
    }
    mx = wave_max(mx);
    ss = wave_sum_d(ss);
    if (lane == 0) norm_scales(mx, ss, k, eps, &amax_s[t], &quant_s[t]);
  }
  lds_barrier();
  const int nthreads = blockDim.x;
  if (vec) {
    const int cpr = static_cast<int>(k / 8);
    for (int c = threadIdx.x; c < m * cpr; c += nthreads) {
      const int t = c / cpr, cc = c - t * cpr;
      float v[8], xv[8];
      norm_values(*reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 8), gain ? gain + cc * 8 : nullptr, v, xv);
      const float qs = quant_s[t];
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= norm_code(v[i], qs) << (8 * i);
        hi |= norm_code(v[4 + i], qs) << (8 * i);
      }
      const uint2 q = make_uint2(lo, hi);
      *reinterpret_cast<uint2*>(xs + t * pitch + cc * 8) = q;
      if (write_out) *reinterpret_cast<uint2*>(xq_out + t * k + cc * 8) = q;
    }
    const int padc = (kpad - static_cast<int>(k)) / 8;
    for (int c = threadIdx.x; c < m * padc; c += nthreads) {
      const int t = c / padc, cc = c - t * padc;
      *reinterpret_cast<uint2*>(xs + t * pitch + static_cast<int>(k) + cc * 8) = make_uint2(0, 0);
    }
  } else {
    for (int c = threadIdx.x; c < m * kpad; c += nthreads) {
      const int t = c / kpad, col = c - t * kpad;
      int8_t q = 0;
      if (col < k) {
        const float xv = __uint_as_float(static_cast<uint32_t>(x[t * k + col]) << 16);
        q = static_cast<int8_t>(norm_code(gain ? xv * gain[col] : xv, quant_s[t]));
        if (write_out) xq_out[t * k + col] = q;
      }
      xs[t * pitch + col] = q;
    }
  }
  if (write_out && threadIdx.x < m) amax_out[threadIdx.x] = amax_s[threadIdx.x];
}

// fp32 activations, any token count: per-token max|x| (LDS atomics on the bit
// patterns), a' = max(., 1e-8), codes clamp(rint(x * (127 / a'))).  vec:
// k % 4 == 0 and x 16-byte aligned (chunks of 4 values).
__device__ void stage_f32(int8_t* xs, int pitch, float* amax_s, unsigned* max_s, const uint4 (&cache)[kCachedChunks],
                          const float* __restrict__ x, int m, int64_t k, int kpad, bool vec,
                          int8_t* __restrict__ xq_out, float* __restrict__ amax_out) {
  const int nthreads = blockDim.x;
  const bool write_out = xq_out != nullptr && blockIdx.x == 0;
  if (threadIdx.x < m) max_s[threadIdx.x] = 0u;
  lds_barrier();
  if (vec) {
    const int cpr = static_cast<int>(k / 4);
    const int total = m * cpr;
    int cur_t = -1;
    unsigned cur = 0;
    int j = 0;
    for (int c = threadIdx.x; c < total; c += nthreads, ++j) {
      const int t = c / cpr;
      if (t != cur_t) {
        if (cur_t >= 0) atomicMax(&max_s[cur_t], cur);
        cur_t = t;
        cur = 0;
      }
      const uint4 v = j < kCachedChunks ? cached(cache, j) : *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 4);
      cur = max(cur, max(max(v.x & 0x7fffffffu, v.y & 0x7fffffffu), max(v.z & 0x7fffffffu, v.w & 0x7fffffffu)));
    }
    if (cur_t >= 0) atomicMax(&max_s[cur_t], cur);
    lds_barrier();
    if (threadIdx.x < m) amax_s[threadIdx.x] = fmaxf(__uint_as_float(max_s[threadIdx.x]), 1e-8f);
    lds_barrier();
    j = 0;
    for (int c = threadIdx.x; c < total; c += nthreads, ++j) {
      const int t = c / cpr, cc = c - t * cpr;
      const uint4 v = j < kCachedChunks ? cached(cache, j) : *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 4);
      const float s = 127.0f / amax_s[t];
      const uint32_t q = norm_code(__uint_as_float(v.x), s) | (norm_code(__uint_as_float(v.y), s) << 8) |
                         (norm_code(__uint_as_float(v.z), s) << 16) | (norm_code(__uint_as_float(v.w), s) << 24);
      *reinterpret_cast<uint32_t*>(xs + t * pitch + cc * 4) = q;
      if (write_out) *reinterpret_cast<uint32_t*>(xq_out + t * k + cc * 4) = q;
    }
    const int padc = (kpad - static_cast<int>(k)) / 4;
    for (int c = threadIdx.x; c < m * padc; c += nthreads) {
      const int t = c / padc, cc = c - t * padc;
      *reinterpret_cast<uint32_t*>(xs + t * pitch + static_cast<int>(k) + cc * 4) = 0u;
    }
  } else {
    for (int t = 0; t < m; ++t) {
      unsigned cur = 0;
      for (int64_t i = threadIdx.x; i < k; i += nthreads) cur = max(cur, __float_as_uint(fabsf(x[t * k + i])));
      atomicMax(&max_s[t], cur);
    }
    lds_barrier();
    if (threadIdx.x < m) amax_s[threadIdx.x] = fmaxf(__uint_as_float(max_s[threadIdx.x]), 1e-8f);
    lds_barrier();
    for (int c = threadIdx.x; c < m * kpad; c += nthreads) {
      const int t = c / kpad, col = c - t * kpad;
      int8_t q = 0;
      if (col < k) {
        q = static_cast<int8_t>(norm_code(x[t * k + col], 127.0f / amax_s[t]));
        if (write_out) xq_out[t * k + col] = q;
      }
      xs[t * pitch + col] = q;
    }
  }
  if (write_out && threadIdx.x < m) amax_out[threadIdx.x] = amax_s[threadIdx.x];
}

__device__ __forceinline__ void prefetch_f32(uint4 (&cache)[kCachedChunks], const float* __restrict__ x, int m,
                                             int64_t k) {
  const int total = m * static_cast<int>(k / 4);
#pragma unroll
  for (int j = 0; j < kCachedChunks; ++j) {
    const int c = threadIdx.x + j * static_cast<int>(blockDim.x);
    cache[j] = c < total ? *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(c) * 4) : make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// main kernel: activation codes in LDS, persistent over row blocks
// ---------------------------------------------------------------------------

// Work items of a workgroup: its row blocks rb = blockIdx.x + i * gridDim.x,
// each cut into chunks of U * WAVES tiles (one chunk unless k is long).  A
// wave's share of item (rb, c) is tiles c*U*WAVES + wave + u*WAVES, u < U.
// With an up matrix (SwiGLU) an item walks 2 * kt_count tiles: the row
// block's gate tiles, then its up tiles.
//
// Binary weights (WB = 1): an item is one 1 KiB binary tile (512 columns),
// one 16-byte-per-lane load; kt_count is then the staged 256-column count
// (twice the binary tiles) and kt_real the binary tiles of a row block.
template <int WAVES, int U, bool SWIGLU, int WB = 2>
__device__ __forceinline__ void load_item(uint4 (&w)[U], const uint4* __restrict__ packed,
                                          const uint4* __restrict__ packed_u, int64_t rb, int c, int kt_count,
                                          int kt_real, int wave, int lane, bool valid) {
  // this row block's tiles as a buffer (empty past the last row block); an
  // item past the row block reads as zero and is never contracted
  const int row_tiles = WB == 1 ? kt_real : kt_count;
  const int64_t row_bytes = valid ? static_cast<int64_t>(row_tiles) * kTileBytes : 0;
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(packed + rb * row_tiles * 64), 0, static_cast<int>(row_bytes), kRawBuffer);
  const __amdgpu_buffer_rsrc_t ru = SWIGLU ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(packed_u + rb * row_tiles * 64), 0, static_cast<int>(row_bytes), kRawBuffer) : rg;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // uniform: the resource choice stays scalar
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kv = c * U * WAVES + wv + u * WAVES;
    const bool up = SWIGLU && kv >= kt_count;
    w[u] = load_tile_nt(up ? ru : rg, ((up ? kv - kt_count : kv) * 64 + lane) * 16);
  }
}

// Operand j of an item: its activation column offset (inside the lane's
// column group: 64 columns of a ternary tile, 128 of a binary one) and its
// expanded weight bytes.  Ternary: word j of the slot, 16 columns each.
// Binary: word j / 2 of the slot (32 columns), half j % 2 of the word.
template <int WB>
__device__ __forceinline__ int item_col(int item, int j) {
  return WB == 1 ? item * kBinTileCols + (j >> 1) * 32 + (j & 1) * 16 : item * kTileCols + 16 * j;
}

template <int WB>
constexpr int group_cols() {
  return WB == 1 ? 128 : 64;
}

template <int WB>
__device__ __forceinline__ v4i item_weights(const uint32_t (&words)[4], int j) {
  return WB == 1 ? expand_binary(words[j >> 1], j & 1) : expand_ternary(words[j]);
}

// SWIGLU: packed / gamma_p are the gate projection, packed_u / gamma_u the up
// projection; y receives h = silu(y_gate) * y_up [m][n] and acc_out (if set)
// the gate then the up accumulators, [m][2n].
// MULTI: the multi-token bf16 prologues (stage_bf16_group,
// stage_bf16_norm_group) are compiled in.  The host launches MULTI = false for
// a single bf16 token: that kernel carries only the single-token prologue
// (measured 1-2% faster per launch than one that carries both).
template <int WAVES, int U, int SRC, bool VEC, bool SWIGLU = false, int WB = 2, bool MULTI = true>
__global__ __launch_bounds__(WAVES * 64) void gemv_lds_kernel(const uint4* __restrict__ packed,
                                                              const float* __restrict__ gamma_p, Dequant dq, int64_t n,
                                                              int64_t k, int kt_count, int kt_real, int64_t rb_count,
                                                              const void* __restrict__ xsrc,
                                                              const float* __restrict__ amax_in, int m,
                                                              float* __restrict__ y, int32_t* __restrict__ acc_out,
                                                              int8_t* __restrict__ xq_out,
                                                              float* __restrict__ amax_out,
                                                              const float* __restrict__ gain, float eps,
                                                              const uint4* __restrict__ packed_u,
                                                              const float* __restrict__ gamma_u) {
  static_assert(WAVES >= 4, "one token group per wave in the epilogues (waves 0-3)");
  static_assert(WB == 2 || !SWIGLU, "binary weights: plain epilogue only");
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];
  __shared__ int red[WAVES * 4 * 64];
  __shared__ float amax_s[16];
  __shared__ float quant_s[SRC == kFromBf16Norm ? 16 : 1];
  __shared__ __attribute__((aligned(16))) double wss_s[SRC == kFromBf16Norm ? WAVES : 1];
  __shared__ unsigned max_s[16];
  __shared__ __attribute__((aligned(16))) unsigned wmax_s[WAVES];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;    // 64-column group of the lane inside a tile
  const int tok = lane & 15;  // token row of the lane's A operand
  const bool has_tok = tok < m;
  const int pitch = static_cast<int>(lds_pitch(kt_count));
  const int kpad = kt_count * kTileCols;
  const int kt_items = WB == 1 ? kt_count / 2 : SWIGLU ? 2 * kt_count : kt_count;  // items per row block
  const int nchunks = (kt_items + U * WAVES - 1) / (U * WAVES);
  constexpr int kOps = WB == 1 ? 8 : 4;  // MFMA operands per item

  int64_t rb = blockIdx.x;
  int c = 0;
  uint4 cache[kCachedChunks];
  float4 gcache[kCachedChunks][2];
  if (SRC == kFromBf16Norm && VEC && m == 1)
    prefetch_gain(gcache, gain, k);
  else if (SRC == kFromBf16Norm && VEC && MULTI && m <= WAVES)
    prefetch_gain_group<WAVES>(gcache, gain, m, k);
  if (VEC) {
    if (SRC == kFromCodes) {
      prefetch_codes(cache, static_cast<const int8_t*>(xsrc), m, k, kpad);
      __builtin_amdgcn_sched_barrier(0);  // the codes are requested before the weight tiles
    }
    else if (SRC == kFromF32)
      prefetch_f32(cache, static_cast<const float*>(xsrc), m, k);
    else if ((SRC == kFromBf16 && !MULTI) || m == 1)  // thread-major; unconditional without MULTI
      prefetch_bf16(cache, static_cast<const uint16_t*>(xsrc), m, k);
    else if (MULTI && m <= WAVES)  // bf16, with or without RMSNorm
      prefetch_bf16_group<WAVES>(cache, static_cast<const uint16_t*>(xsrc), m, k);
  }
  uint4 wcur[U];
  load_item<WAVES, U, SWIGLU, WB>(wcur, packed, packed_u, rb, c, kt_count, kt_real, wave, lane, rb < rb_count);
  // codes input: a' of the token this lane scales in the epilogue (token
  // 4g + wave, waves 0-3), into a register.  Only the epilogue waits for it,
  // by which time the first weight tiles, requested before it, have landed;
  // staged through LDS it would hold the prologue barrier, and with it the
  // next item's request, until those tiles arrive.  Every lane requests one
  // (clamped) a', so the request count is the same on every path and the
  // prologue's waits stay exact.
  float a_lane = 0.0f;
  if (SRC == kFromCodes) {
    const int ta = 4 * g + (wave & 3);
    a_lane = amax_in[(ta < m ? ta : m - 1) * dq.astride];
  }

  if (SRC == kFromCodes) {
    stage_codes(xs, pitch, cache, static_cast<const int8_t*>(xsrc), m, k, kpad, VEC);
  } else if (SRC == kFromBf16Norm && VEC && m == 1) {
    stage_bf16_norm_single<WAVES>(xs, amax_s, quant_s, wmax_s, wss_s, cache, gcache, static_cast<const uint16_t*>(xsrc),
                                  gain, eps, k, kpad, xq_out, amax_out);
  } else if (SRC == kFromBf16Norm && VEC && MULTI && m <= WAVES) {
    stage_bf16_norm_group<WAVES>(xs, pitch, amax_s, quant_s, wmax_s, wss_s, cache, gcache,
                                 static_cast<const uint16_t*>(xsrc), gain, eps, m, k, kpad, xq_out, amax_out);
  } else if (SRC == kFromBf16Norm) {
    stage_bf16_norm<WAVES>(xs, pitch, amax_s, quant_s, static_cast<const uint16_t*>(xsrc), gain, eps, m, k, kpad, VEC,
                           xq_out, amax_out);
  } else if (SRC == kFromF32) {
    stage_f32(xs, pitch, amax_s, max_s, cache, static_cast<const float*>(xsrc), m, k, kpad, VEC, xq_out, amax_out);
  } else if (VEC && m == 1) {
    stage_bf16_single<WAVES>(xs, amax_s, wmax_s, cache, static_cast<const uint16_t*>(xsrc), k, kpad, xq_out,
                             amax_out);
  } else if (VEC && MULTI && m <= WAVES) {
    stage_bf16_group<WAVES>(xs, pitch, amax_s, wmax_s, cache, static_cast<const uint16_t*>(xsrc), m, k, kpad, xq_out,
                            amax_out);
  } else {
    stage_bf16<!MULTI>(xs, pitch, amax_s, max_s, cache, static_cast<const uint16_t*>(xsrc), m, k, kpad, VEC, xq_out,
               amax_out);
  }
  lds_barrier();

  const float gamma = dq.row_scale ? 0.0f : *gamma_p;  // no tensor scale with per-row scales
  const float gamma_up = SWIGLU ? *gamma_u : 0.0f;
  const v4i zero4 = {0, 0, 0, 0};
  const int8_t* xrow = xs + (has_tok ? tok : 0) * pitch + g * group_cols<WB>();
  v4i acc = zero4;
  v4i acc_u = zero4;  // SwiGLU: the up projection's partial sums
  while (rb < rb_count) {
    int64_t rbn = rb;
    int cn = c + 1;
    if (cn == nchunks) {
      cn = 0;
      rbn = rb + gridDim.x;
    }
    uint4 wnext[U];
    load_item<WAVES, U, SWIGLU, WB>(wnext, packed, packed_u, rbn, cn, kt_count, kt_real, wave, lane, rbn < rb_count);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kv = c * U * WAVES + wave + u * WAVES;
      if (kv < kt_items) {
        const bool up = SWIGLU && kv >= kt_count;
        const int kt = up ? kv - kt_count : kv;
        const uint32_t words[4] = {wcur[u].x, wcur[u].y, wcur[u].z, wcur[u].w};
        if (up) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const v4i a = has_tok ? *reinterpret_cast<const v4i*>(xrow + kt * kTileCols + 16 * s) : zero4;
            acc_u = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, expand_ternary(words[s]), acc_u, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < kOps; ++j) {
            const v4i a = has_tok ? *reinterpret_cast<const v4i*>(xrow + item_col<WB>(kt, j)) : zero4;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, item_weights<WB>(words, j), acc, 0, 0, 0);
          }
        }
      }
    }
    if (SWIGLU && c == nchunks - 1) {
      // gate partials through LDS, then up partials; a wave < 4 owns token group r = wave
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
      lds_barrier();
      int vg = 0;
      if (wave < 4) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) vg += red[(w * 4 + wave) * 64 + lane];
      }
      lds_barrier();
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc_u[r];
      lds_barrier();
      const int64_t row = rb * kTileRows + tok;
      if (wave < 4) {
        int vu = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) vu += red[(w * 4 + wave) * 64 + lane];
        const int t = 4 * g + wave;
        if (t < m && row < n) {
          vg >>= kWeightShift;  // exact: the sums are multiples of 64
          vu >>= kWeightShift;
          const float at = SRC == kFromCodes ? a_lane : amax_s[t];
          const float gv = static_cast<float>(vg) * (gamma * at / 127.0f);
          const float uv = static_cast<float>(vu) * (gamma_up * at / 127.0f);
          y[t * n + row] = gv * uv / (1.0f + expf(-gv));
          if (acc_out) {
            acc_out[t * 2 * n + row] = vg;
            acc_out[t * 2 * n + n + row] = vu;
          }
        }
      }
      lds_barrier();
      acc = zero4;
      acc_u = zero4;
    } else if (c == nchunks - 1) {
      // lane holds 64 * acc for tokens 4g + r (r = 0..3) of weight row 16 rb + tok
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
      lds_barrier();
      const int64_t row = rb * kTileRows + tok;
      for (int r = wave; r < 4; r += WAVES) {
        int v = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += red[(w * 4 + r) * 64 + lane];
        const int t = 4 * g + r;
        if (t < m && row < n) {
          v >>= kWeightShift;  // exact: the sum is a multiple of 64
          const float ws = dq.row_scale ? half_bits_to_float(dq.row_scale[row]) : gamma;
          const float scale = ws * (SRC == kFromCodes ? a_lane : amax_s[t]) / dq.qdiv;
          y[t * n + row] = static_cast<float>(v) * scale;
          if (acc_out) acc_out[t * n + row] = v;
        }
      }
      lds_barrier();
      acc = zero4;
    }
    rb = rbn;
    c = cn;
#pragma unroll
    for (int u = 0; u < U; ++u) wcur[u] = wnext[u];
  }
}

// ---------------------------------------------------------------------------
// fallback: A operand read from the int8 codes in global memory
// ---------------------------------------------------------------------------

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

template <int WAVES, int U, bool VEC, int WB = 2>
__global__ __launch_bounds__(WAVES * 64) void gemv_global_kernel(const uint4* __restrict__ packed,
                                                                 const float* __restrict__ gamma_p, Dequant dq,
                                                                 int64_t n, int64_t k, int kt_count, int kt_real,
                                                                 const int8_t* __restrict__ xq,
                                                                 const float* __restrict__ amax, int m,
                                                                 float* __restrict__ y, int32_t* __restrict__ acc_out) {
  __shared__ int red[WAVES][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t rb = blockIdx.x;
  const int g = lane >> 4;
  const int tok = lane & 15;
  const bool has_tok = tok < m;
  const int8_t* xrow = xq + static_cast<int64_t>(has_tok ? tok : 0) * k;
  constexpr int kOps = WB == 1 ? 8 : 4;
  const int items = WB == 1 ? kt_count / 2 : kt_count;

  v4i acc = {0, 0, 0, 0};
  for (int i0 = wave; i0 < items; i0 += WAVES * U) {
    uint4 wv[U];
    v4i xv[U][kOps];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = i0 + u * WAVES;
      const bool in = it < items;
      wv[u] = in ? load_weights_nt(packed + (rb * kt_real + it) * 64 + lane)  // item it is tile it
                 : make_uint4(kZeroWord, kZeroWord, kZeroWord, kZeroWord);
#pragma unroll
      for (int j = 0; j < kOps; ++j)
        xv[u][j] = load_x16(xrow, static_cast<int64_t>(item_col<WB>(it, j)) + g * group_cols<WB>(), k,
                            in && has_tok, VEC);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t words[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
      for (int j = 0; j < kOps; ++j)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(xv[u][j], item_weights<WB>(words, j), acc, 0, 0, 0);
    }
  }
  const int64_t row = rb * kTileRows + tok;
  const float gamma = dq.row_scale ? 0.0f : *gamma_p;
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
  lds_barrier();
  for (int r = wave; r < 4; r += WAVES) {
    int v = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][r][lane];
    const int t = 4 * g + r;
    if (t < m && row < n) {
      v >>= kWeightShift;
      const float ws = dq.row_scale ? half_bits_to_float(dq.row_scale[row]) : gamma;
      const float scale = ws * amax[t * dq.astride] / dq.qdiv;
      y[t * n + row] = static_cast<float>(v) * scale;
      if (acc_out) acc_out[t * n + row] = v;
    }
  }
}

// Binary weights (WB = 1) stage the codes over an even number of 256-column
// tiles, since an item spans two.
inline int64_t staged_tiles(int64_t k, int wb) {
  const int64_t kt = k_tiles(k);
  return wb == 1 ? kt + (kt & 1) : kt;
}

template <int SRC, int WAVES, int U, bool SWIGLU = false, int WB = 2>
hipError_t launch_lds(const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k, const void* xsrc,
                      const float* amax_in, int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out,
                      const float* gain, float eps, hipStream_t s, bool vec, const void* packed_u = nullptr,
                      const float* gamma_u = nullptr) {
  const int kt = static_cast<int>(staged_tiles(k, WB));
  const int kt_real = static_cast<int>(WB == 1 ? bin_tiles(k) : k_tiles(k));
  const int64_t rbs = row_blocks(n);
  // balanced persistent grid: every workgroup takes the same number of row blocks (+-1)
  // the same number of resident waves whatever the workgroup size
  const int64_t cap = kMaxResidentGroups * kWaves / WAVES;
  const int64_t per = (rbs + cap - 1) / cap;
  const dim3 grid(static_cast<unsigned>((rbs + per - 1) / per));
  const size_t lds = lds_bytes(m, kt);
  const uint4* p = static_cast<const uint4*>(packed);
  const uint4* pu = static_cast<const uint4*>(packed_u);
  constexpr bool kBf16 = SRC == kFromBf16 || SRC == kFromBf16Norm;
  const bool one = kBf16 && m == 1;  // single bf16 token: the kernel without the multi-token prologues
  static const bool attr_vec = hipFuncSetAttribute(
      reinterpret_cast<const void*>(gemv_lds_kernel<WAVES, U, SRC, true, SWIGLU, WB>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes) == hipSuccess;
  static const bool attr_one = !kBf16 || hipFuncSetAttribute(
      reinterpret_cast<const void*>(gemv_lds_kernel<WAVES, U, SRC, true, SWIGLU, WB, !kBf16>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes) == hipSuccess;
  static const bool attr_any = hipFuncSetAttribute(
      reinterpret_cast<const void*>(gemv_lds_kernel<WAVES, U, SRC, false, SWIGLU, WB>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes) == hipSuccess;
  if (!(vec ? (one ? attr_one : attr_vec) : attr_any)) return hipErrorInvalidConfiguration;
  if (vec && one)
    gemv_lds_kernel<WAVES, U, SRC, true, SWIGLU, WB, !kBf16><<<grid, WAVES * 64, lds, s>>>(
        p, gamma, dq, n, k, kt, kt_real, rbs, xsrc, amax_in, static_cast<int>(m), y, acc, xq_out, amax_out, gain, eps,
        pu, gamma_u);
  else if (vec)
    gemv_lds_kernel<WAVES, U, SRC, true, SWIGLU, WB><<<grid, WAVES * 64, lds, s>>>(
        p, gamma, dq, n, k, kt, kt_real, rbs, xsrc, amax_in, static_cast<int>(m), y, acc, xq_out, amax_out, gain, eps,
        pu, gamma_u);
  else
    gemv_lds_kernel<WAVES, U, SRC, false, SWIGLU, WB><<<grid, WAVES * 64, lds, s>>>(
        p, gamma, dq, n, k, kt, kt_real, rbs, xsrc, amax_in, static_cast<int>(m), y, acc, xq_out, amax_out, gain, eps,
        pu, gamma_u);
  return hipGetLastError();
}

// U = items per wave per chunk. A chunk is U * waves items of one row block;
// each wave requests the next chunk's items before it consumes the current
// one's. The smallest U that covers the row block in one chunk is the start.
// U is then halved while a workgroup walks fewer than 8 chunks in all, as long
// as the last chunk of a row block stays at least half full. Shorter chunks
// put the first contraction and the last row block's tail closer to the bytes'
// arrival; a mostly empty last chunk costs a loop trip with idle waves. On the
// 70B-shaped down projection (112 items, 2 row blocks per workgroup) U = 2
// against 8 took the layer from 4.22 to 4.59 TB/s.
int items_per_wave(int64_t items, int64_t row_blocks_per_group, int waves) {
  int u = items <= waves ? 1 : items <= 2 * waves ? 2 : items <= 4 * waves ? 4 : 8;
  while (u > 1) {
    const int64_t half = u / 2 * waves;  // items per chunk after halving
    const int64_t last = items % half == 0 ? half : items % half;
    const int64_t walk = row_blocks_per_group * ((items + u * waves - 1) / (u * waves));
    if (walk >= 8 || 2 * last < half) break;
    u /= 2;
  }
  return u;
}

// SWIGLU items hold 2 * kt tiles (gate then up) and binary items two tiles.
template <int SRC, int W, bool SWIGLU, int WB>
hipError_t dispatch_lds_waves(const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k,
                              const void* xsrc, const float* amax_in, int64_t m, float* y, int32_t* acc,
                              int8_t* xq_out, float* amax_out, const float* gain, float eps, hipStream_t s, bool vec,
                              const void* packed_u, const float* gamma_u) {
  const int64_t items = WB == 1 ? staged_tiles(k, 1) / 2 : (SWIGLU ? 2 : 1) * k_tiles(k);
  const int64_t cap = kMaxResidentGroups * kWaves / W;  // the grid cap of launch_lds
  const int64_t per = (row_blocks(n) + cap - 1) / cap;
  const int u = items_per_wave(items, per, W);
  if (u == 1)
    return launch_lds<SRC, W, 1, SWIGLU, WB>(packed, gamma, dq, n, k, xsrc, amax_in, m, y, acc, xq_out, amax_out,
                                                  gain, eps, s, vec, packed_u, gamma_u);
  if (u == 2)
    return launch_lds<SRC, W, 2, SWIGLU, WB>(packed, gamma, dq, n, k, xsrc, amax_in, m, y, acc, xq_out, amax_out,
                                                  gain, eps, s, vec, packed_u, gamma_u);
  if (u == 4)
    return launch_lds<SRC, W, 4, SWIGLU, WB>(packed, gamma, dq, n, k, xsrc, amax_in, m, y, acc, xq_out, amax_out,
                                                  gain, eps, s, vec, packed_u, gamma_u);
  return launch_lds<SRC, W, 8, SWIGLU, WB>(packed, gamma, dq, n, k, xsrc, amax_in, m, y, acc, xq_out, amax_out,
                                                gain, eps, s, vec, packed_u, gamma_u);
}

// Workgroup size: one 16-wave workgroup per CU, or two 8-wave workgroups
// (the same resident waves), each of which stages the activations itself.
//   * Fused quantisation + decode: two 8-wave workgroups for rows of at most 3072
//     values, where staging is cheap and the second workgroup overlaps the
//     first one's prologue and tail (fused, one token, us per launch, 16 vs
//     2 x 8 waves: 13824 x 2560 5.27 / 4.54, 3840 x 2560 3.13 / 2.92,
//     2048 x 2048 2.91 / 2.71); 16 waves on longer rows (28672 x 4096 8.38 /
//     9.03, 4096 x 14336 5.80 / 7.31, 8192 x 28672 13.56 / 17.79).
//   * RMSNorm prologue: two 8-wave workgroups on rows of at most 8192 values
//     (3840 x 2560: 4.39 against 4.70 us per launch).  On longer rows every
//     workgroup's fp64 RMSNorm pass over the row dominates, and two
//     workgroups per CU do it twice: 4096 x 14336 took 9.55 us with 8 waves
//     and 8.40 with 16, 8192 x 28672 24.5 and 16.8.
template <int SRC, bool SWIGLU = false, int WB = 2>
hipError_t dispatch_lds(const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k, const void* xsrc,
                        const float* amax_in, int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out,
                        const float* gain, float eps, hipStream_t s, bool vec, const void* packed_u = nullptr,
                        const float* gamma_u = nullptr) {
  if constexpr (SRC == kFromBf16Norm && !SWIGLU) {
    if (k <= 8192)
      return dispatch_lds_waves<SRC, 8, SWIGLU, WB>(packed, gamma, dq, n, k, xsrc, amax_in, m, y, acc, xq_out,
                                                    amax_out, gain, eps, s, vec, packed_u, gamma_u);
  }
  if constexpr (SRC == kFromBf16 && !SWIGLU && WB == 2) {
    if (k <= 3072)
      return dispatch_lds_waves<SRC, 8, SWIGLU, WB>(packed, gamma, dq, n, k, xsrc, amax_in, m, y, acc, xq_out,
                                                    amax_out, gain, eps, s, vec, packed_u, gamma_u);
  }
  return dispatch_lds_waves<SRC, kWaves, SWIGLU, WB>(packed, gamma, dq, n, k, xsrc, amax_in, m, y, acc, xq_out,
                                                     amax_out, gain, eps, s, vec, packed_u, gamma_u);
}

template <int WB>
hipError_t launch_global(const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k, const int8_t* xq,
                         const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s, bool vec) {
  const int kt = static_cast<int>(staged_tiles(k, WB));
  const int kt_real = static_cast<int>(WB == 1 ? bin_tiles(k) : k_tiles(k));
  const dim3 grid(static_cast<unsigned>(row_blocks(n)));
  const uint4* p = static_cast<const uint4*>(packed);
  if (vec)
    gemv_global_kernel<4, 4, true, WB><<<grid, 256, 0, s>>>(p, gamma, dq, n, k, kt, kt_real, xq, amax,
                                                            static_cast<int>(m), y, acc);
  else
    gemv_global_kernel<4, 4, false, WB><<<grid, 256, 0, s>>>(p, gamma, dq, n, k, kt, kt_real, xq, amax,
                                                             static_cast<int>(m), y, acc);
  return hipGetLastError();
}

}  // namespace

bool gemv_fits_lds(int64_t m, int64_t k) { return lds_bytes(m, k_tiles(k)) <= kMaxLdsBytes; }

// SwiGLU decode path: codes staged in LDS; an item's tiles are the gate row
// block followed by the up row block.
hipError_t launch_gemv_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u, const float* gamma_u,
                              int64_t f, int64_t k, const int8_t* xq, const float* amax, int64_t m, float* h,
                              int32_t* acc, hipStream_t s) {
  if (!gemv_fits_lds(m, k)) return hipErrorInvalidValue;
  const bool vec = (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
  return dispatch_lds<kFromCodes, true>(packed_g, gamma_g, kTokenDequant, f, k, xq, amax, m, h, acc, nullptr, nullptr, nullptr, 0.0f,
                                        s, vec, packed_u, gamma_u);
}

hipError_t launch_norm_quant_gemv_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u,
                                         const float* gamma_u, int64_t f, int64_t k, const uint16_t* x,
                                         const float* gain, float eps, int64_t m, float* h, int32_t* acc,
                                         int8_t* xq_out, float* amax_out, hipStream_t s) {
  const bool vec = (k % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (gain == nullptr || reinterpret_cast<uintptr_t>(gain) % 16 == 0) &&
                   (xq_out == nullptr || reinterpret_cast<uintptr_t>(xq_out) % 8 == 0);
  return dispatch_lds<kFromBf16Norm, true>(packed_g, gamma_g, kTokenDequant, f, k, x, nullptr, m, h, acc, xq_out, amax_out, gain, eps,
                                           s, vec, packed_u, gamma_u);
}

hipError_t launch_quant_gemv_f32(const void* packed, const float* gamma, int64_t n, int64_t k, const float* x,
                                 int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out, hipStream_t s) {
  const bool vec = (k % 4 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (xq_out == nullptr || reinterpret_cast<uintptr_t>(xq_out) % 4 == 0);
  return dispatch_lds<kFromF32>(packed, gamma, kTokenDequant, n, k, x, nullptr, m, y, acc, xq_out, amax_out, nullptr, 0.0f, s, vec);
}

hipError_t launch_gemv_ex(const void* packed, bool binary, const float* gamma, Dequant dq, int64_t n, int64_t k,
                          const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  const bool vec = (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
  if (binary) {
    if (lds_bytes(m, staged_tiles(k, 1)) <= kMaxLdsBytes)
      return dispatch_lds<kFromCodes, false, 1>(packed, gamma, dq, n, k, xq, amax, m, y, acc, nullptr, nullptr, nullptr,
                                                0.0f, s, vec);
    return launch_global<1>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s, vec);
  }
  if (gemv_fits_lds(m, k))
    return dispatch_lds<kFromCodes>(packed, gamma, dq, n, k, xq, amax, m, y, acc, nullptr, nullptr, nullptr, 0.0f, s,
                                    vec);
  return launch_global<2>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s, vec);
}

hipError_t launch_gemv(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                       const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  return launch_gemv_ex(packed, false, gamma, kTokenDequant, n, k, xq, amax, m, y, acc, s);
}

bool gemv_binary_fits_lds(int64_t m, int64_t k) { return lds_bytes(m, staged_tiles(k, 1)) <= kMaxLdsBytes; }

hipError_t launch_quant_gemv_binary(const void* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                                    int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out, hipStream_t s) {
  if (!gemv_binary_fits_lds(m, k)) return hipErrorInvalidValue;
  const bool vec = (k % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (xq_out == nullptr || reinterpret_cast<uintptr_t>(xq_out) % 8 == 0);
  return dispatch_lds<kFromBf16, false, 1>(packed, scale, kTokenDequant, n, k, x, nullptr, m, y, acc, xq_out,
                                           amax_out, nullptr, 0.0f, s, vec);
}

hipError_t launch_quant_gemv(const void* packed, const float* gamma, int64_t n, int64_t k, const uint16_t* x,
                             int64_t m, float* y, int32_t* acc, int8_t* xq_out, float* amax_out, hipStream_t s) {
  const bool vec = (k % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (xq_out == nullptr || reinterpret_cast<uintptr_t>(xq_out) % 8 == 0);
  return dispatch_lds<kFromBf16>(packed, gamma, kTokenDequant, n, k, x, nullptr, m, y, acc, xq_out, amax_out, nullptr, 0.0f, s, vec);
}

hipError_t launch_norm_quant_gemv(const void* packed, const float* gamma, int64_t n, int64_t k, const uint16_t* x,
                                  const float* gain, float eps, int64_t m, float* y, int32_t* acc, int8_t* xq_out,
                                  float* amax_out, hipStream_t s) {
  const bool vec = (k % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (gain == nullptr || reinterpret_cast<uintptr_t>(gain) % 16 == 0) &&
                   (xq_out == nullptr || reinterpret_cast<uintptr_t>(xq_out) % 8 == 0);
  return dispatch_lds<kFromBf16Norm>(packed, gamma, kTokenDequant, n, k, x, nullptr, m, y, acc, xq_out, amax_out, gain, eps, s, vec);
}

}  // namespace bitlinear
