// Batched (prefill) BitLinear forward for any token count.
//
// "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
// "The Mathematical Mechanism", items 3-4 (ternary x int8 contraction in
// int32, de-quantisation by gamma * a' / 127).  With many tokens per weight
// the contraction is dense and compute-bound ("BitNet 1-bit LLM Inference
// Framework", section "Scalability with Thread Count": prompt processing is
// compute-intensive), so it runs on the int8 matrix cores.
//
// Tiling: a workgroup owns a BM x BN output tile (tokens x weight rows) and
// walks k in 256-column steps, the width of one packed weight tile.  A step's
// operands are the BM x 256 int8 activation tile and the BN/16 packed weight
// tiles (1 KiB each, copied verbatim: still 2 bits per weight).  Its waves
// are WM x WN blocks of the tile, or KG groups of them that share the tile
// and each multiply part of every step (gemm_mfma_kernel).
//
// Matrix-core instruction: v_mfma_i32_32x32x32_i8 (measured ~4.5 POPS on
// MI355X, against ~2.5-3.2 for the 16x16x64 form).  A 32-bit word of a
// packed slot holds 16 columns of one weight row; expand_ternary turns it
// into the int8 operand 64 * w with one shift and one mask per 4 weights,
// reused for every 32-token block of the wave.  The accumulators hold
// 64 * acc exactly; the epilogue shifts, scales by gamma * a'[t] / 127 and
// stores fp32.  The order in which a step's eight MFMAs take the columns is
// each kernel's own (gemm_mfma_kernel: chunk 8h + q of the step for MFMA q
// and lane half h, so a 16-byte slot serves four MFMAs; gemm_kernel: words
// 2(q % 2) + h of slot (r % 16) + 16(q / 2)); the activation operand takes
// the same columns.
//
// Main path (k % 16 == 0, 16-byte aligned codes): gemm_mfma_kernel, with the
// operands in LDS stages filled by buffer-to-LDS copies and one barrier per
// step.  Otherwise gemm_kernel, register-staged over two stages, handles any
// k and alignment.
//
// The per-token output scale gamma * a'[t] / 127 is computed once per
// workgroup into LDS, so the epilogue is stores only.
//
// Workgroup order is XCD-aware: hardware deals workgroups to the 8 XCDs
// round-robin, so the linear id is remapped to give each XCD a contiguous
// range of tiles in (weight tile, token tile) order -- the token tiles that
// share a weight tile run on one XCD, at the same time, and share its L2.
#include "bitlinear_internal.hpp"

namespace bitlinear {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kAPitch = kTileCols + 16;  // LDS row pitch of the activation tile (bytes)
constexpr int kXcds = 8;

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

// WB: 2 = ternary, 1 = binary.  Bytes of one row block's weights per
// 256-column k-step: a whole ternary tile, or one half of a binary tile.
template <int WB>
constexpr int wtile_bytes() {
  return WB == 1 ? kBinStepBytes : kTileBytes;
}

// The lane's 16-byte weight slot for 64-column group g of a k-step, and its
// operand for step `half` (columns 64g + 32 half + 16h + [0, 16)).  Ternary:
// slot g (64 columns), word 2 half + h.  Binary: slot g / 2 of the half tile
// (128 columns), word 2 (g % 2) + half, half h of that word.
template <int WB>
__device__ __forceinline__ int group_offset(int g) {
  return WB == 1 ? (g >> 1) * 256 : g * 256;
}

// A lane's part of a slot: binary lanes keep the whole slot; ternary lanes of
// half h need only words h and 2 + h, fetched at a lane-dependent offset by
// one two-dword LDS read (no per-lane select, half the bytes).
template <int WB>
__device__ __forceinline__ uint4 read_slot(const uint8_t* p, int h) {
  if (WB == 1) return *reinterpret_cast<const uint4*>(p);
  const uint32_t* w = reinterpret_cast<const uint32_t*>(p) + h;
  return make_uint4(w[0], w[2], 0, 0);
}

template <int WB>
__device__ __forceinline__ v4i slot_operand(uint4 slot, int g, int half, int h) {
  // g and half are compile-time constants at every call
  if (WB == 1) {
    const uint32_t word = (g & 1) ? (half == 0 ? slot.z : slot.w) : (half == 0 ? slot.x : slot.y);
    return expand_binary(word, h);
  }
  return expand_ternary(half == 0 ? slot.x : slot.y);  // words h and 2 + h (read_slot)
}

template <int WB>
__device__ __forceinline__ int slot_offset(int b_row) {  // + nb * 2 row blocks + group_offset(g)
  return (b_row >> 4) * wtile_bytes<WB>() + (b_row & 15) * 16;
}

// Output scale of token t (LDS-staged): gamma * a / qdiv, or a alone when the
// scale is per weight row (then applied in the epilogue).
__device__ __forceinline__ float token_scale(const float* gamma_p, Dequant dq, const float* amax, int64_t t) {
  const float a = amax[t * dq.astride];
  return dq.row_scale ? a : *gamma_p * a / dq.qdiv;
}

__device__ __forceinline__ float out_scale(Dequant dq, float staged, int64_t j) {
  return dq.row_scale ? half_bits_to_float(dq.row_scale[j]) * staged / dq.qdiv : staged;
}

template <int BM, int BN, int WB = 2>
struct TileShape {
  static constexpr int kABytes = BM * kAPitch;
  static constexpr int kBBytes = (BN / kTileRows) * wtile_bytes<WB>();
  static constexpr int kStage = kABytes + kBBytes;
  static constexpr int kLds = 2 * kStage;
};

template <int BM, int BN, int WM, int WN, bool VEC, int WB = 2>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const uint4* __restrict__ packed,
                                                           const float* __restrict__ gamma_p, Dequant dq, int64_t n,
                                                           int64_t k,
                                                           int kt_count, const int8_t* __restrict__ xq,
                                                           const float* __restrict__ amax, int64_t m, int mt_count,
                                                           int nt_count, float* __restrict__ y,
                                                           int32_t* __restrict__ acc_out) {
  static_assert(WM * WN == kThreads / 64, "4 waves");
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;  // 32 x 32 output blocks per wave
  constexpr int A_PER = BM * 16 / kThreads;  // 16-byte activation chunks per thread per step
  constexpr int TB = wtile_bytes<WB>();
  constexpr int CPT = TB / 16;  // 16-byte chunks per weight tile
  constexpr int B_CHUNKS = (BN / kTileRows) * CPT;
  constexpr int B_PER = (B_CHUNKS + kThreads - 1) / kThreads;
  using TS = TileShape<BM, BN, WB>;
  static_assert(A_PER >= 1 && MB >= 1 && NB >= 1 && TM % 32 == 0 && TN % 32 == 0, "tile too small");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps stage addresses scalar
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31;  // operand row (token for A, weight row for B)
  const int h = lane >> 5;    // which 16 of the step's 32 columns

  // XCD-aware tile order
  const int total = mt_count * nt_count;
  int id = blockIdx.x;
  if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
  const int nt = id / mt_count, mt = id - nt * mt_count;
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int64_t n0 = static_cast<int64_t>(nt) * BN;
  const int64_t rb0 = n0 / kTileRows;
  const int64_t rb_count = row_blocks(n);
  const int bt = (kt_count + 1) / 2;  // binary tiles per row block

  uint4 areg[A_PER];
  uint4 breg[B_PER];
  auto load_global = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + kThreads * i;
      areg[i] = load_a16(xq, m0 + (c >> 4), static_cast<int64_t>(kt) * kTileCols + (c & 15) * 16, m, k, VEC);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + kThreads * i;
      const int64_t rbg = rb0 + c / CPT;
      // binary: half kt % 2 of tile kt / 2 (bt tiles per row block)
      const int64_t src = WB == 1 ? (rbg * bt + kt / 2) * 64 + (kt & 1) * 32 + c % CPT
                                  : (rbg * kt_count + kt) * CPT + c % CPT;
      breg[i] = (c < B_CHUNKS && rbg < rb_count) ? packed[src]
                                                 : make_uint4(kZeroWord, kZeroWord, kZeroWord, kZeroWord);
    }
  };
  auto store_lds = [&](int stage) {
    uint8_t* As = smem + stage * TS::kStage;
    uint4* Bs = reinterpret_cast<uint4*>(As + TS::kABytes);
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<uint4*>(As + (c >> 4) * kAPitch + (c & 15) * 16) = areg[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + kThreads * i;
      if (c < B_CHUNKS) Bs[c] = breg[i];
    }
  };

  v16i acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v16i{};

  // per-lane LDS offsets: A row (token), B slot of the lane's weight row
  const int a_off = (wm * TM + l32) * kAPitch + 16 * h;
  const int b_row = wn * TN + l32;           // + nb * 32
  const int b_off = slot_offset<WB>(b_row);  // + nb * 2 tiles + g * 16 slots

  __shared__ float scale_s[BM];
  if (tid < BM) {
    const int64_t t = m0 + tid;
    scale_s[tid] = t < m ? token_scale(gamma_p, dq, amax, t) : 0.0f;
  }

  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < kt_count; ++kt) {
    const bool more = kt + 1 < kt_count;
    if (more) load_global(kt + 1);
    const uint8_t* As = smem + (kt & 1) * TS::kStage;
    const uint8_t* Bs = As + TS::kABytes;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // the lane's packed slot for column group g: words h (columns 64g + 16h
      // + [0,16)) and 2 + h (columns 64g + 32 + 16h + [0,16))
      uint4 slot[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        slot[nb] = read_slot<WB>(Bs + b_off + nb * 2 * TB + group_offset<WB>(g), h);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        v4i b[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) b[nb] = slot_operand<WB>(slot[nb], g, half, h);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const v4i a = *reinterpret_cast<const v4i*>(As + a_off + mb * 32 * kAPitch + g * 64 + half * 32);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
    if (more) store_lds((kt + 1) & 1);
    __syncthreads();
  }

  // 32 x 32 block layout: element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tl = wm * TM + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const int64_t t = m0 + tl;
      if (t >= m) continue;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t j = n0 + wn * TN + nb * 32 + l32;
        if (j < n) {
          const int v = acc[mb][nb][r] >> kWeightShift;  // exact: multiples of 64
          y[t * n + j] = static_cast<float>(v) * out_scale(dq, scale_s[tl], j);
          if (acc_out) acc_out[t * n + j] = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel: activations through LDS, weights straight to registers
// ---------------------------------------------------------------------------
//
// A workgroup of WM x WN = 4 waves owns a BM x BN output tile, BM = WM * MB *
// 32 tokens and BN = WN * NB * 32 weight rows; each wave holds MB x NB
// accumulator blocks of 32 x 32.  It walks k in 256-column steps:
//   * the BM x 256 activation codes of a step are copied into LDS by
//     buffer-to-LDS loads (two stages, one step in flight), read by every
//     wave of the same token rows;
//   * each wave reads the packed weights of its own rows straight into
//     registers (no other wave uses them), one step ahead, still 2 bits per
//     weight, and expands each 16-column word once for its MB token blocks.
//
// k order inside a step: MFMA step q (0..7) of the lanes of half h takes the
// 16 columns of chunk 8h + q.  A ternary lane (weight row r, half h) holds
// slots (r % 16) + 32h and (r % 16) + 32h + 16 of its row block's tile:
// columns 128h + [0, 128), words 0-3 of the first slot for q < 4 and of the
// second for q >= 4.  A binary lane holds slot (r % 16) + 16h of the step's
// half tile, word q / 2, half q % 2.  Either way a lane's weight bytes are
// whole 16-byte slots, and a wave's loads cover contiguous 256-byte runs.
//
// The activation tile is stored with chunk c of row t at position
// c ^ (t % 16), so the 16 lanes of a half that read one chunk of 16
// consecutive rows meet 16 different 16-byte bank groups.  The LDS address of
// a lane's chunk for each q is computed once; the token blocks and the two
// stages add constants.
//
// Reads past a buffer descriptor's byte count return zeros: token rows past
// m, weight row blocks past n; columns past k meet zero ternary weights (the
// packed padding), and for binary weights (whose padding is +1) their
// activation chunks are sent past the descriptor.

constexpr int kRawBufferWord3 = 0x00020000;     // raw (untyped) buffer, 32-bit data format
constexpr int kOffPastDescriptor = 0x7fffff00;  // byte offset beyond any descriptor's range (reads return 0)

#define BITLINEAR_LDS(p) ((__attribute__((address_space(3))) void*)(p))

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const v4u t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4] and lgkmcnt [11:8] at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Deeper rings (S > 2 stages) copy both operands with buffer-to-LDS loads
// written as inline assembly, so the compiler tracks none of them: it would
// otherwise assume any outstanding copy may write the stage being read and
// wait for all of them before every LDS read.  The kernel waits for its own
// copies instead (copies_landed), in the same assembly block as the barrier,
// with a memory clobber so no LDS read moves above it.  These copies have no
// output registers.
typedef unsigned v4u_d __attribute__((ext_vector_type(4)));

// raw buffer descriptor (32-bit untyped records, no stride) of `bytes` bytes at `base`
__device__ __forceinline__ v4u_d raw_descriptor(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4u_d r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bytes));
  r.w = kRawBufferWord3;
  return r;
}

// 16 bytes per lane from byte `voff` of the buffer into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void lds_copy16(v4u_d rsrc, int voff, uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

// wait until at most N of the wave's copies are outstanding, then the workgroup barrier
template <int N>
__device__ __forceinline__ void copies_landed() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(BITLINEAR_LDS(p)));
}

// weight operand of MFMA step q from a lane's slots (BREGS 16-byte slots per 32-row block)
template <int WB>
__device__ __forceinline__ v4i weight_operand(const uint4* s, int q) {
  if (WB == 1) {
    const uint4 v = s[0];
    const uint32_t w = (q >> 1) == 0 ? v.x : (q >> 1) == 1 ? v.y : (q >> 1) == 2 ? v.z : v.w;
    return expand_binary(w, q & 1);
  }
  const uint4 v = s[q >> 2];
  const uint32_t w = (q & 3) == 0 ? v.x : (q & 3) == 1 ? v.y : (q & 3) == 2 ? v.z : v.w;
  return expand_ternary(w);
}

// SWIGLU: packed_b / gamma_p are the gate projection, packed_u / gamma_u the
// up projection (both [n][k], n = features); a wave's first NB / 2 blocks are
// gate rows and its last NB / 2 the up rows of the same features, so the
// workgroup covers BN / 2 features and writes h = silu(y_gate) * y_up to
// y [m][n] (acc_out, if set, is [m][2n]: gate accumulators, then up).
//
// SPLIT: the grid holds ceil(kt_count / kt_per) k-slices of every output tile
// (slice-major); a workgroup walks k-steps [slice * kt_per, ...) and adds its
// partial sums, exact in int32, to split_acc with atomics (zeroed before,
// converted by split_finish_kernel after).
//
// KG > 1 (ring configurations only): KG groups of WM x WN waves share the
// workgroup's tile; group g takes MFMA steps q in [8g / KG, 8(g + 1) / KG)
// of every k-step, so each wave holds a full MB x NB block of the tile with
// 1 / KG of its MFMAs, and the CU keeps KG times the waves of one tile.  The
// groups' partial sums (exact int32) meet in LDS after the last step and the
// first group writes the outputs.
template <int MB, int NB, int WM, int WN, int S, int OCC, int WB = 2, bool SWIGLU = false, bool SPLIT = false,
          int KG = 1>
__global__ __launch_bounds__(64 * WM * WN * KG, OCC) void gemm_mfma_kernel(
    const uint8_t* __restrict__ packed_b, const float* __restrict__ gamma_p, Dequant dq, int64_t n, int64_t k,
    int kt_count, const int8_t* __restrict__ xq, const float* __restrict__ amax, int64_t m, int mt_count,
    int nt_count, float* __restrict__ y, int32_t* __restrict__ acc_out, const uint8_t* __restrict__ packed_u,
    const float* __restrict__ gamma_u, int kt_per, int32_t* __restrict__ split_acc) {
  static_assert(WM * WN * KG == 4 || WM * WN * KG == 8, "4 or 8 waves");
  static_assert(KG == 1 || KG == 2, "k-groups");
  static_assert(KG == 1 || (S > 2 && !SWIGLU && WB == 2), "k-groups: ternary ring configurations, plain epilogue");
  static_assert(WB == 2 || !SWIGLU, "binary weights: plain epilogue");
  static_assert(!(SPLIT && SWIGLU), "k-slices: plain epilogue only");
  static_assert(!SWIGLU || NB % 2 == 0, "gate and up blocks pair up inside a wave");
  constexpr int BM = WM * MB * 32;
  constexpr int BN = WN * NB * 32;
  constexpr int FB = SWIGLU ? BN / 2 : BN;          // output columns (features) per workgroup
  constexpr int kStage = BM * kTileCols;            // activation bytes per stage
  constexpr int kWavesWG = WM * WN * KG;
  constexpr int kDma = BM / (4 * kWavesWG);         // 1 KiB activation copies per wave per stage
  static_assert(kDma >= 1 && kDma * 4 * kWavesWG == BM, "activation copies split over the waves");
  constexpr int QN = 8 / KG;                        // MFMA steps per k-step and wave
  constexpr int BREGS = WB == 1 ? 1 : 2;            // 16-byte slots per 32-row block per step
  constexpr int NBH = SWIGLU ? NB / 2 : NB;         // 32-row blocks per wave and matrix

  static_assert(S >= 2 && S <= 6, "2..6 stages");
  // S = 2: activations in two stage arrays (one per stage: the compiler tells
  // their outstanding copies apart), weights in registers.  S > 2: a ring of
  // S stages, each the activation tile followed by the weight tiles of the
  // workgroup's row blocks, filled by untracked copies.
  constexpr bool kRing = S > 2;
  constexpr int TBS = WB == 1 ? kBinStepBytes : kTileBytes;           // one row block's bytes per k-step
  constexpr int kStageBytes = kStage + (kRing ? (BN / kTileRows) * TBS : 0);
  constexpr int kBDma = kRing ? (BN / kTileRows) * TBS / 1024 / kWavesWG : 0;  // weight copies per wave per stage
  static_assert(!kRing || (BN / kTileRows) * TBS % (1024 * kWavesWG) == 0, "weight copies split over the waves");
  // the k-groups' partial sums after the last step (groups 1 .. KG - 1), in the ring's memory
  constexpr int kRedBytes = (KG - 1) * WM * WN * MB * NB * 16 * 64 * 4;
  constexpr int kRingBytes = S * kStageBytes > kRedBytes ? S * kStageBytes : kRedBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kRing ? 16 : kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kRing ? 16 : kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing ? kRingBytes : 16];
  __shared__ __attribute__((aligned(16))) float scale_s[BM];
  __shared__ __attribute__((aligned(16))) float scale_u[SWIGLU ? BM : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps stage addresses scalar
  const int kg = wave / (WM * WN);                              // k-group
  const int wl = wave - kg * (WM * WN);                         // wave inside the group
  const int wm = wl / WN, wn = wl % WN;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int q0 = KG == 1 ? 0 : kg * QN;                         // first MFMA step of the group

  const int total = mt_count * nt_count;
  int id = blockIdx.x;
  int kt_begin = 0, kt_end = kt_count;
  if (SPLIT) {
    const int slice = id / total;
    id -= slice * total;
    kt_begin = slice * kt_per;
    kt_end = kt_begin + kt_per < kt_count ? kt_begin + kt_per : kt_count;
  }
  // XCD-aware order: the token tiles of one weight tile run on one XCD and share its L2
  // (with SPLIT and total % 8 == 0 the hardware XCD of a workgroup is still id % 8)
  if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
  const int nt = id / mt_count, mt = id - nt * mt_count;
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int64_t f0 = static_cast<int64_t>(nt) * FB;
  const int64_t rb0 = f0 / kTileRows;
  const int64_t rb_count = row_blocks(n);

  // per-token output scale gamma * a'[t] / 127 (one per matrix), staged once
  if (tid < BM) {
    const int64_t t = m0 + tid;
    scale_s[tid] = t < m ? token_scale(gamma_p, dq, amax, t) : 0.0f;
    if (SWIGLU) scale_u[tid] = t < m ? *gamma_u * amax[t] / 127.0f : 0.0f;
  }

  // operand descriptors: this workgroup's token rows and weight row blocks
  const int64_t rows_here = m - m0 < BM ? m - m0 : BM;
  const int64_t rbs_here = rb_count - rb0 < FB / kTileRows ? rb_count - rb0 : FB / kTileRows;
  const int row_tiles = WB == 1 ? (kt_count + 1) / 2 : kt_count;  // 1 KiB tiles per row block
  const int64_t row_bytes = static_cast<int64_t>(row_tiles) * kTileBytes;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(xq + m0 * k), 0, static_cast<int>(rows_here * k), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed_b + rb0 * row_bytes), 0, static_cast<int>(rbs_here * row_bytes), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t u_rsrc = SWIGLU ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed_u + rb0 * row_bytes), 0, static_cast<int>(rbs_here * row_bytes), kRawBufferWord3)
                                               : b_rsrc;
  const int k32 = static_cast<int>(k);

  // activation copies: copy i of this wave moves rows 4 * (wave * kDma + i) + lane / 16,
  // stored chunk lane % 16 = logical chunk (lane % 16) ^ (row % 16)
  int a_src[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int row = 4 * (wave * kDma + i) + (lane >> 4);
    a_src[i] = row * k32 + (((lane & 15) ^ (row & 15)) << 4);
  }
  // (the whole offset goes in the range-checked part: a chunk past the end
  // of the last token row reads zero instead of the memory beyond it)
  auto issue_a = [&](uint8_t* stage, int kt) {
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      int off = a_src[i] + kt * kTileCols;
      if (WB == 1) {  // binary padding weights are +1: columns past k must read as zero codes
        const int col = kt * kTileCols + (((lane & 15) ^ ((4 * (wave * kDma + i) + (lane >> 4)) & 15)) << 4);
        if (col >= k32) off = kOffPastDescriptor;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, BITLINEAR_LDS(stage + (wave * kDma + i) * 1024), 16, off, 0, 0,
                                               0);
    }
  };

  // weight loads: 32-row block nb of the wave, lane row l32, half h
  int b_src[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int blk = wn * NBH + (SWIGLU ? nb % NBH : nb);  // 32-row block inside the workgroup (per matrix)
    const int rbl = 2 * blk + (l32 >> 4);                 // row block inside the descriptor
    b_src[nb] = rbl * row_tiles * kTileBytes + (l32 & 15) * 16 + (WB == 1 ? 256 * h : 512 * h);
  }
  const int b_step = WB == 1 ? kBinStepBytes : kTileBytes;  // bytes of a row block per k-step
  auto issue_b = [&](uint4 (&br)[NB][BREGS], int kt) {
    const int soff = __builtin_amdgcn_readfirstlane(kt * b_step);  // uniform: the k-step's offset in a row block
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const __amdgpu_buffer_rsrc_t r = (SWIGLU && nb >= NBH) ? u_rsrc : b_rsrc;
#pragma unroll
      for (int j = 0; j < BREGS; ++j) br[nb][j] = load_b128(r, b_src[nb] + 256 * j, soff);
    }
  };

  // LDS offsets of the lane's activation chunk for the group's MFMA steps q0 + qq (token block 0, stage 0)
  int a_off[QN];
#pragma unroll
  for (int qq = 0; qq < QN; ++qq)
    a_off[qq] = (wm * MB * 32 + l32) * kTileCols + (((8 * h + q0 + qq) ^ (l32 & 15)) << 4);

  v16i acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v16i{};

  // The activation operands of step q + 1 are read while step q multiplies.
  // With weights in registers (two stages) scheduling barriers keep that
  // order, so at most two steps' operands are live next to the accumulators
  // and the weight slots; the ring configuration leaves the order to the
  // compiler (measured 1-3% faster there, 4% slower on the wide tile).
  // (every array index below is a compile-time step qq of the group; the
  // weight operand of step qq comes from wop(nb, qq))
  auto read_a = [&](const uint8_t* st, int qq, v4i (&a)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const v4i*>(st + a_off[qq] + mb * 32 * kTileCols);
  };
  auto mul = [&](const v4i (&a)[MB], auto&& wop, int qq) {
    v4i b[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = wop(nb, qq);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
  };
  auto compute = [&](const uint8_t* st, auto&& wop) {
    v4i a0[MB], a1[MB];
    read_a(st, 0, a0);
#pragma unroll
    for (int qq = 0; qq < QN; qq += 2) {
      read_a(st, qq + 1, a1);
      if (!kRing) __builtin_amdgcn_sched_barrier(0);
      mul(a0, wop, qq);
      if (!kRing) __builtin_amdgcn_sched_barrier(0);
      if (qq + 2 < QN) read_a(st, qq + 2, a0);
      if (!kRing) __builtin_amdgcn_sched_barrier(0);
      mul(a1, wop, qq + 1);
      if (!kRing) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // S - 1 steps in flight: the copies of step kt + S - 1 go out while step kt
  // is multiplied.  At the top of a step each wave waits for its own copies
  // of that step (the younger ones stay in flight), then the barrier covers
  // everyone's and makes sure no wave still reads the stage about to be
  // refilled.  The body is unrolled S times so the stages are compile-time
  // offsets.
  if constexpr (kRing) {
    // untracked copies: descriptors as plain registers
    const v4u_d a_desc = raw_descriptor(xq + m0 * k, rows_here * k);
    const v4u_d b_desc = raw_descriptor(packed_b + rb0 * row_bytes, rbs_here * row_bytes);
    const v4u_d u_desc = SWIGLU ? raw_descriptor(packed_u + rb0 * row_bytes, rbs_here * row_bytes) : b_desc;
    const uint32_t ring0 = lds_address(ring);
    // weight copy i of this wave: LDS row block d = wave * kBDma + i of the stage's weight region
    // (ternary: one 1 KiB tile; binary: the 512-byte step halves of row blocks 2d and 2d + 1)
    auto issue = [&](int u, int kt) {
      const uint32_t base = ring0 + u * kStageBytes;
#pragma unroll
      for (int i = 0; i < kDma; ++i) {
        int off = a_src[i] + kt * kTileCols;
        if (WB == 1) {
          const int col = kt * kTileCols + (((lane & 15) ^ ((4 * (wave * kDma + i) + (lane >> 4)) & 15)) << 4);
          if (col >= k32) off = kOffPastDescriptor;
        }
        lds_copy16(a_desc, off, base + (wave * kDma + i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < kBDma; ++i) {
        const int d = wave * kBDma + i;
        if (WB == 1) {
          const int rb = 2 * d + (lane >> 5);
          lds_copy16(b_desc, rb * row_tiles * kTileBytes + kt * kBinStepBytes + (lane & 31) * 16,
                     base + kStage + d * 1024);
        } else if (SWIGLU) {
          const bool up = d >= FB / kTileRows;  // uniform
          const int rb = up ? d - FB / kTileRows : d;
          lds_copy16(up ? u_desc : b_desc, (rb * row_tiles + kt) * kTileBytes + lane * 16, base + kStage + d * 1024);
        } else {
          lds_copy16(b_desc, (d * row_tiles + kt) * kTileBytes + lane * 16, base + kStage + d * 1024);
        }
      }
    };
    // LDS offset (inside a stage's weight region) of the lane's slot j for 32-row block nb
    int b_lds[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lblk = SWIGLU ? (nb < NBH ? wn * NBH + nb : FB / 32 + wn * NBH + nb - NBH) : wn * NB + nb;
      b_lds[nb] = kStage + (2 * lblk + (l32 >> 4)) * TBS + ((l32 & 15) + (WB == 1 ? 16 : 32) * h) * 16;
    }
    auto compute_ring = [&](int u) {
      const uint8_t* st = ring + u * kStageBytes;
      if constexpr (KG == 1) {
        uint4 bc[NB][BREGS];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int j = 0; j < BREGS; ++j) bc[nb][j] = *reinterpret_cast<const uint4*>(st + b_lds[nb] + 256 * j);
        compute(st, [&](int nb, int qq) { return weight_operand<WB>(bc[nb], qq); });
      } else {
        // ternary: the four words of steps q0 .. q0 + 3 are the lane's slot q0 / 4
        uint32_t bw[NB][QN];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint4 v = *reinterpret_cast<const uint4*>(st + b_lds[nb] + 256 * (q0 >> 2));
          bw[nb][0] = v.x;
          bw[nb][1] = v.y;
          bw[nb][2] = v.z;
          bw[nb][3] = v.w;
        }
        compute(st, [&](int nb, int qq) { return expand_ternary(bw[nb][qq]); });
      }
    };
    constexpr int kPer = kDma + kBDma;  // copies per step and wave
    static_assert((S - 2) * kPer < 64, "vmcnt range");
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
      if (kt_begin + u < kt_end) issue(u, kt_begin + u);  // uniform
    for (int kt0 = kt_begin; kt0 < kt_end; kt0 += S) {
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int kt = kt0 + u;
        if (kt < kt_end) {  // uniform
          // steps issued after this one: min(S - 2, kt_end - 1 - kt)
          const int younger = kt_end - 1 - kt;
          if (S > 5 && younger >= 4)
            copies_landed<(S > 5 ? 4 : 0) * kPer>();
          else if (S > 4 && younger >= 3)
            copies_landed<(S > 4 ? 3 : 0) * kPer>();
          else if (S > 3 && younger >= 2)
            copies_landed<(S > 3 ? 2 : 0) * kPer>();
          else if (younger >= 1)
            copies_landed<kPer>();
          else
            copies_landed<0>();
          if (kt + S - 1 < kt_end) issue((u + S - 1) % S, kt + S - 1);
          compute_ring(u);
        }
      }
    }
  } else {
    // two stages, weights in registers; steps go in pairs with the same code
    // on every trip, an odd last step after the loop
    uint4 b0[NB][BREGS], b1[NB][BREGS];
    issue_a(st0, kt_begin);
    issue_b(b0, kt_begin);
    int kt = kt_begin;
    for (; kt + 1 < kt_end; kt += 2) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      issue_a(st1, kt + 1);
      issue_b(b1, kt + 1);
      compute(st0, [&](int nb, int qq) { return weight_operand<WB>(b0[nb], qq); });
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (kt + 2 < kt_end) {  // uniform
        issue_a(st0, kt + 2);
        issue_b(b0, kt + 2);
      }
      compute(st1, [&](int nb, int qq) { return weight_operand<WB>(b1[nb], qq); });
    }
    if (kt < kt_end) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      compute(st0, [&](int nb, int qq) { return weight_operand<WB>(b0[nb], qq); });
    }
  }

  if constexpr (KG > 1) {
    // the two k-groups' partial sums meet in LDS, each group finishing one
    // half of the token blocks (group 0 the first MB / 2, group 1 the rest):
    // each hands the other its half, so the stores are split between them.
    // Every wave is past its last stage read (the barrier), and the last
    // step waited for every copy.
    static_assert(KG == 2 && MB % 2 == 0, "two k-groups, even token blocks");
    __syncthreads();
    int32_t* red = reinterpret_cast<int32_t*>(ring);
    constexpr int kHalf = MB / 2 * NB * 16 * 64;  // int32 per wave and half
#pragma unroll
    for (int mh = 0; mh < MB / 2; ++mh)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[(kg * WM * WN + wl) * kHalf + ((mh * NB + nb) * 16 + r) * 64 + lane] =
              kg == 0 ? acc[MB / 2 + mh][nb][r] : acc[mh][nb][r];
    __syncthreads();
#pragma unroll
    for (int mh = 0; mh < MB / 2; ++mh)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = red[((1 - kg) * WM * WN + wl) * kHalf + ((mh * NB + nb) * 16 + r) * 64 + lane];
          if (kg == 0)
            acc[mh][nb][r] += v;
          else
            acc[MB / 2 + mh][nb][r] += v;
        }
  }
  // token blocks this wave stores: all, or its group's half
  auto mine = [&](int mb) { return KG == 1 || (mb < MB / 2) == (kg == 0); };

  // 32 x 32 block layout: element r of lane l is token 8 * (r / 4) + 4 * (l / 32) + r % 4, row l % 32
  const int tw = wm * MB * 32;  // the wave's first token inside the tile
  if (SPLIT) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (!mine(mb)) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = m0 + tw + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (t >= m) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int64_t j = f0 + (wn * NB + nb) * 32 + l32;
          if (j < n) atomicAdd(&split_acc[t * n + j], acc[mb][nb][r] >> kWeightShift);
        }
      }
    }
    return;
  }

  if (SWIGLU) {
    // blocks nb (gate) and nb + NBH (up) hold the same 32 features: h = silu(g) * u in registers
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tl = tw + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t t = m0 + tl;
        if (t >= m) continue;
        const float sg = scale_s[tl], su = scale_u[tl];
#pragma unroll
        for (int nb = 0; nb < NBH; ++nb) {
          const int64_t j = f0 + (wn * NBH + nb) * 32 + l32;
          if (j < n) {
            const int vg = acc[mb][nb][r] >> kWeightShift;
            const int vu = acc[mb][nb + NBH][r] >> kWeightShift;
            const float g = static_cast<float>(vg) * sg;
            const float u = static_cast<float>(vu) * su;
            __builtin_nontemporal_store(g * u / (1.0f + expf(-g)), y + t * n + j);
            if (acc_out) {
              acc_out[t * 2 * n + j] = vg;
              acc_out[t * 2 * n + n + j] = vu;
            }
          }
        }
      }
    }
    return;
  }

  // plain epilogue: y = (acc >> 6) * (gamma * a'[t] / 127), or with the
  // row's own scale; rows and tokens of a full tile need no bounds checks
  const bool full = m0 + BM <= m && f0 + FB <= n;
  float* yl = y + (m0 + tw + 4 * h) * n + f0 + wn * NB * 32 + l32;
  int32_t* al = acc_out ? acc_out + (m0 + tw + 4 * h) * n + f0 + wn * NB * 32 + l32 : nullptr;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (!mine(mb)) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = mb * 32 + 8 * (r >> 2) + (r & 3);  // token of the lane's element, less 4h
      const int tl = tw + tr + 4 * h;
      if (!full && m0 + tl >= m) continue;
      const float sc = scale_s[tl];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (!full && f0 + (wn * NB + nb) * 32 + l32 >= n) continue;
        const int v = acc[mb][nb][r] >> kWeightShift;
        const int64_t o = static_cast<int64_t>(tr) * n + nb * 32;
        // written once, read by the next kernel: streamed past the caches
        __builtin_nontemporal_store(static_cast<float>(v) * out_scale(dq, sc, f0 + (wn * NB + nb) * 32 + l32), yl + o);
        if (al) al[o] = v;
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int WB>
hipError_t launch(const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k, const int8_t* xq,
                  const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s, bool vec) {
  const int kt = static_cast<int>(k_tiles(k));
  const int64_t mt = (m + BM - 1) / BM;
  const int64_t ntl = (n + BN - 1) / BN;
  if (mt * ntl > 0x7fffffff) return hipErrorInvalidConfiguration;  // beyond one grid dimension
  const dim3 grid(static_cast<unsigned>(mt * ntl));
  constexpr int lds = TileShape<BM, BN, WB>::kLds;
  const uint4* p = static_cast<const uint4*>(packed);
  if (vec) {
    static const bool attr = lds <= 65536 || hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel<BM, BN, WM, WN, true, WB>),
                                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
    (void)attr;
    gemm_kernel<BM, BN, WM, WN, true, WB><<<grid, kThreads, lds, s>>>(p, gamma, dq, n, k, kt, xq, amax, m,
                                                                      static_cast<int>(mt), static_cast<int>(ntl), y, acc);
  } else {
    static const bool attr = lds <= 65536 || hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel<BM, BN, WM, WN, false, WB>),
                                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
    (void)attr;
    gemm_kernel<BM, BN, WM, WN, false, WB><<<grid, kThreads, lds, s>>>(p, gamma, dq, n, k, kt, xq, amax, m,
                                                                       static_cast<int>(mt), static_cast<int>(ntl), y, acc);
  }
  return hipGetLastError();
}


// Candidate tiles (BM, BN, WM, WN).  The choice maximises the fraction of
// the 256 CUs kept busy over the rounds of workgroups (one resident
// workgroup per CU) times the useful fraction of each tile, preferring the
// earlier (larger) tile on ties: more reuse per loaded byte.
// Register-staged fallback (k % 16 != 0 or unaligned codes): two tile sizes.
struct Cand {
  int bm, bn, wm, wn;
};

Cand choose(int64_t m, int64_t /*n*/) {
  if (m <= 64) return Cand{64, 64, 2, 2};
  return Cand{128, 128, 2, 2};
}

// ---- direct-to-LDS pipeline configurations ---------------------------------

// k-slices: zero the int32 target, and afterwards turn the summed
// accumulators into y with the per-token (and per-row) scale of the one-pass
// epilogue, the same functions in the same order, so y is bit-identical.
__global__ void split_zero_kernel(int32_t* __restrict__ p, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) p[i] = 0;
}

__global__ void split_finish_kernel(const int32_t* acc, float* y, const float* __restrict__ gamma_p, Dequant dq,
                                    const float* __restrict__ amax, int64_t m, int64_t n) {
  // acc may alias y (the sums are held in y's own memory): each element is
  // read and then written by the same thread
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < m * n; i += stride) {
    const int64_t t = i / n, j = i - t * n;
    const int v = acc[i];
    y[i] = static_cast<float>(v) * out_scale(dq, token_scale(gamma_p, dq, amax, t), j);
  }
}

// k-steps per slice for a grid of `tiles` output tiles with `occ` resident
// workgroups per CU (0: no split).  Only a grid that fills at most a quarter
// of the resident slots is split, into up to 4 slices of at least
// kMinSliceSteps k-steps.  The sums cost one device-scope atomic per output
// and slice plus the zeroing and finishing passes (about 2.5 us per million
// atomics), so filling a half-empty chip does not pay: the 6144-wide QKV
// matrix at m = 512 (256 tiles in 512 slots) went from 22 to 38 us split in
// two.  At m = 64, 8192 x 28672 (128 tiles in 768 slots) took 51.2 us
// unsplit and 38.9 / 37.6 / 33.9 / 37.0 / 38.3 us in 2 / 3 / 4 / 6 / 8
// slices.
constexpr int kCus = 256;
constexpr int kMinSliceSteps = 8;
constexpr int kMaxSlices = 4;
int slice_steps(int64_t tiles, int occ, int kt) {
  const int64_t slots = static_cast<int64_t>(kCus) * occ;
  if (4 * tiles > slots) return 0;
  int ks = kMaxSlices;
  if (ks > kt / kMinSliceSteps) ks = kt / kMinSliceSteps;
  if (ks < 2) return 0;
  return (kt + ks - 1) / ks;
}

// Launch of the matrix-core kernel for one configuration; the k extent is
// split when the output tiles fill at most a quarter of the resident slots.
template <int MB, int NB, int WM, int WN, int S, int OCC, int WB = 2, int KG = 1>
hipError_t launch_mfma(const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k, const int8_t* xq,
                       const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  constexpr int BM = WM * MB * 32, BN = WN * NB * 32;
  constexpr int kThreadsWG = 64 * WM * WN * KG;
  static_assert(S * (BM * kTileCols + (S > 2 ? BN * kTileBytes / kTileRows : 0)) + 2 * BM * 4 <= 163840 / OCC &&
                    (KG - 1) * WM * WN * MB * NB * 16 * 64 * 4 + 2 * BM * 4 <= 163840 / OCC,
                "LDS per workgroup");
  // 32-bit buffer offsets: BM rows of at most 2^18 codes, BN / 16 row blocks of at most 1024 tiles
  static_assert(static_cast<int64_t>(BM) << 18 <= 0x7fffffff &&
                    static_cast<int64_t>(BN / kTileRows) * 1024 * kTileBytes <= 0x7fffffff,
                "buffer offsets fit 31 bits");
  const int kt = static_cast<int>(k_tiles(k));
  const int64_t mt = (m + BM - 1) / BM;
  const int64_t ntl = (n + BN - 1) / BN;
  if (mt * ntl > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int kt_per = slice_steps(mt * ntl, OCC, kt);
  const uint8_t* p = static_cast<const uint8_t*>(packed);
  if (kt_per == 0) {
    gemm_mfma_kernel<MB, NB, WM, WN, S, OCC, WB, false, false, KG><<<dim3(static_cast<unsigned>(mt * ntl)),
                                                                    kThreadsWG, 0, s>>>(
        p, gamma, dq, n, k, kt, xq, amax, m, static_cast<int>(mt), static_cast<int>(ntl), y, acc, nullptr, nullptr,
        0, nullptr);
    return hipGetLastError();
  }
  // the int32 sums go to acc when the caller wants them, else into y's memory
  int32_t* sums = acc ? acc : reinterpret_cast<int32_t*>(y);
  const int64_t slices = (kt + kt_per - 1) / kt_per;
  const int64_t count = m * n;
  const unsigned fill_grid = static_cast<unsigned>(count / 256 + 1 < 2048 ? count / 256 + 1 : 2048);
  split_zero_kernel<<<fill_grid, 256, 0, s>>>(sums, count);
  gemm_mfma_kernel<MB, NB, WM, WN, S, OCC, WB, false, true, KG><<<dim3(static_cast<unsigned>(mt * ntl * slices)),
                                                                   kThreadsWG, 0, s>>>(
      p, gamma, dq, n, k, kt, xq, amax, m, static_cast<int>(mt), static_cast<int>(ntl), y, acc, nullptr, nullptr,
      kt_per, sums);
  split_finish_kernel<<<fill_grid, 256, 0, s>>>(sums, y, gamma, dq, amax, m, n);
  return hipGetLastError();
}

template <int MB, int NB, int WM, int WN, int S, int OCC>
hipError_t launch_mfma_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u, const float* gamma_u,
                              int64_t f, int64_t k, const int8_t* xq, const float* amax, int64_t m, float* h,
                              int32_t* acc, hipStream_t s) {
  constexpr int BM = WM * MB * 32, FB = WN * NB * 16;
  const int kt = static_cast<int>(k_tiles(k));
  const int64_t mt = (m + BM - 1) / BM;
  const int64_t ntl = (f + FB - 1) / FB;
  if (mt * ntl > 0x7fffffff) return hipErrorInvalidConfiguration;
  gemm_mfma_kernel<MB, NB, WM, WN, S, OCC, 2, true><<<dim3(static_cast<unsigned>(mt * ntl)), kThreads, 0, s>>>(
      static_cast<const uint8_t*>(packed_g), gamma_g, kTokenDequant, f, k, kt, xq, amax, m, static_cast<int>(mt),
      static_cast<int>(ntl), h, acc, static_cast<const uint8_t*>(packed_u), gamma_u, 0, nullptr);
  return hipGetLastError();
}

// Configurations of the matrix-core kernel.  Measured on MI355X over the 8B-
// and 70B-shaped matrices (us per launch, cold weights):
//   * 128 x 256, two stages, weights in registers (MB 4, NB 2, 1 x 4 waves)
//     for more than 64 tokens on wide matrices: 512 x 28672 x 4096 53-54;
//   * 64 x 128 with two k-groups (MB 2, NB 1, 1 x 4 waves x 2, ring of three)
//     when the 64 x 128 grid has 129..256 tiles, one workgroup per CU:
//     512 x 4096 x 4096 12.5 and 512 x 4096 x 14336 31.1-32.0, against
//     12.8-12.9 and 32.8-33.8 with four waves;
//   * 64 x 128 with a ring of three stages (MB 2, NB 1, 1 x 4) otherwise:
//     512 x 6144 x 4096 17.4-18.2, 64 x 57344 x 8192 37.6-38.5,
//     64 x 8192 x 28672 27.8-28.5 (k-sliced).
//   Not faster at those shapes: rings of four to six stages, 2 x 2 waves of
//   32 x 64, waves of 64 x 64 with two or four k-groups, reading operands two
//   to eight steps ahead.  With four waves per CU each SIMD runs one wave,
//   whose matrix-core stream stalls at every copy issue, LDS read and weight
//   expansion (the same instruction mix in isolation: 39% of peak with four
//   waves, 50% with eight); about 5 us of each launch is fixed (the first
//   copies from HBM, the fp32 outputs written after the last step).
enum MfmaConfig {
  kT128x256 = 0,   // MB 4, NB 2, 1 x 4 waves, 2 stages (weights in registers)
  kT64x128 = 1,    // MB 2, NB 1, 1 x 4 waves, ring of 3 stages
  kT64x128k2 = 2,  // MB 2, NB 1, 1 x 4 waves x 2 k-groups, ring of 3 stages
};

#ifndef BITLINEAR_GEMM_FORCE
#define BITLINEAR_GEMM_FORCE -1
#endif

MfmaConfig choose_mfma(int64_t m, int64_t n) {
  if (BITLINEAR_GEMM_FORCE >= 0) return static_cast<MfmaConfig>(BITLINEAR_GEMM_FORCE);
  if (m > 64 && n >= 16384) return kT128x256;
  // (more than 128 tiles: no k-slices at either occupancy)
  const int64_t tiles = ((m + 63) / 64) * ((n + 127) / 128);
  if (tiles > 128 && tiles <= kCus) return kT64x128k2;
  return kT64x128;
}

template <int WB>
hipError_t launch_mfma_any(MfmaConfig c, const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k,
                           const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  if (c == kT128x256) return launch_mfma<4, 2, 1, 4, 2, 2, WB>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
  if constexpr (WB == 2) {  // (k-groups: ternary weights)
    if (c == kT64x128k2) return launch_mfma<2, 1, 1, 4, 3, 1, WB, 2>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
  }
  return launch_mfma<2, 1, 1, 4, 3, 2, WB>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
}

}  // namespace

bool gemm_swiglu_supported(int64_t k, const int8_t* xq) {
  return (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
}

hipError_t launch_gemm_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u, const float* gamma_u,
                              int64_t f, int64_t k, const int8_t* xq, const float* amax, int64_t m, float* h,
                              int32_t* acc, hipStream_t s) {
  if (!gemm_swiglu_supported(k, xq)) return hipErrorInvalidValue;
  if (m > 64)
    return launch_mfma_swiglu<4, 2, 1, 4, 2, 2>(packed_g, gamma_g, packed_u, gamma_u, f, k, xq, amax, m, h, acc, s);
  return launch_mfma_swiglu<2, 2, 1, 4, 2, 2>(packed_g, gamma_g, packed_u, gamma_u, f, k, xq, amax, m, h, acc, s);
}

hipError_t launch_gemm_ex(const void* packed, bool binary, const float* gamma, Dequant dq, int64_t n, int64_t k,
                          const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  const bool vec = (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
  if (vec) {
    const MfmaConfig c = choose_mfma(m, n);
    return binary ? launch_mfma_any<1>(c, packed, gamma, dq, n, k, xq, amax, m, y, acc, s)
                  : launch_mfma_any<2>(c, packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
  }
  const Cand c = choose(m, n);
#define BITLINEAR_GEMM_CASE(BM_, BN_, WM_, WN_)                                                            \
  if (c.bm == BM_ && c.bn == BN_ && c.wm == WM_ && c.wn == WN_)                                            \
    return binary ? launch<BM_, BN_, WM_, WN_, 1>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s, vec)    \
                  : launch<BM_, BN_, WM_, WN_, 2>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s, vec);
  BITLINEAR_GEMM_CASE(128, 128, 2, 2)
  BITLINEAR_GEMM_CASE(64, 64, 2, 2)
#undef BITLINEAR_GEMM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const void* packed, const float* gamma, int64_t n, int64_t k, const int8_t* xq,
                       const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  return launch_gemm_ex(packed, false, gamma, kTokenDequant, n, k, xq, amax, m, y, acc, s);
}

}  // namespace bitlinear
