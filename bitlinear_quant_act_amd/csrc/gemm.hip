// Batched (prefill) BitLinear forward for any token count.
//
// "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
// "The Mathematical Mechanism", items 3-4 (ternary x int8 contraction in
// int32, de-quantisation by gamma * a' / 127).  With many tokens per weight
// the contraction is dense and compute-bound ("BitNet 1-bit LLM Inference
// Framework", section "Scalability with Thread Count": prompt processing is
// compute-intensive), so it runs on the int8 matrix cores.
//
// Tiling: a workgroup of 4 waves (WM x WN) owns a BM x BN output tile
// (tokens x weight rows) and walks k in 256-column steps, the width of one
// packed weight tile.  A step's operands are the BM x 256 int8 activation
// tile and the BN/16 packed weight tiles (1 KiB each, copied verbatim: still
// 2 bits per weight).
//
// Matrix-core instruction: v_mfma_i32_32x32x32_i8 (measured ~4.5 POPS on
// MI355X, against ~2.5-3.2 for the 16x16x64 form).  With the packed layout
// unchanged, step q (0..7) of a 256-column tile takes columns 32q .. 32q+31:
// lane (row r, half h) supplies word 2(q%2)+h of slot (r%16)+16(q/2), i.e.
// 16 columns, expanded to int8 64*w with one shift and one mask per 4
// weights (expand_ternary) and reused for every 32-token block of the wave;
// its A operand is the same 16 columns of its token.  The accumulators hold
// 64 * acc exactly; the epilogue shifts, scales by gamma * a'[t] / 127 and
// stores fp32.
//
// Main path (k % 16 == 0, 16-byte aligned codes): an S-stage ring of LDS
// buffers filled by buffer-to-LDS copies (buffer_load_dwordx4 ... lds), S - 1
// steps in flight, one barrier per step; see gemm_dma_kernel.  Otherwise a
// register-staged two-stage variant (gemm_kernel) handles any k.
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
// S-stage pipeline with buffer-to-LDS loads (k % 16 == 0, codes 16-byte aligned)
// ---------------------------------------------------------------------------
//
// buffer_load_dwordx4 ... lds moves 16 bytes per lane straight into LDS (64
// lanes -> 1 KiB contiguous), so no registers stage the tiles and S - 1 tiles
// can be in flight while one is consumed.  Each stage is its own LDS array so
// the compiler tracks the outstanding copies per stage; a wave waits for its
// own copies of the tile it is about to read (s_waitcnt vmcnt), then a plain
// s_barrier (no memory fence, which would drain every copy) publishes them.
// The buffer (MUBUF) form rather than the global (FLAT) one keeps the
// compiler's LDS-read waits exact: a pending FLAT operation forces every
// lgkmcnt wait to zero.
//
// Each workgroup addresses its operands through two buffer descriptors: its
// BM token rows of codes and its BN / 16 weight row blocks.  Reads past a
// descriptor's byte count return zeros, which covers token rows past m and
// row blocks past n; columns past k (inside the last token row) meet zero
// weight padding.
//
// The activation tile has no padding; instead the 16 chunks of 16 bytes in
// a 256-byte row are stored XOR-swizzled by (row % 16), which keeps the 32
// token rows of one MFMA operand read on distinct banks.

#define BITLINEAR_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int BM, int BN, int WB = 2>
struct DmaShape {
  static constexpr int kABytes = BM * kTileCols;
  static constexpr int kBBytes = (BN / kTileRows) * wtile_bytes<WB>();
  static constexpr int kStage = kABytes + kBBytes;
  static constexpr int kADma = BM / 16;   // 1 KiB copies per wave for the activation tile
  static constexpr int kBDma = BN / 64;   // 1 KiB copies per wave for the (ternary) weight tiles
  static constexpr int kDma = kADma + kBDma;
};

constexpr int DmaStageBytes(int bm, int bn, int wb = 2) {
  return bm * kTileCols + (bn / kTileRows) * (wb == 1 ? kBinTileBytes : kTileBytes);
}

constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format
constexpr int kPastDescriptor = 0x7fffff00;  // byte offset beyond any descriptor's range (reads return 0)

// With SWIGLU the BN weight rows of a stage come from two matrices, gate and
// up, in alternating 32-row blocks over BN / 2 features: 32-row block v holds
// rows 32 * (v / 2) + [0, 32) of the workgroup's features, from gate for even
// v and from up for odd v (b_rsrc / u_rsrc).
//
// Binary weights (WB = 1): one 1 KiB copy carries the k-step's 512-byte half
// tiles of two row blocks (lanes 0-31 the first, 32-63 the second); the
// BN / 32 copies of a stage are dealt to the waves round-robin, so waves may
// issue different counts (the binary kernel runs two stages and waits for
// all copies).
template <int BM, int BN, bool SWIGLU = false, int WB = 2>
__device__ __forceinline__ void issue_tile(uint8_t* stage, __amdgpu_buffer_rsrc_t a_rsrc, __amdgpu_buffer_rsrc_t b_rsrc,
                                           __amdgpu_buffer_rsrc_t u_rsrc, int k, int kt_count, int kt, int wave,
                                           int lane) {
  using DS = DmaShape<BM, BN, WB>;
  const int ktc = kt < kt_count ? kt : 0;  // tiles past the end re-read tile 0 into an unused stage
#pragma unroll
  for (int i = 0; i < DS::kADma; ++i) {
    const int blk = wave * DS::kADma + i;  // 1 KiB = 4 rows
    const int row = 4 * blk + (lane >> 4);
    const int chunk = (lane & 15) ^ (row & 15);
    int off = row * k + ktc * kTileCols + chunk * 16;
    // binary padding weights are +1, not 0: columns past k must read as zero
    // codes, so their chunk is sent past the descriptor (which returns zeros)
    // instead of into the next token's row
    if (WB == 1 && ktc * kTileCols + chunk * 16 >= k) off = kPastDescriptor;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, BITLINEAR_LDS(stage + blk * 1024), 16, off, 0, 0, 0);
  }
  if (WB == 1) {
    const int bt = (kt_count + 1) / 2;
    for (int i = wave; i < BN / 32; i += kThreads / 64) {
      const int rbl = 2 * i + (lane >> 5);
      const int off = (rbl * bt + (ktc >> 1)) * kBinTileBytes + (ktc & 1) * kBinStepBytes + (lane & 31) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, BITLINEAR_LDS(stage + DS::kABytes + i * 1024), 16, off, 0, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < DS::kBDma; ++i) {
    const int rbl = wave * DS::kBDma + i;
    if (SWIGLU) {
      const int src = ((rbl >> 2) << 1) | (rbl & 1);  // row block of the features
      const int off = (src * kt_count + ktc) * kTileBytes + lane * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds((rbl & 2) ? u_rsrc : b_rsrc,
                                               BITLINEAR_LDS(stage + DS::kABytes + rbl * 1024), 16, off, 0, 0, 0);
    } else {
      const int off = (rbl * kt_count + ktc) * kTileBytes + lane * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, BITLINEAR_LDS(stage + DS::kABytes + rbl * 1024), 16, off, 0, 0, 0);
    }
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4] and lgkmcnt [11:8] at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// SWIGLU: packed_b / gamma_p are the gate projection, packed_u / gamma_u the
// up projection (same [n][k] shape, n = features); the workgroup covers
// BN / 2 features and writes h = silu(y_gate) * y_up to y [m][n] (acc_out, if
// set, is [m][2n]: gate accumulators, then up accumulators).
//
// SPLIT: the grid holds ceil(kt_count / kt_per) k-slices of every output tile
// (slice-major); a workgroup walks k-steps [slice * kt_per, ...) and adds its
// partial sums, exact in int32, to split_acc with atomics (zeroed before,
// converted by split_finish_kernel after).
template <int BM, int BN, int WM, int WN, int S, int OCC, bool SWIGLU = false, int WB = 2, bool SPLIT = false>
__global__ __launch_bounds__(kThreads, OCC) void gemm_dma_kernel(const uint8_t* __restrict__ packed_b,
                                                               const float* __restrict__ gamma_p, Dequant dq, int64_t n,
                                                               int64_t k, int kt_count, const int8_t* __restrict__ xq,
                                                               const float* __restrict__ amax, int64_t m,
                                                               int mt_count, int nt_count, float* __restrict__ y,
                                                               int32_t* __restrict__ acc_out,
                                                               const uint8_t* __restrict__ packed_u,
                                                               const float* __restrict__ gamma_u, int kt_per = 0,
                                                               int32_t* __restrict__ split_acc = nullptr) {
  static_assert(WM * WN == kThreads / 64, "4 waves");
  static_assert(S >= 2 && S <= 4, "2..4 stages");
  static_assert(WB == 2 || (S == 2 && !SWIGLU), "binary weights: two stages, plain epilogue");
  static_assert(!(SPLIT && SWIGLU), "k-slices: plain epilogue only");
  using DS = DmaShape<BM, BN, WB>;
  constexpr int TB = wtile_bytes<WB>();
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;
  static_assert(MB >= 1 && NB >= 1 && TM % 32 == 0 && TN % 32 == 0 && BN % 64 == 0, "tile shape");
  static_assert(!SWIGLU || NB % 2 == 0, "gate and up blocks pair up inside a wave");
  constexpr int FB = SWIGLU ? BN / 2 : BN;  // output columns (features) per workgroup

  __shared__ __attribute__((aligned(1024))) uint8_t st0[DS::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[DS::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[S > 2 ? DS::kStage : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[S > 3 ? DS::kStage : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps stage addresses scalar
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int total = mt_count * nt_count;
  int id = blockIdx.x;
  int kt_begin = 0, kt_end = kt_count;
  if (SPLIT) {
    const int slice = id / total;
    id -= slice * total;
    kt_begin = slice * kt_per;
    kt_end = kt_begin + kt_per < kt_count ? kt_begin + kt_per : kt_count;
  }
  // (with SPLIT and total % 8 == 0 the hardware XCD of a workgroup is still id % 8)
  if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
  const int nt = id / mt_count, mt = id - nt * mt_count;
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int64_t n0 = static_cast<int64_t>(nt) * FB;
  const int64_t rb0 = n0 / kTileRows;
  const int64_t rb_count = row_blocks(n);

  v16i acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v16i{};

  // per-lane LDS offsets
  const int a_row0 = wm * TM + l32;                                   // + mb * 32; row % 16 == l32 % 16
  const int a_x = (l32 & 15) ^ h;                                     // swizzle key with the lane's half folded in
  const int b_row = wn * TN + l32;                                    // + nb * 32
  const int b_off = DS::kABytes + slot_offset<WB>(b_row);              // + nb * 2 tiles + g * 16 slots

  // operands of one 64-column group: NB weight slots and 2 x MB activation chunks
  struct Ops {
    uint4 slot[NB];
    v4i a[2][MB];
  };
  auto read_ops = [&](const uint8_t* st, int g, Ops& o) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o.slot[nb] = read_slot<WB>(st + b_off + nb * 2 * TB + group_offset<WB>(g), h);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int chunk = (4 * g + 2 * half) ^ a_x;  // logical chunk 4g + 2 half + h, swizzled by row % 16
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        o.a[half][mb] = *reinterpret_cast<const v4i*>(st + (a_row0 + mb * 32) * kTileCols + chunk * 16);
    }
  };
  auto math = [&](const Ops& o, int g) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      v4i b[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) b[nb] = slot_operand<WB>(o.slot[nb], g, half, h);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[half][mb], b[nb], acc[mb][nb], 0, 0, 0);
    }
  };
  // software-pipelined over the tile's four 64-column groups: the operands
  // of group g + 1 are read from LDS while group g is on the matrix cores
  // (scheduling barriers keep that order)
  auto compute = [&](const uint8_t* st) {
    Ops o0, o1;
    read_ops(st, 0, o0);
    __builtin_amdgcn_sched_barrier(0);
    read_ops(st, 1, o1);
    __builtin_amdgcn_sched_barrier(0);
    math(o0, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_ops(st, 2, o0);
    __builtin_amdgcn_sched_barrier(0);
    math(o1, 1);
    __builtin_amdgcn_sched_barrier(0);
    read_ops(st, 3, o1);
    __builtin_amdgcn_sched_barrier(0);
    math(o0, 2);
    __builtin_amdgcn_sched_barrier(0);
    math(o1, 3);
  };

  // per-token output scale gamma * a'[t] / 127, staged once (one per matrix)
  __shared__ float scale_s[BM];
  __shared__ float scale_u[SWIGLU ? BM : 1];
  if (tid < BM) {
    const int64_t t = m0 + tid;
    scale_s[tid] = t < m ? token_scale(gamma_p, dq, amax, t) : 0.0f;
    if (SWIGLU) scale_u[tid] = t < m ? *gamma_u * amax[t] / 127.0f : 0.0f;
  }
  lds_barrier();

  // operand descriptors: this workgroup's token rows and weight row blocks
  const int64_t rows_here = m - m0 < BM ? m - m0 : BM;
  const int64_t rbs_here = rb_count - rb0 < FB / kTileRows ? rb_count - rb0 : FB / kTileRows;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(xq + m0 * k), 0, static_cast<int>(rows_here * k), kBufferWord3);
  const int64_t row_bytes = WB == 1 ? static_cast<int64_t>((kt_count + 1) / 2) * kBinTileBytes
                                    : static_cast<int64_t>(kt_count) * kTileBytes;  // one row block's weights
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed_b + rb0 * row_bytes), 0, static_cast<int>(rbs_here * row_bytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t u_rsrc = SWIGLU ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed_u + rb0 * kt_count * kTileBytes), 0,
      static_cast<int>(rbs_here * kt_count * kTileBytes), kBufferWord3) : b_rsrc;
  const int k32 = static_cast<int>(k);

  // prologue: tiles 0 .. S-2 in flight (k-slice: relative to kt_begin; a tile
  // past the slice re-reads its first tile into a stage nothing reads)
  auto tile_at = [&](int kt) { return SPLIT ? (kt < kt_end ? kt : kt_begin) : kt; };
  issue_tile<BM, BN, SWIGLU, WB>(st0, a_rsrc, b_rsrc, u_rsrc, k32, kt_count, tile_at(kt_begin), wave, lane);
  if (S > 2) issue_tile<BM, BN, SWIGLU, WB>(st1, a_rsrc, b_rsrc, u_rsrc, k32, kt_count, tile_at(kt_begin + 1), wave, lane);
  if (S > 3) issue_tile<BM, BN, SWIGLU, WB>(st2, a_rsrc, b_rsrc, u_rsrc, k32, kt_count, tile_at(kt_begin + 2), wave, lane);

  // one pipeline step: tile kt sits in stage `cur`; tile kt + S - 1 goes to `nxt`
  auto step = [&](int kt, uint8_t* cur, uint8_t* nxt) {
    wait_vmcnt<(S - 2) * DS::kDma>();
    __builtin_amdgcn_s_barrier();
    issue_tile<BM, BN, SWIGLU, WB>(nxt, a_rsrc, b_rsrc, u_rsrc, k32, kt_count, tile_at(kt + S - 1), wave, lane);
    compute(cur);
  };
  for (int kt = kt_begin; kt < kt_end; kt += S) {
    step(kt, st0, S == 2 ? st1 : S == 3 ? st2 : st3);
    if (kt + 1 < kt_end) step(kt + 1, st1, S == 2 ? st0 : S == 3 ? st0 : st0);
    if (S > 2 && kt + 2 < kt_end) step(kt + 2, st2, S == 3 ? st1 : st1);
    if (S > 3 && kt + 3 < kt_end) step(kt + 3, st3, st2);
  }
  wait_vmcnt<0>();

  if (SPLIT) {
    // partial sums of this k-slice (multiples of 64, shifted exactly)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = m0 + wm * TM + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (t >= m) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int64_t j = n0 + wn * TN + nb * 32 + l32;
          if (j < n) atomicAdd(&split_acc[t * n + j], acc[mb][nb][r] >> kWeightShift);
        }
      }
    }
    return;
  }

  if (SWIGLU) {
    // blocks nb (gate) and nb + 1 (up) hold the same 32 features; the lane's
    // elements line up, so h = silu(g) * u is formed in registers
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tl = wm * TM + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t t = m0 + tl;
        if (t >= m) continue;
        const float sg = scale_s[tl], su = scale_u[tl];
#pragma unroll
        for (int nb = 0; nb < NB; nb += 2) {
          const int64_t j = n0 + 16 * (wn * NB + nb) + l32;
          if (j < n) {
            const int vg = acc[mb][nb][r] >> kWeightShift;
            const int vu = acc[mb][nb + 1][r] >> kWeightShift;
            const float g = static_cast<float>(vg) * sg;
            const float u = static_cast<float>(vu) * su;
            y[t * n + j] = g * u / (1.0f + expf(-g));
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
          const int v = acc[mb][nb][r] >> kWeightShift;
          y[t * n + j] = static_cast<float>(v) * out_scale(dq, scale_s[tl], j);
          if (acc_out) acc_out[t * n + j] = v;
        }
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

template <int BM, int BN, int WM, int WN, int S, int OCC, int WB = 2>
hipError_t launch_dma(const void* packed, const float* gamma, Dequant dq, int64_t n, int64_t k, const int8_t* xq,
                      const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  static_assert(S * DmaStageBytes(BM, BN, WB) <= 163840, "LDS per workgroup");  // OCC: register-budget hint
  // 32-bit buffer offsets: BM rows of at most 2^18 codes, BN / 16 row blocks of at most 1024 tiles
  static_assert(static_cast<int64_t>(BM) << 18 <= 0x7fffffff && static_cast<int64_t>(BN / kTileRows) * 1024 * kTileBytes <= 0x7fffffff,
                "buffer offsets fit 31 bits");
  const int kt = static_cast<int>(k_tiles(k));
  const int64_t mt = (m + BM - 1) / BM;
  const int64_t ntl = (n + BN - 1) / BN;
  if (mt * ntl > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int kt_per = slice_steps(mt * ntl, OCC, kt);
  if (kt_per == 0) {
    gemm_dma_kernel<BM, BN, WM, WN, S, OCC, false, WB><<<dim3(static_cast<unsigned>(mt * ntl)), kThreads, 0, s>>>(
        static_cast<const uint8_t*>(packed), gamma, dq, n, k, kt, xq, amax, m, static_cast<int>(mt),
        static_cast<int>(ntl), y, acc, nullptr, nullptr);
    return hipGetLastError();
  }
  // the int32 sums go to acc when the caller wants them, else into y's memory
  int32_t* sums = acc ? acc : reinterpret_cast<int32_t*>(y);
  const int64_t slices = (kt + kt_per - 1) / kt_per;
  const int64_t count = m * n;
  const unsigned fill_grid = static_cast<unsigned>(count / 256 + 1 < 2048 ? count / 256 + 1 : 2048);
  split_zero_kernel<<<fill_grid, 256, 0, s>>>(sums, count);
  gemm_dma_kernel<BM, BN, WM, WN, S, OCC, false, WB, true><<<dim3(static_cast<unsigned>(mt * ntl * slices)), kThreads, 0, s>>>(
      static_cast<const uint8_t*>(packed), gamma, dq, n, k, kt, xq, amax, m, static_cast<int>(mt),
      static_cast<int>(ntl), y, acc, nullptr, nullptr, kt_per, sums);
  split_finish_kernel<<<fill_grid, 256, 0, s>>>(sums, y, gamma, dq, amax, m, n);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int S, int OCC>
hipError_t launch_dma_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u, const float* gamma_u,
                             int64_t f, int64_t k, const int8_t* xq, const float* amax, int64_t m, float* h,
                             int32_t* acc, hipStream_t s) {
  static_assert(S * DmaStageBytes(BM, BN) <= 163840, "LDS per workgroup");
  static_assert(static_cast<int64_t>(BM) << 18 <= 0x7fffffff && static_cast<int64_t>(BN / kTileRows) * 1024 * kTileBytes <= 0x7fffffff,
                "buffer offsets fit 31 bits");
  const int kt = static_cast<int>(k_tiles(k));
  const int64_t mt = (m + BM - 1) / BM;
  const int64_t ntl = (f + BN / 2 - 1) / (BN / 2);
  if (mt * ntl > 0x7fffffff) return hipErrorInvalidConfiguration;
  gemm_dma_kernel<BM, BN, WM, WN, S, OCC, true><<<dim3(static_cast<unsigned>(mt * ntl)), kThreads, 0, s>>>(
      static_cast<const uint8_t*>(packed_g), gamma_g, kTokenDequant, f, k, kt, xq, amax, m, static_cast<int>(mt),
      static_cast<int>(ntl), h, acc, static_cast<const uint8_t*>(packed_u), gamma_u);
  return hipGetLastError();
}

// Tile choice, from measurements on MI355X of every (tile, stages,
// workgroups per CU) candidate on the 8B- and 70B-shaped layers: wide weight
// tiles with two resident workgroups per CU for wide matrices, their four
// waves side by side along n (each wave 64 tokens x 64 rows, so every
// expanded weight operand feeds two matrix-core steps; about 5% faster than
// 2 x 2 waves); 64 x 192 for
// mid widths; small 64 x 64 tiles with three workgroups per CU otherwise
// (enough workgroups to fill 256 CUs, and one workgroup's barrier and copy
// latency hidden behind the others' matrix-core work).
enum DmaConfig { kWide = 0, kMid = 1, kSmall = 2 };

#ifndef BITLINEAR_GEMM_FORCE
#define BITLINEAR_GEMM_FORCE -1
#endif

DmaConfig choose_dma(int64_t m, int64_t n) {
  if (BITLINEAR_GEMM_FORCE >= 0) return static_cast<DmaConfig>(BITLINEAR_GEMM_FORCE);
  if (n >= 16384) return kWide;
  if (m > 64 && n >= 6144) return kMid;
  return kSmall;
}

}  // namespace

bool gemm_swiglu_supported(int64_t k, const int8_t* xq) {
  return (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
}

hipError_t launch_gemm_swiglu(const void* packed_g, const float* gamma_g, const void* packed_u, const float* gamma_u,
                              int64_t f, int64_t k, const int8_t* xq, const float* amax, int64_t m, float* h,
                              int32_t* acc, hipStream_t s) {
  if (!gemm_swiglu_supported(k, xq)) return hipErrorInvalidValue;
  if (f >= 8192)
    return launch_dma_swiglu<64, 256, 2, 2, 2, 2>(packed_g, gamma_g, packed_u, gamma_u, f, k, xq, amax, m, h, acc, s);
  return launch_dma_swiglu<64, 128, 2, 2, 2, 2>(packed_g, gamma_g, packed_u, gamma_u, f, k, xq, amax, m, h, acc, s);
}

hipError_t launch_gemm_ex(const void* packed, bool binary, const float* gamma, Dequant dq, int64_t n, int64_t k,
                          const int8_t* xq, const float* amax, int64_t m, float* y, int32_t* acc, hipStream_t s) {
  const bool vec = (k % 16 == 0) && (reinterpret_cast<uintptr_t>(xq) % 16 == 0);
  if (vec && binary) {  // two stages: the binary tiles' copies are not the same count on every wave
    switch (choose_dma(m, n)) {
      case kWide: return launch_dma<64, 256, 1, 4, 2, 2, 1>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
      case kMid: return launch_dma<64, 192, 2, 2, 2, 2, 1>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
      case kSmall: return launch_dma<64, 64, 2, 2, 2, 3, 1>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
    }
  }
  if (vec) {
    switch (choose_dma(m, n)) {
      case kWide: return launch_dma<64, 256, 1, 4, 2, 2>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
      case kMid: return launch_dma<64, 192, 2, 2, 2, 2>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
      case kSmall: return launch_dma<64, 64, 2, 2, 3, 3>(packed, gamma, dq, n, k, xq, amax, m, y, acc, s);
    }
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
