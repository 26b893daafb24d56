// Kernel templates of the persistent grouped GEMM (internal; included by the
// launch units grouped_gemm*.hip, each of which instantiates one family of
// tiles, so that they compile in parallel).
#pragma once
// Persistent, block-scheduled grouped GEMM for the MoE expert layer (gfx950).
//
// One launch computes, for every group g (an expert, or the shared expert),
//   out[rows of g] = epilogue( act[rows of g] * W[g] ),
// where W[g] is [K][N] with N contiguous and the epilogue is either a plain
// store (bf16, or fp32 for the fused layer's down projection, whose output
// feeds the combine without a bf16 rounding) or, in the gated form, SwiGLU
// over two weight matrices: out = silu(act*W_gate) * (act*W_up). In the gated
// form the gate and up products only ever live in accumulator registers, so
// the SwiGLU input never reaches memory (the dispatch-kernel post
// (lumeric.app), summary paragraph). Grouping many independent GEMMs into one
// persistent launch follows the grouped-GEMM news page (meineki.news); block
// scheduling over variable expert batch sizes follows the Triton MoE page
// (setupai.cc), key points.
//
// Work items and scheduling. An item is one (group, M-tile, N-tile, K-slice):
// BT activation rows by BF output columns over a K range. Items of a segment
// have equal cost, so a static round-robin over a persistent grid stays
// balanced however skewed the expert counts are. Each workgroup rebuilds the
// per-group item prefix from the device-side expert offsets in its prologue:
// there is no host synchronisation. Items are numbered group by group,
// N-tile by N-tile, M-tile next and K-slice fastest; the workgroup -> slot map
// gives every XCD a contiguous run of items (workgroups are dispatched
// round-robin over the 8 XCDs), so the M-tiles sharing a weight tile run
// together under one L2. K-slices (split-K) are used only for plain fp32
// outputs: slice s writes its partial sums to out + s*slice_stride and the
// consumer adds the slices in order, so results stay deterministic.
//
// Operand roles ("swap A/B"). The MFMA A operand is the weight tile and the
// B operand the activations, i.e. the kernel computes (W^T X^T)^T: output
// features fill the 16-wide MFMA M side and tokens the N side. A decode-size
// group with a handful of rows then wastes only the token side of the MFMA,
// and each lane ends up owning 4 consecutive output features of one token.
// The same role swap for small expert batches appears in the DeepGEMM
// article (itsolotime.com), section 3.2, and in the HPC-Ops article
// (ntfzh.com), FusedMoE paragraph.
//
// Data path. Tiles move global -> LDS with gfx950's direct-to-LDS loads
// (global_load_lds_dwordx4: no VGPR staging) into a ring of STAGES buffers,
// so STAGES-1 K-steps are in flight while one is computed. Each ring buffer
// is its own __shared__ array, so the compiler's LDS-DMA alias tracking does
// not make a read of one stage wait for loads into another; the wait for a
// stage is an explicit vmcnt followed by a bare s_barrier (a __syncthreads
// fence would drain every outstanding load). Each wave-wide DMA instruction
// fills 1 KB of LDS in lane order, so tiles are stored in their global
// layouts (activations [BT][BK] K-contiguous) with an XOR swizzle of 16-byte
// chunks chosen on the global side. The weight operand needs K-consecutive
// values per lane. Row-major weights ([BK][BF], N-contiguous) do not give
// them, and the transposing LDS read ds_read_b64_tr_b16 delivers them;
// packed weights (pack_weights_kernel) already hold each column's
// K-values contiguously, so a lane reads its fragment with one 16-byte LDS
// read. MFMA: v_mfma_f32_16x16x32_bf16, fp32 accumulation.
#include <algorithm>
#include <cmath>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {

namespace {

constexpr int kMaxGroups = kMaxExperts + 1;  // routed experts + one shared

// gfx950's v_cvt_scalef32_pk_bf16_fp8 / _fp4 decode two OCP E4M3 codes (the
// low or the high word of a dword) or two E2M1 codes (one byte) straight to
// bf16, times a power-of-two scale. Every such product of a weight is a bf16
// value, so the conversion is exact. (Compiler builtins, so that the compiler
// keeps its hazard waits against MFMAs still reading registers.)
__device__ __forceinline__ bf16x8 cat4(bf16x2_t a, bf16x2_t b, bf16x2_t c, bf16x2_t d) {
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight E4M3 codes (the bytes of u, in order) times a power-of-two scale.
__device__ __forceinline__ bf16x8 fp8x8_scaled_to_bf16(uint2 u, float scale) {
  return cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, scale, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, scale, true),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, scale, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, scale, true));
}

// Eight E4M3 codes (the bytes of u, in order), unscaled.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 u) { return fp8x8_scaled_to_bf16(u, 1.0f); }

// Eight E2M1 codes (the nibbles of u, low nibble first) times a power-of-two
// scale.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t u, float scale) {
  return cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, scale, 0),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, scale, 1),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, scale, 2),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, scale, 3));
}

// MXFP4 scale bytes per 64-column block: K-blocks of 32, rounded up to a
// whole number of 128-value steps, so a stage up to 128 deep stays inside
// its block's scales.
__host__ __device__ __forceinline__ int mx_scale_kblocks(int K) { return 4 * ((K + 127) / 128); }

// Lambdas of the kernel body are always inlined: their operands (the
// accumulators, fragment sets and ring buffers) must stay in registers and
// fixed LDS arrays.
#define INL __attribute__((always_inline))

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BT_, int BF_, int BK_, int WT_, int WF_, int STAGES_, bool GATED_,
          bool PREFETCH_, int MIN_WAVES_ = 1, int WBITS_ = 16, bool PP_ = false,
          bool MX_ = (WBITS_ == 4)>
struct TileCfg {
  static constexpr int BT = BT_;  // activation rows (tokens) per tile
  static constexpr int BF = BF_;  // output columns per tile
  static constexpr int BK = BK_;  // K per pipeline stage
  static constexpr int WT = WT_;  // waves along tokens
  static constexpr int WF = WF_;  // waves along output columns
  static constexpr int STAGES = STAGES_;
  static constexpr bool GATED = GATED_;
  // Read the next stage's MFMA fragments into a second register set while
  // this stage's MFMAs run (costs one more fragment set of registers).
  static constexpr bool PREFETCH = PREFETCH_;
  // waves per SIMD the register allocation must leave room for (so that
  // this many fit by registers as well as by LDS)
  static constexpr int MIN_WAVES = MIN_WAVES_;
  // bits per weight element: 16 (bf16), 8 (fp8 E4M3 codes) or 4 (MXFP4
  // E2M1 codes); the 8- and 4-bit codes exist in their packed layouts only
  static constexpr int WBITS = WBITS_;
  // block scales: one E8M0 scale byte per 32 K-values of a column (MXFP4,
  // and MXFP8 on 8-bit codes), carried in the ring behind each stage's
  // operands; 8-bit codes without them have per-column fp32 scales
  static constexpr bool MX = MX_;
  // Ping-pong schedule: the two waves of each SIMD alternate between an
  // MFMA phase and a memory phase (LDS fragment reads, DMA issue), so one of
  // them always feeds the matrix core (8 waves, no fragment prefetch).
  static constexpr bool PP = PP_;
  // Ping-pong tiles on 8- or 4-bit codes (fp8, mxfp8, mxfp4) widen each
  // stage's weights once into a double-buffered bf16 tile (packed bf16
  // layout), instead of every wave widening the fragments it reads.
  static constexpr bool WIDEN = PP_ && WBITS_ != 16;
  static constexpr int WW_BYTES = WIDEN ? (GATED_ ? 2 : 1) * BK_ * BF_ * 2 : 1;
  static constexpr int NW = WT * WF;
  static constexpr int kThreads = NW * kWave;
  static constexpr int NMAT = GATED ? 2 : 1;
  static constexpr int TF = BF / WF;  // columns per wave
  static constexpr int TT = BT / WT;  // tokens per wave
  static constexpr int FF = TF / 16;  // MFMA blocks per wave (columns)
  static constexpr int FT = TT / 16;  // MFMA blocks per wave (tokens)
  static constexpr int W_BYTES = BK * BF * WBITS / 8;  // one weight matrix per stage
  static constexpr int SB = BF / 64;                   // 64-column sub-blocks per matrix
  static constexpr int SB_BYTES = BK * 64 * WBITS / 8; // one sub-block: BK rows of 64 columns
  static constexpr int X_BYTES = BT * BK * 2;
  static constexpr int OP_BYTES = NMAT * W_BYTES + X_BYTES;  // the MFMA operands
  // MXFP4: the scale bytes of the stage's weights after the operands, as
  // pieces (matrix, sub-block) of BK/32 K-blocks x 64 columns; each wave
  // loads one slot of SC_SLOT bytes (one partial DMA instruction)
  static constexpr int SC_PIECE = MX ? (BK / 32) * 64 : 0;
  static constexpr int SC_BYTES = MX ? NMAT * SB * SC_PIECE : 0;
  static constexpr int SC_SLOT = SC_BYTES / NW;
  static constexpr int STAGE_BYTES = OP_BYTES + SC_BYTES;
  static constexpr int INSTR = OP_BYTES / 1024;     // 1 KB operand DMA instructions
  static constexpr int OPW = INSTR / NW;            // per wave per stage
  static constexpr int IPW = OPW + (MX ? 1 : 0);    // vector-memory operations per wave per stage
  static constexpr int W_INSTR = NMAT * W_BYTES / 1024;
  static_assert(BF % (16 * WF) == 0 && BT % (16 * WT) == 0, "wave tiling");
  static_assert((BK == 32 || BK % 64 == 0) && BF % 64 == 0, "swizzle geometry");
  static_assert(W_BYTES % 1024 == 0 && X_BYTES % 1024 == 0, "1 KB DMA granules");
  static_assert(INSTR % NW == 0 && W_INSTR % NW == 0,
                "equal DMA share per wave, one operand kind per instruction slot");
  static_assert(STAGES >= 3 && STAGES <= 8, "ring depth");
  static_assert(WBITS == 16 || WBITS == 8 || WBITS == 4, "bf16, fp8 or mxfp4 weights");
  static_assert((WBITS == 4) <= MX && !(WBITS == 16 && MX), "4-bit codes carry block scales");
  static_assert(!MX || (SC_SLOT % 16 == 0 && SC_SLOT > 0 && SC_PIECE % SC_SLOT == 0),
                "each wave's scale slot: whole 16-byte chunks inside one piece");
  // vmcnt holds at most 63 outstanding operations per wave: the K-steps in
  // flight must fit, and for chaining across items also the epilogue's
  // stores issued while the next item's first K-steps are in flight
  static constexpr int STORES = (BF / WF / 16) * (BT / WT / 16);
  static_assert((PREFETCH ? STAGES : STAGES - 1) * IPW <= 63, "vector-memory counter range");
  static constexpr bool CHAIN_OK = PREFETCH && STAGES * IPW + STORES <= 63;
  static_assert(!PP || (NW == 8 && !PREFETCH), "ping-pong: two waves per SIMD");
  static_assert(!WIDEN || (BK == 32 && (NMAT * SB * 64 * 2) % kThreads == 0 && STAGES >= 5),
                "widening: whole 16-code units per thread, two steps of look-ahead");
};

// 16-byte chunk swizzles (chunk index within a row), chosen by measuring
// LDS throughput of each access pattern on gfx950.
// Weights are held as 64-column sub-blocks with 128-byte rows: the 4 rows a
// 16-lane transpose read touches land in 4 distinct chunk pairs
// (XOR 2*(row%4)), and the row groups 8 apart that other lanes of the same
// instruction read land on the other bank half (XOR 2*((row/8)%2)). Rows r
// and r+4, read by one lane, share the swizzle (bit 2 of the row is unused;
// so do rows r and r+32, which lets a 32-deep stage read half of a packed
// 64-row block). Activations: 8 consecutive token rows at the same K
// chunk land in 8 distinct 16-byte bank groups: with rows of >= 128 bytes the
// chunk is XORed with row % 8; with 64-byte rows (BK = 32) two rows share a
// 128-byte window, so row % 2 picks the half and (row / 2) % 4 is XORed in.
__device__ __forceinline__ int swz_w(int row, int chunk) {
  return chunk ^ ((row & 3) << 1) ^ (((row >> 3) & 1) << 1);
}
template <int BK>
__device__ __forceinline__ int swz_x(int row, int chunk) {
  return BK == 32 ? chunk ^ ((row >> 1) & 3) : chunk ^ (row & 7);
}

struct GroupView {
  int seg;      // segment index
  int local;    // group index within the segment
  int r0;       // first activation row
  int M;        // number of rows
};

__device__ __forceinline__ GroupView group_view(const GemmProblem& p, int g) {
  GroupView v;
  const int ng0 = p.seg[0].ngroups;
  v.seg = g < ng0 ? 0 : 1;
  v.local = v.seg ? g - ng0 : g;
  const GemmSegment& s = v.seg ? p.seg[1] : p.seg[0];
  if (s.offsets) {
    int a = s.offsets[v.local], b = s.offsets[v.local + 1];
    a = a < 0 ? 0 : (a > s.rows ? s.rows : a);
    b = b < a ? a : (b > s.rows ? s.rows : b);
    v.r0 = a;
    v.M = b - a;
  } else {
    v.r0 = 0;
    v.M = s.rows;
  }
  return v;
}

// Output stores go through the global address space with builtin vector
// types: a flat store (what a generic pointer, or a HIP vector class whose
// assignment takes a generic `this`, compiles to) also counts as an LDS
// access, so every later LDS wait would wait for the store as well.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store4(bf16_t* p, const float v[4]) {
  *(__attribute__((address_space(1))) u32x2_t*)(p) =
      u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *(__attribute__((address_space(1))) f32x4_t*)(p) = f32x4_t{v[0], v[1], v[2], v[3]};
}
// Device-scope stores and loads (relaxed atomics at agent scope): they
// write through to, and read from, the memory all eight XCDs share, instead
// of an XCD's own L2, so partial sums handed to another workgroup need no
// write-back or invalidation of the whole L2 (which agent-scope fences do).
// The logistic sigmoid 1/(1 + e^-z) with the reciprocal taken by v_rcp_f32
// (1 ulp) instead of an IEEE division (about ten VALU instructions, which the
// SwiGLU epilogues pay once per output element): h is rounded to bf16 right
// after, 2^15 times coarser. 1 + e^-z >= 1, so no denormal reaches the
// reciprocal; e^-z = inf gives 0, as the division would.
__device__ __forceinline__ float sigmoid_rcp(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ void store4_device(float* p, const float v[4]) {
  typedef __attribute__((address_space(1))) float gfloat_t;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __hip_atomic_store((gfloat_t*)(p) + i, v[i], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_device(const float* p) {
  typedef __attribute__((address_space(1))) const float gcfloat_t;
  return __hip_atomic_load((gcfloat_t*)(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

template <class C, typename OutT, bool KTAIL, bool PACKED, bool TRANSW = false>
__global__ __launch_bounds__(C::kThreads, C::MIN_WAVES) void grouped_gemm_kernel(
    GemmProblem prob) {
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st3[C::STAGE_BYTES];
  // deeper rings only (unreferenced otherwise, hence not allocated)
  __shared__ __attribute__((aligned(1024))) char st4[C::STAGES > 4 ? C::STAGE_BYTES : 1];
  __shared__ __attribute__((aligned(1024))) char st5[C::STAGES > 5 ? C::STAGE_BYTES : 1];
  __shared__ __attribute__((aligned(1024))) char st6[C::STAGES > 6 ? C::STAGE_BYTES : 1];
  __shared__ __attribute__((aligned(1024))) char st7[C::STAGES > 7 ? C::STAGE_BYTES : 1];
  __shared__ __attribute__((aligned(1024))) char wide0[C::WW_BYTES];  // widened weights
  __shared__ __attribute__((aligned(1024))) char wide1[C::WW_BYTES];
  // sized at launch: item prefix [groups + 1], then (first row, rows) per
  // group, so that looking up an item reads LDS only (a global load inside
  // the K pipeline would wait for every DMA in flight)
  extern __shared__ __attribute__((aligned(16))) int s_pref[];
  __shared__ int s_wave_total[C::NW];
  // decode-size fp32 tiles: the combine folded into the epilogue
  // (ScatterArgs); the token of each row of the item whose column tile this
  // workgroup completes, else -1
  constexpr bool kScatterTile = !C::GATED && sizeof(OutT) == 4 && !TRANSW && C::BT <= 32;
  __shared__ int s_scat[kScatterTile ? C::BT : 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wf = wave % C::WF;
  const int wt = wave / C::WF;
  const int g16 = lane >> 4;   // k-group of the lane in an MFMA operand
  const int i16 = lane & 15;   // row/column of the lane in an MFMA operand

  // ---- prologue: item prefix over all groups of both segments ----
  const int NG = prob.seg[0].ngroups + (prob.nseg > 1 ? prob.seg[1].ngroups : 0);
  int2* const s_rows = reinterpret_cast<int2*>(s_pref + ((NG + 2) & ~1));
  constexpr int GPT = (kMaxGroups + C::kThreads - 1) / C::kThreads;
  int cnt[GPT];
  int my_sum = 0;
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    cnt[i] = 0;
    if (g < NG) {
      const GroupView v = group_view(prob, g);
      const GemmSegment& s = v.seg ? prob.seg[1] : prob.seg[0];
      cnt[i] = ((v.M + C::BT - 1) / C::BT) * ((s.N + C::BF - 1) / C::BF) * s.ksplit;
      s_rows[g] = int2{v.r0, v.M};
    }
    my_sum += cnt[i];
  }
  const int incl = wave_inclusive_scan(my_sum);
  if (lane == kWave - 1) s_wave_total[wave] = incl;
  __syncthreads();
  int run = incl - my_sum;
  for (int w = 0; w < wave; ++w) run += s_wave_total[w];
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    if (g <= NG) s_pref[g] = run;  // s_pref[NG] = total
    run += cnt[i];
  }
  __syncthreads();
  const int total = s_pref[NG];

  // Balanced persistent schedule: with R = ceil(total / grid) rounds, only
  // ceil(total / R) workgroups take items (spread evenly over the 8 XCDs,
  // workgroups being dispatched round-robin over them), so every active
  // workgroup gets R or R-1 items and none works alone through a last,
  // sparse round. Each XCD's active workgroups take a contiguous run of
  // slots, so consecutive items (the M-tiles of one weight tile) share an L2.
  const int G = gridDim.x;
  int slot, stride;
  if (total == 0) return;
  if (G % 8 == 0) {
    const int rounds = (total + G - 1) / G;
    const int per_xcd = ((total + rounds - 1) / rounds + 7) / 8;  // active per XCD
    if (static_cast<int>(blockIdx.x / 8) >= per_xcd) {
      wait_vmcnt<0>();
      return;
    }
    slot = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    stride = 8 * per_xcd;
  } else {
    slot = blockIdx.x;
    stride = G;
  }

  constexpr int W_PER_MAT = C::W_BYTES / 1024;   // DMA instructions per weight matrix
  constexpr int IPS = C::SB_BYTES / 1024;        // instructions per weight sub-block
  constexpr bool FP8 = C::WBITS == 8 && !C::MX;  // per-column fp32 scales
  constexpr bool MX = C::MX;                     // block scale bytes (MXFP4, MXFP8)
  static_assert(!(FP8 || MX) || PACKED, "fp8 and mxfp4 weights exist only in packed layouts");
  constexpr int RPI_X = 1024 / (C::BK * 2);      // activation rows per instruction

  // ---- one work item: where its operands are, its K range, its output ----
  struct ItemInfo {
    const bf16_t* w0;
    const bf16_t* w1;
    const bf16_t* x;  // activations of the tile's first row (x itself when gathering)
    OutT* out;        // output of this item's K-slice
    bf16_t* out2;     // backward epilogues: second and third outputs, G and U inputs
    bf16_t* out3;
    const bf16_t* aux0;
    const bf16_t* aux1;
    const bf16_t* aux2;
    const float* wrow;
    float* part;
    int K, N;
    int seg;          // segment of the item's group (0 routed, 1 shared)
    int n0;           // first output column
    int row_base;     // first activation row
    int rows_valid;   // rows of the tile inside the group
    int kt_begin;     // first K-step (BK each) of the slice
    int nk;           // K-steps of the slice
    int nk_all;       // K-steps of the whole K
    int nblk, kblk;   // packed: 64-column and 64-row blocks of one group
    const void* sc0;  // fp8: the group's column scales (gate / plain matrix, up);
    const void* sc1;  // mxfp4/mxfp8: sc0 = this wave's slot source of the scale bytes
    // per-lane byte offsets of this wave's DMA sources within a K-step,
    // relative to the step's scalar base
    uint32_t voff[C::OPW];
  };
  auto make_item = [&](int item) INL {
    // group owning the item: the largest g with s_pref[g] <= item
    int lo = 0, hi = NG;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= item) lo = mid; else hi = mid;
    }
    GroupView v;
    v.seg = lo < prob.seg[0].ngroups ? 0 : 1;
    v.local = v.seg ? lo - prob.seg[0].ngroups : lo;
    const int2 rows = s_rows[lo];
    v.r0 = rows.x;
    v.M = rows.y;
    const GemmSegment& S = v.seg ? prob.seg[1] : prob.seg[0];
    ItemInfo it;
    it.K = S.K;
    it.N = S.N;
    it.seg = v.seg;
    const int mtiles = (v.M + C::BT - 1) / C::BT;
    int local = item - s_pref[lo];
    const int ksplit = S.ksplit;
    const int ks = local % ksplit;
    local /= ksplit;
    const int mt = local % mtiles;
    it.n0 = (local / mtiles) * C::BF;
    it.row_base = v.r0 + mt * C::BT;
    it.rows_valid = min(C::BT, v.M - mt * C::BT);
    // K range of this slice: whole K-steps (the last step of K may be short),
    // split as evenly as the steps allow, so that no slice is empty when
    // there are at least as many steps as slices (the plan keeps >= 4 per slice)
    const int nk_all = (S.K + C::BK - 1) / C::BK;
    it.kt_begin = ks * nk_all / ksplit;
    it.nk = (ks + 1) * nk_all / ksplit - it.kt_begin;
    it.nk_all = nk_all;
    it.nblk = (S.N + 63) / 64;
    it.kblk = (S.K + 63) / 64;
    it.w0 = S.w0 + static_cast<int64_t>(v.local) * S.w_stride;
    it.w1 = C::GATED ? S.w1 + static_cast<int64_t>(v.local) * S.w_stride : it.w0;
    // gathered rows: row p of the group's block is activation row S.gather[p]
    it.x = S.gather ? S.act : S.act + static_cast<int64_t>(it.row_base) * it.K;
    it.out = static_cast<OutT*>(S.out) + static_cast<int64_t>(ks) * S.slice_stride;
    it.out2 = uniform(static_cast<bf16_t*>(S.out2));
    it.out3 = uniform(static_cast<bf16_t*>(S.out3));
    it.aux0 = uniform(S.aux0);
    it.aux1 = uniform(S.aux1);
    it.aux2 = uniform(S.aux2);
    it.wrow = uniform(S.wrow);
    it.part = uniform(S.part);
    if constexpr (FP8) {
      it.sc0 = static_cast<const float*>(S.scale0) + static_cast<int64_t>(v.local) * S.N;
      it.sc1 = C::GATED ? static_cast<const float*>(S.scale1) + static_cast<int64_t>(v.local) * S.N
                        : it.sc0;
    } else if constexpr (MX) {
      // scale bytes [G][nblk][4 * ceil(K/128)][64]; each wave loads one slot
      // of every stage's scales: piece (matrix m, sub-block sb), so the item
      // keeps only that slot's source at K-block 0 (a stage adds its K-block)
      const int kb = mx_scale_kblocks(S.K);
      const int64_t per_group = static_cast<int64_t>(it.nblk) * kb * 64;
      const int pw = (wave * C::SC_SLOT) / C::SC_PIECE;
      const int m = pw / C::SB, sb = pw % C::SB;
      const int nb = min(it.n0 / 64 + sb, it.nblk - 1);  // sub-blocks past N: the last
      it.sc0 = static_cast<const uint8_t*>(m ? S.scale1 : S.scale0) + v.local * per_group +
               static_cast<int64_t>(nb) * kb * 64 + (wave * C::SC_SLOT) % C::SC_PIECE;
      it.sc1 = it.sc0;
    } else {
      it.sc0 = it.sc1 = nullptr;
    }
    // every field is wave-uniform: keep them in scalar registers
    it.w0 = uniform(it.w0);
    it.w1 = uniform(it.w1);
    it.x = uniform(it.x);
    it.out = uniform(it.out);
    if constexpr (FP8 || MX) {
      it.sc0 = uniform(it.sc0);
      it.sc1 = uniform(it.sc1);
    }
    it.K = __builtin_amdgcn_readfirstlane(it.K);
    it.N = __builtin_amdgcn_readfirstlane(it.N);
    it.seg = __builtin_amdgcn_readfirstlane(it.seg);
    it.n0 = __builtin_amdgcn_readfirstlane(it.n0);
    it.row_base = __builtin_amdgcn_readfirstlane(it.row_base);
    it.rows_valid = __builtin_amdgcn_readfirstlane(it.rows_valid);
    it.kt_begin = __builtin_amdgcn_readfirstlane(it.kt_begin);
    it.nk = __builtin_amdgcn_readfirstlane(it.nk);
    it.nk_all = __builtin_amdgcn_readfirstlane(it.nk_all);
    it.nblk = __builtin_amdgcn_readfirstlane(it.nblk);
    it.kblk = __builtin_amdgcn_readfirstlane(it.kblk);
    {
#pragma unroll
      for (int i = 0; i < C::OPW; ++i) {
        const int j = i * C::NW + wave;
        if (i < C::W_INSTR / C::NW) {
          const int mat = j / W_PER_MAT;
          const int jj = j - mat * W_PER_MAT;  // instruction within the matrix
          const int r = (jj % IPS) * 8 + lane / 8;
          const int col = min(it.n0 + (jj / IPS) * 64 + swz_w(r, lane % 8) * 8, it.N - 8);
          it.voff[i] = PACKED ? static_cast<uint32_t>(lane) * 16u
                                 : static_cast<uint32_t>(r * it.N + col) * 2u;
          if constexpr (TRANSW) {
            // [N][K] weights into the packed LDS order: the instruction fills
            // 16 column rows (64 bytes: 32 K-values) of half q / 4 of its
            // sub-block; the lane's chunk holds logical chunk p ^ ((c >> 1) & 3)
            const int q = jj % IPS;
            const int c = (q % 4) * 16 + lane / 4;
            const int n = min(it.n0 + (jj / IPS) * 64 + c, it.N - 1);
            const int kc = (q / 4) * 32 + ((lane % 4) ^ ((c >> 1) & 3)) * 8;
            it.voff[i] = static_cast<uint32_t>(n * it.K + kc) * 2u;
          }
        } else {
          const int r = (j - C::W_INSTR) * RPI_X + lane / (C::BK / 8);
          const int kc = swz_x<C::BK>(r, lane % (C::BK / 8)) * 8;
          const int rr = min(r, it.rows_valid - 1);
          const int row = S.gather ? min(max(S.gather[it.row_base + rr], 0), S.gather_rows - 1)
                                   : rr;
          it.voff[i] = static_cast<uint32_t>(row * it.K + kc) * 2u;
        }
      }
    }
    return it;
  };

  // ---- DMA of one K-step of an item into one ring buffer ----
  // Instruction i of this wave fills 16-byte slots 64*j .. 64*j+63 of the
  // stage, j = i*NW + wave, so whether it loads weights (and which matrix)
  // or activations is known at compile time. A weight instruction fills 8
  // rows of one 64-column sub-block; an activation instruction whole rows of
  // the [BT][BK] tile. The lane's slot is a tile (row, physical chunk); the
  // swizzle gives the logical chunk, hence the global source (row-major
  // weights), or the packed weights hold the block in LDS order already.
  // Rows and columns are clamped to the valid range: clamped lanes fetch
  // finite in-bounds data whose products only reach masked outputs or
  // activation columns past K, whose fragments are zeroed (K-steps past the
  // item's range load rows that are in bounds and never used).
  auto issue = [&](const ItemInfo& it, int kt, char* buf) INL {
    // Steps past the item's range re-load the last step of K. Each source is
    // a scalar base (matrix, step) plus the item's lane offset; in the last
    // step of a K that is not a whole number of steps (KTAIL) the rows past K
    // (weights) and the columns past K (activations) are clamped to the last
    // ones inside K.
    const int64_t k0 = static_cast<int64_t>(min(kt, it.nk_all - 1)) * C::BK;
    const int kleft = it.K - static_cast<int>(k0);  // K values from k0 on
#pragma unroll
    for (int i = 0; i < C::OPW; ++i) {
      const int j = i * C::NW + wave;
      const bf16_t* base;
      uint32_t voff = it.voff[i];
      if (i < C::W_INSTR / C::NW) {
        const int mat = j / W_PER_MAT;  // wave-uniform
        const int jj = j - mat * W_PER_MAT;  // instruction within the matrix
        const bf16_t* const w = mat ? it.w1 : it.w0;
        if constexpr (PACKED) {
          // 64x64 blocks in LDS order, [n-block][k-block]; the instruction
          // copies 8 consecutive rows (1 KB) of one block. Sub-blocks past N
          // re-load the last block (their outputs are masked).
          const int nb = min(it.n0 / 64 + jj / IPS, it.nblk - 1);
          // blocks of BLK bf16-unit elements, two 32-row halves each:
          // 8 KB blocks [32-row half][64 columns][32 K-values] (bf16); 4 KB
          // of codes [32-row half][64 columns][32 bytes] (8-bit, 2 codes per
          // bf16 unit); 2 KB of E2M1 codes [32-row half][64 columns][16
          // bytes] (4 codes per unit). A 32-deep step reads one half, a
          // 64-deep step the whole block. The instruction's block row at
          // K-block 0 is the same for every step of the item, so it is
          // formed apart from the step's K offset.
          constexpr int BLK = C::WBITS == 8 ? 2048 : C::WBITS == 4 ? 1024 : 4096;
          const bf16_t* const wrow =
              w + static_cast<int64_t>(nb) * it.kblk * BLK + (jj % IPS) * 512;
          const uint32_t kb = static_cast<uint32_t>(k0);  // >= 0, below K
          base = wrow + static_cast<int64_t>(kb >> 6) * BLK + ((kb >> 5) & 1u) * (BLK / 2);
        } else if constexpr (TRANSW) {
          base = w + k0;
          if constexpr (KTAIL) {
            const int q = jj % IPS;
            const int c = (q % 4) * 16 + lane / 4;
            const int kc = (q / 4) * 32 + ((lane % 4) ^ ((c >> 1) & 3)) * 8;
            if (kc > kleft - 8) voff -= static_cast<uint32_t>(kc - (kleft - 8)) * 2u;
          }
        } else {
          base = w + k0 * it.N;
          if constexpr (KTAIL) {
            const int r = (jj % IPS) * 8 + lane / 8;
            if (r >= kleft) voff -= static_cast<uint32_t>((r - kleft + 1) * it.N) * 2u;
          }
        }
      } else {
        base = it.x + k0;
        if constexpr (KTAIL) {
          const int r = (j - C::W_INSTR) * RPI_X + lane / (C::BK / 8);
          const int kc = swz_x<C::BK>(r, lane % (C::BK / 8)) * 8;
          if (kc > kleft - 8) voff -= static_cast<uint32_t>(kc - (kleft - 8)) * 2u;
        }
      }
      dma16(base, voff, buf + j * 1024);
    }
    if constexpr (MX) {
      // this wave's slot of the stage's scale bytes (piece and offset fixed
      // per item, in sc0), BK/32 K-blocks of 64 columns from K-block k0/32
      constexpr int LANES = C::SC_SLOT / 16;
      const uint8_t* sbase = static_cast<const uint8_t*>(it.sc0) + (k0 / 32) * 64;
      char* const dst = buf + C::OP_BYTES + wave * C::SC_SLOT;
      if (LANES == kWave || lane < LANES) dma16(sbase, static_cast<uint32_t>(lane) * 16u, dst);
    }
  };

  floatx4 acc[C::NMAT][C::FF][C::FT];

  // MFMA operand fragments of one stage (all its 32-deep substeps)
  struct Frags {
    bf16x8 a[C::BK / 32][C::NMAT][C::FF];
    bf16x8 b[C::BK / 32][C::FT];
  };
  auto weight_frag = [&](const char* buf, int s, int m, int fi) INL {
    if constexpr (FP8) {
      // the lane's column and its 8 consecutive K codes (one 8-byte chunk
      // of the column's 32 bytes in this 32-row half; chunk q sits at
      // q ^ ((c >> 2) & 3), so 16 lanes of one q cover all banks), widened
      // exactly to bf16 (the column's scale is applied in the epilogue)
      const int col = wf * C::TF + fi * 16 + i16;
      const int c = col & 63;
      const char* p = buf + m * C::W_BYTES + (col >> 6) * C::SB_BYTES + s * 2048 + c * 32 +
                      ((g16 ^ ((c >> 2) & 3)) << 3);
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      return fp8x8_to_bf16(u);
    } else if constexpr (MX && C::WBITS == 8) {
      // MXFP8: the lane's column and its 8 consecutive K codes (one 8-byte
      // chunk, as for fp8 above), widened exactly to bf16 with the
      // K-block's scale byte (behind the stage's operands, as for mxfp4)
      const int col = wf * C::TF + fi * 16 + i16;
      const int c = col & 63;
      const char* p = buf + m * C::W_BYTES + (col >> 6) * C::SB_BYTES + s * 2048 + c * 32 +
                      ((g16 ^ ((c >> 2) & 3)) << 3);
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      const uint32_t e8 = *reinterpret_cast<const uint8_t*>(
          buf + C::OP_BYTES + ((m * C::SB + (col >> 6)) * (C::BK / 32) + s) * 64 + c);
      return fp8x8_scaled_to_bf16(u, __uint_as_float(e8 << 23));
    } else if constexpr (MX) {
      // the lane's column and its 8 consecutive K codes (one dword of the
      // column's 16 bytes in this 32-row half; 16 consecutive columns' rows
      // fill all 64 banks), widened exactly to bf16 with the K-block's scale
      const int col = wf * C::TF + fi * 16 + i16;
      const int c = col & 63;
      const char* sub = buf + m * C::W_BYTES + (col >> 6) * C::SB_BYTES;
      const uint32_t u = *reinterpret_cast<const uint32_t*>(sub + s * 1024 + c * 16 + g16 * 4);
      const uint32_t e8 = *reinterpret_cast<const uint8_t*>(
          buf + C::OP_BYTES + ((m * C::SB + (col >> 6)) * (C::BK / 32) + s) * 64 + c);
      return fp4x8_to_bf16(u, __uint_as_float(e8 << 23));
    } else if constexpr (PACKED || TRANSW) {
      // packed bf16 (and [N][K] weights, staged in the same order): each
      // column's 32 K-values of a half are one 64-byte row
      // (16-byte chunk q at q ^ ((c >> 1) & 3)), so the lane's 8 consecutive
      // K-values of its column are one 16-byte read
      const int col = wf * C::TF + fi * 16 + i16;
      const int c = col & 63;
      const char* p = buf + m * C::W_BYTES + (col >> 6) * C::SB_BYTES + s * 4096 + c * 64 +
                      ((g16 ^ ((c >> 1) & 3)) << 4);
      return *reinterpret_cast<const bf16x8*>(p);
    }
    const int row = s * 32 + 8 * g16 + (i16 >> 2);          // k within the stage
    const int col = wf * C::TF + fi * 16 + 4 * (i16 & 3);   // column within the tile
    const int c64 = col & 63;                                // column within the sub-block
    const int chunk = swz_w(row, c64 >> 3);                  // rows row, row+4 share it
    const char* p = buf + m * C::W_BYTES + (col >> 6) * C::SB_BYTES + row * 128 + chunk * 16 +
                    (c64 & 7) * 2;
    const short4_t lo4 = lds_read_tr16(p);
    const short4_t hi4 = lds_read_tr16(p + 4 * 128);
    typedef short short8_t __attribute__((ext_vector_type(8)));
    const short8_t s8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8, s8);
  };
  // kvalid: K values of the stage inside K. The lane's 8 K values start at a
  // multiple of 8 and K is a multiple of 8, so they are all valid or all
  // past K; past K the fragment is zeroed (the DMA loaded clamped, finite
  // columns there), which makes the products with whatever weight rows the
  // clamped DMA put beside them exactly 0.
  auto act_frag = [&](const char* buf, int s, int ti, int kvalid) INL {
    const int tok = wt * C::TT + ti * 16 + i16;
    const int chunk = swz_x<C::BK>(tok, s * 4 + g16);
    bf16x8 v = *reinterpret_cast<const bf16x8*>(buf + C::NMAT * C::W_BYTES +
                                                 tok * (C::BK * 2) + chunk * 16);
    if (KTAIL && s * 32 + 8 * g16 >= kvalid) v = bf16x8{};
    return v;
  };
  // widened (bf16, packed-layout) weight fragment: [matrix][sub-block]
  // [64 columns][32 K-values], 16-byte chunk q at q ^ ((c >> 1) & 3)
  auto wide_frag = [&](const char* wbuf, int m, int fi) INL {
    const int col = wf * C::TF + fi * 16 + i16;
    const int c = col & 63;
    return *reinterpret_cast<const bf16x8*>(wbuf + m * (C::BK * C::BF * 2) + (col >> 6) * 4096 +
                                            c * 64 + ((g16 ^ ((c >> 1) & 3)) << 4));
  };
  // A stage's codes widened into the bf16 tile, in units of 16 codes (half
  // of one column's 32); unit u = thread index (+ kThreads), so the first
  // threads' units cover the first columns. Unit cr = (matrix, sub-block,
  // column) is the column's row of bf16 values at cr * 64; block scales
  // (mxfp8, mxfp4): the 32 codes are one K-block, whose scale byte is byte
  // cr of the stage's scales.
  //  - 8-bit codes: the column's codes at cr * 32; its logical chunks 2hr
  //    and 2hr+1 sit at physical positions 2hr ^ x and (2hr ^ x) ^ 1,
  //    x = (c >> 2) & 3: one aligned 16-byte pair, read with one instruction
  //    (one address register per ring stage instead of two).
  //  - 4-bit codes: the column's codes at cr * 16, dword q holding K rows
  //    8q .. 8q+7; the unit's rows 16hr .. 16hr+15 are dwords 2hr and 2hr+1.
  auto widen = [&](const char* codes, char* wbuf) INL {
    constexpr int UNITS = C::NMAT * C::SB * 64 * 2;
#pragma unroll
    for (int u0 = 0; u0 < UNITS; u0 += C::kThreads) {
      const int unit = u0 + tid;
      const int cr = unit >> 1, hr = unit & 1;
      const int c = cr & 63;
      float scale = 1.f;
      if constexpr (MX) {
        const uint32_t e8 = *reinterpret_cast<const uint8_t*>(codes + C::OP_BYTES + cr);
        scale = __uint_as_float(e8 << 23);
      }
      const int y = (c >> 1) & 3;             // the bf16 tile's chunk rotation
      char* const wb = wbuf + cr * 64;
      if constexpr (C::WBITS == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(codes + cr * 16 + hr * 8);
        const int q0 = 2 * hr;
        *reinterpret_cast<bf16x8*>(wb + ((q0 ^ y) << 4)) = fp4x8_to_bf16(v.x, scale);
        *reinterpret_cast<bf16x8*>(wb + (((q0 + 1) ^ y) << 4)) = fp4x8_to_bf16(v.y, scale);
      } else {
        const int x = (c >> 2) & 3;
        const int p0 = (2 * hr) ^ (x & 2);  // even position of the pair
        const uint4 v = *reinterpret_cast<const uint4*>(codes + cr * 32 + p0 * 8);
        const int qlo = p0 ^ x, qhi = qlo ^ 1;  // logical chunks of the low and high half
        const uint2 lo = uint2{v.x, v.y}, hi = uint2{v.z, v.w};
        *reinterpret_cast<bf16x8*>(wb + ((qlo ^ y) << 4)) =
            MX ? fp8x8_scaled_to_bf16(lo, scale) : fp8x8_to_bf16(lo);
        *reinterpret_cast<bf16x8*>(wb + ((qhi ^ y) << 4)) =
            MX ? fp8x8_scaled_to_bf16(hi, scale) : fp8x8_to_bf16(hi);
      }
    }
  };
  auto load_frags = [&](const char* buf, Frags& F, int kvalid) INL {
#pragma unroll
    for (int s = 0; s < C::BK / 32; ++s) {
#pragma unroll
      for (int ti = 0; ti < C::FT; ++ti) F.b[s][ti] = act_frag(buf, s, ti, kvalid);
#pragma unroll
      for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m) F.a[s][m][fi] = weight_frag(buf, s, m, fi);
    }
  };
  // live: the wave's 16-row token blocks that hold at least one row of the
  // item (blocks 0 .. live-1). In the widening tiles the MFMAs of the other
  // blocks are skipped: the epilogue stores none of their rows, and each
  // accumulator still takes its K-substeps in order, so the stored sums are
  // unchanged (FP8 layer at the DeepSeek-V3-shaped T = 4096 6.57 -> 6.41 ms,
  // Mixtral-shaped T = 512 0.77 -> 0.73 ms, T = 8192 5.39 -> 5.28 ms). The
  // bf16 tiles keep the whole burst: the branch cost the 256-row ping-pong
  // tile 2-3 % at T = 8192 (a uniform skip of whole bands as well), and among
  // the prefetching tiles' interleaved fragment reads it made them spill.
  constexpr bool kSkipDeadBlocks = C::FT > 1 && C::WIDEN;
  auto mfma = [&](const Frags& F, int live) INL {
    if constexpr (kSkipDeadBlocks) {
#pragma unroll
      for (int ti = 0; ti < C::FT; ++ti) {
        if (ti >= live) break;
#pragma unroll
        for (int s = 0; s < C::BK / 32; ++s)
#pragma unroll
          for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
              acc[m][fi][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  F.a[s][m][fi], F.b[s][ti], acc[m][fi][ti], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < C::BK / 32; ++s)
#pragma unroll
        for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int ti = 0; ti < C::FT; ++ti)
              acc[m][fi][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  F.a[s][m][fi], F.b[s][ti], acc[m][fi][ti], 0, 0, 0);
    }
  };

  // the wave's live token blocks of an item (wave-uniform)
  auto live_blocks = [&](const ItemInfo& it) INL {
    const int r = it.rows_valid - wt * C::TT;
    return __builtin_amdgcn_readfirstlane(r <= 0 ? 0 : min(C::FT, (r + 15) / 16));
  };
  // Without prefetch, the gated kernel interleaves the weight-fragment reads
  // column block by column block with the MFMAs that use them; the plain
  // kernel reads all fragments first (each order measured faster for its
  // kernel), except on mxfp4 weights, where all widened fragments of a
  // 64-deep stage would not fit the registers.
  auto compute_interleaved = [&](const char* buf, int kvalid, int live) INL {
#pragma unroll
    for (int s = 0; s < C::BK / 32; ++s) {
      bf16x8 b[C::FT];
#pragma unroll
      for (int ti = 0; ti < C::FT; ++ti) b[ti] = act_frag(buf, s, ti, kvalid);
#pragma unroll
      for (int fi = 0; fi < C::FF; ++fi) {
        bf16x8 a[C::NMAT];
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m) a[m] = weight_frag(buf, s, m, fi);
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
          for (int ti = 0; ti < C::FT; ++ti) {
            if (kSkipDeadBlocks && ti >= live) break;
            acc[m][fi][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a[m], b[ti], acc[m][fi][ti], 0, 0, 0);
          }
      }
    }
  };

  // ---- the ring ----
  // K-step t of an item lives in buffer t % S. Without prefetch, step t
  // waits for K-step t, refills the buffer of step t-1 with step t+S-1 and
  // multiplies step t: S-1 steps in flight. With prefetch, step t waits for
  // K-step t+1, refills buffer t % S (step t's fragments were read into
  // registers during step t-1) with step t+S, reads step t+1's fragments and
  // multiplies step t's: S steps in flight. Either way each wave then has at
  // most S-2 newer K-steps outstanding, so every wait count is a constant;
  // the lgkmcnt(0) in the wait makes every wave's reads of the buffer being
  // refilled complete before the barrier.
  //
  // Items are chained (prefetching tiles): when an item's K-steps are a whole number of
  // unrolled turns (below) and the next item of this workgroup has at least D of them, the
  // last refills of the item already fetch the next item's first D steps
  // (into buffers 0.., as its own prologue would), so the ring never drains
  // between items. Otherwise refills past the end re-load in-bounds rows of
  // the item (their values are never used) and the next item starts with a
  // drained ring.
  constexpr int S = C::STAGES;
  constexpr int D = C::PREFETCH ? S : S - 1;  // K-steps in flight after a refill
  // Steps are unrolled a turn at a time, so that each step's buffer and
  // fragment set are compile-time choices. Prefetching alternates two
  // fragment sets by step parity, so its turn is an even number of steps
  // (two ring turns when S is odd).
  constexpr int TURN = (C::PREFETCH && S % 2 == 1) ? 2 * S : S;
  constexpr int WAIT = (S - 2) * C::IPW;
  // Chaining is used by the decode-size (prefetching) tiles, whose time is
  // memory latency; the large tiles keep their registers for the MFMA
  // operands and restart the ring per item.
  constexpr bool CHAIN = C::CHAIN_OK && !KTAIL;
  auto stage_buf = [&](auto I) INL -> char* {
    constexpr int i = decltype(I)::value % S;
    if constexpr (i == 0) return st0;
    else if constexpr (i == 1) return st1;
    else if constexpr (i == 2) return st2;
    else if constexpr (i == 3) return st3;
    else if constexpr (i == 4) return st4;
    else if constexpr (i == 5) return st5;
    else if constexpr (i == 6) return st6;
    else return st7;
  };

  Frags fa, fb;
  bool primed = false;  // the current item's first D K-steps are in flight

  // ---- ping-pong schedule (C::PP) ----
  // Waves 0-3 (group 0) and 4-7 (group 1) hold one wave per SIMD each. Every
  // K-step is a memory phase M (read the step's fragments from LDS, wait for
  // the wave's own DMA of the next step, issue the DMA of step t+D, wait for
  // the fragments; issuing the DMA first measured 3 % slower) and an MFMA
  // phase C, each closed by a workgroup barrier.
  // Group 1 passes one extra barrier first, so between any two barriers one
  // group multiplies while the other moves data:
  //   interval 2t:   group 0 M(t),  group 1 C(t-1)
  //   interval 2t+1: group 0 C(t),  group 1 M(t)
  // Step t+1 is read in intervals 2t+2 (group 0) and 2t+3 (group 1); both
  // groups' DMAs of it have landed by the end of intervals 2t and 2t+1
  // (each wave waits for its own in M(t)). Step t+D goes into the buffer of
  // step t-1 (D = S-1), whose last reads were waited for by the end of
  // interval 2t-1; group 0 issues it in interval 2t, group 1 in 2t+1. Group 0
  // passes one extra barrier at the end, so both groups leave in step.
  auto pp_barrier = [&]() INL {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // (Chaining items as the decode tiles do measured 1 % slower here: items
  // are long, and the chained start must also wait for the epilogue's stores.)
  // Widening (C::WIDEN): the memory phase M(t) also converts this group's
  // half of step t+1's codes into the bf16 tile wide[(t+1) % 2] and reads
  // step t's weight fragments from wide[t % 2]. Step t+1's codes must have
  // landed for every wave before interval 2t, so each wave waits for its DMA
  // of step t+2 in M(t) (step t+1's in M(t-1)); the prologue lands steps 0
  // and 1 and widens step 0. wide[(t+1) % 2] last held step t-1, read in
  // intervals 2t-2 and 2t-1; step t+1's halves are written in 2t and 2t+1
  // and read from 2t+2 on. The ring buffer refilled in M(t) held step t-1,
  // whose codes were widened in M(t-2) and its activations read in M(t-1).
  auto run_pingpong = [&](const ItemInfo& cur) INL {
    constexpr int DP = S - 1;
    constexpr bool WD = C::WIDEN;
    constexpr int PTURN = (WD && S % 2 == 1) ? 2 * S : S;  // wide buffer = step parity
    const bool grp1 = wave >= 4;
    const int live = kSkipDeadBlocks ? live_blocks(cur) : C::FT;
    wait_vmcnt<0>();               // the last item's stores and DMAs are done and
    __builtin_amdgcn_s_barrier();  // every wave has finished reading the ring
    static_for<DP>([&](auto I) INL { issue(cur, cur.kt_begin + decltype(I)::value, stage_buf(I)); });
    if constexpr (WD) {
      wait_vmcnt<(DP - 2) * C::IPW>();
      pp_barrier();                // K-steps 0 and 1 have landed for every wave
      widen(st0, wide0);
      wait_vmcnt_lgkm0<63>();
    } else {
      wait_vmcnt<(DP - 1) * C::IPW>();
    }
    pp_barrier();                  // K-step 0 has landed (and is widened) for every wave
    if (grp1) pp_barrier();
    auto pp_step = [&](int t, auto I) INL {
      constexpr int i = decltype(I)::value;
      if constexpr (WD) {
        char* const wcur = i % 2 == 0 ? wide0 : wide1;
        char* const wnext = i % 2 == 0 ? wide1 : wide0;
        // widen step t+1 first, so its temporaries are dead before the
        // fragments are read (registers)
        widen(stage_buf(std::integral_constant<int, i + 1>{}), wnext);
        __builtin_amdgcn_sched_barrier(0);
        const char* const sb = stage_buf(I);
        const int kvalid = cur.K - (cur.kt_begin + t) * C::BK;
#pragma unroll
        for (int ti = 0; ti < C::FT; ++ti) fa.b[0][ti] = act_frag(sb, 0, ti, kvalid);
#pragma unroll
        for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m) fa.a[0][m][fi] = wide_frag(wcur, m, fi);
        wait_vmcnt<(DP - 3) * C::IPW>();  // this wave's DMA of step t+2 has landed
      } else {
        load_frags(stage_buf(I), fa, cur.K - (cur.kt_begin + t) * C::BK);
        wait_vmcnt<(DP - 2) * C::IPW>();  // this wave's DMA of step t+1 has landed
      }
      issue(cur, cur.kt_begin + t + DP, stage_buf(std::integral_constant<int, i + DP>{}));
      wait_vmcnt_lgkm0<63>();           // fragments in registers (and widened codes written)
      pp_barrier();
      mfma(fa, live);
      pp_barrier();
    };
    const int full = cur.nk / PTURN;
    int t = 0;
    for (int turn = 0; turn < full; ++turn, t += PTURN)
      static_for<PTURN>([&](auto I) INL { pp_step(t + decltype(I)::value, I); });
    const int rem = cur.nk - t;
    static_for<PTURN - 1>([&](auto I) INL {
      if (decltype(I)::value < rem) pp_step(t + decltype(I)::value, I);
    });
    if (!grp1) pp_barrier();
  };
  for (int item = slot; item < total; item += stride) {
    const ItemInfo cur = make_item(item);
    const bool has_next = CHAIN && item + stride < total;
    const ItemInfo nx = has_next ? make_item(item + stride) : cur;
    const bool chain = has_next && cur.nk % TURN == 0 && nx.nk >= D;

#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
      for (int a = 0; a < C::FF; ++a)
#pragma unroll
        for (int b = 0; b < C::FT; ++b) acc[m][a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    if constexpr (C::PP) {
      run_pingpong(cur);
    } else {
    const int live = kSkipDeadBlocks ? live_blocks(cur) : C::FT;
    if (!primed) {
      wait_vmcnt<0>();               // every DMA into the ring has landed and
      __builtin_amdgcn_s_barrier();  // every wave is done with the last item
      static_for<D>([&](auto I) INL { issue(cur, cur.kt_begin + decltype(I)::value, stage_buf(I)); });
      if (C::PREFETCH) {
        wait_vmcnt<(D - 1) * C::IPW>();
        __builtin_amdgcn_s_barrier();  // K-step 0 has landed
        load_frags(st0, fa, cur.K - cur.kt_begin * C::BK);
      }
    }

    // step t = TURN*turn + I; I is a compile-time constant, so every buffer
    // is a fixed LDS array (no early exits inside the loop: they would keep the
    // accumulators from being updated in place and double their registers)
    auto step = [&](int t, auto I) INL {
      constexpr int i = decltype(I)::value;
      wait_vmcnt_lgkm0<WAIT>();
      __builtin_amdgcn_s_barrier();
      {
        const int u = t + D;
        char* const rb = stage_buf(std::integral_constant<int, i + D>{});
        if (CHAIN && chain && u >= cur.nk) issue(nx, nx.kt_begin + (u - cur.nk), rb);
        else issue(cur, cur.kt_begin + u, rb);
      }
      if constexpr (C::PREFETCH) {
        char* const nb = stage_buf(std::integral_constant<int, i + 1>{});
        const int kvalid = cur.K - (cur.kt_begin + t + 1) * C::BK;
        if constexpr (i % 2 == 0) {
          load_frags(nb, fb, kvalid);
          mfma(fa, live);
        } else {
          load_frags(nb, fa, kvalid);
          mfma(fb, live);
        }
      } else {
        char* const cb = stage_buf(I);
        const int kvalid = cur.K - (cur.kt_begin + t) * C::BK;
        if constexpr (C::GATED || C::MX) {
          compute_interleaved(cb, kvalid, live);
        } else {
          load_frags(cb, fa, kvalid);
          mfma(fa, live);
        }
      }
    };
    {
      const int full = cur.nk / TURN;
      int t = 0;
      for (int turn = 0; turn < full; ++turn, t += TURN)
        static_for<TURN>([&](auto I) INL { step(t + decltype(I)::value, I); });
      const int rem = cur.nk - t;
      static_for<TURN - 1>([&](auto I) INL {
        if (decltype(I)::value < rem) step(t + decltype(I)::value, I);
      });
    }
    }  // ring schedule

    // ---- epilogue: lane holds columns 4*g16..+3 of one token per block ----
    // (bf16 stores round to nearest even; fp32 stores keep the accumulator)
#pragma unroll
    for (int fi = 0; fi < C::FF; ++fi) {
      // fp8: the columns' power-of-two scales (exact on the fp32 sums)
      float4 s0 = float4{1.f, 1.f, 1.f, 1.f}, s1 = s0;
      if constexpr (FP8) {
        const int fc = min(cur.n0 + wf * C::TF + fi * 16 + 4 * g16, cur.N - 4);
        s0 = *reinterpret_cast<const float4*>(static_cast<const float*>(cur.sc0) + fc);
        if (C::GATED) s1 = *reinterpret_cast<const float4*>(static_cast<const float*>(cur.sc1) + fc);
      }
      // (only in the transposed-weight bf16 kernels, which the backward's dh
      // product runs: the forward's kernels carry no code for it)
      if constexpr (TRANSW && !C::GATED && sizeof(OutT) == 2) {
        if (prob.epi == kSwigluBwd) {
          // acc = g = dout W_down^T for the row; with its routing weight w
          // and the forward's G, U, h: dh = w g, dG = dh U silu'(G),
          // dU = dh silu(G), silu'(z) = s (1 + z (1 - s)), s = 1/(1+e^-z);
          // and the fragment's partial sum of h g (the routing-weight
          // gradient <dout, y> = <h, g>), summed over its 16 columns across
          // the four lanes of the token. The column's loads for all of the
          // wave's token blocks are issued first, with no store between
          // them, so that they are in flight together (issued block by
          // block between the stores, each block waited for its own).
          const int f = cur.n0 + wf * C::TF + fi * 16 + 4 * g16;
          uint2 gq[C::FT], uq[C::FT], hq[C::FT];
          float wv[C::FT];
#pragma unroll
          for (int ti = 0; ti < C::FT; ++ti) {
            const int tok = wt * C::TT + ti * 16 + i16;
            gq[ti] = uq[ti] = hq[ti] = uint2{0u, 0u};
            wv[ti] = 0.f;
            if (tok < cur.rows_valid && f < cur.N) {
              const int64_t o = static_cast<int64_t>(cur.row_base + tok) * cur.N + f;
              gq[ti] = *reinterpret_cast<const uint2*>(cur.aux0 + o);
              uq[ti] = *reinterpret_cast<const uint2*>(cur.aux1 + o);
              hq[ti] = *reinterpret_cast<const uint2*>(cur.aux2 + o);
              wv[ti] = cur.wrow[cur.row_base + tok];
            }
          }
#pragma unroll
          for (int ti = 0; ti < C::FT; ++ti) {
            const int tok = wt * C::TT + ti * 16 + i16;
            float part = 0.f;
            if (tok < cur.rows_valid && f < cur.N) {
              const int64_t o = static_cast<int64_t>(cur.row_base + tok) * cur.N + f;
              const uint32_t gw[2] = {gq[ti].x, gq[ti].y}, uw[2] = {uq[ti].x, uq[ti].y},
                             hw[2] = {hq[ti].x, hq[ti].y};
              float dg[4], du[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float g = bf16_to_f32(static_cast<bf16_t>(gw[r / 2] >> (16 * (r % 2))));
                const float u = bf16_to_f32(static_cast<bf16_t>(uw[r / 2] >> (16 * (r % 2))));
                const float hv = bf16_to_f32(static_cast<bf16_t>(hw[r / 2] >> (16 * (r % 2))));
                const float sg = sigmoid_rcp(g);
                const float gr = acc[0][fi][ti][r];
                const float dh = wv[ti] * gr;
                dg[r] = dh * u * sg * (1.0f + g * (1.0f - sg));
                du[r] = dh * g * sg;
                part += hv * gr;
              }
              store4(cur.out + o, dg);
              store4(cur.out2 + o, du);
            }
            part += __shfl_xor(part, 16, kWave);
            part += __shfl_xor(part, 32, kWave);
            const int fc = cur.n0 + wf * C::TF + fi * 16;  // the fragment's first column
            if (g16 == 0 && tok < cur.rows_valid && fc < cur.N)
              cur.part[static_cast<int64_t>(cur.row_base + tok) * ((cur.N + 15) / 16) + fc / 16] =
                  part;
          }
          continue;
        }
      }
      const float sc0[4] = {s0.x, s0.y, s0.z, s0.w};
      const float sc1[4] = {s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int ti = 0; ti < C::FT; ++ti) {
        const int tok = wt * C::TT + ti * 16 + i16;
        const int f = cur.n0 + wf * C::TF + fi * 16 + 4 * g16;
        if (tok < cur.rows_valid && f < cur.N) {
          const int64_t o = static_cast<int64_t>(cur.row_base + tok) * cur.N + f;
          float vals[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (C::GATED) {
              const float gt = FP8 ? acc[0][fi][ti][r] * sc0[r] : acc[0][fi][ti][r];
              const float up = FP8 ? acc[C::NMAT - 1][fi][ti][r] * sc1[r]
                                   : acc[C::NMAT - 1][fi][ti][r];
              vals[r] = gt * sigmoid_rcp(gt) * up;
            } else {
              vals[r] = FP8 ? acc[0][fi][ti][r] * sc0[r] : acc[0][fi][ti][r];
            }
          }
          if constexpr (C::GATED && !FP8 && !MX) {
            if (prob.epi == kStoreGUH) {  // the forward's G and U for the backward
              float g4[4], u4[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) g4[r] = acc[0][fi][ti][r], u4[r] = acc[1][fi][ti][r];
              store4(cur.out2 + o, g4);
              store4(cur.out3 + o, u4);
            }
          }
          if constexpr (kScatterTile) {
            if (prob.scat.cnt) store4_device(reinterpret_cast<float*>(cur.out) + o, vals);
            else store4(cur.out + o, vals);
          } else {
            store4(cur.out + o, vals);
          }
        }
      }
    }
    if constexpr (kScatterTile) {
      if (prob.scat.cnt) {
        const ScatterArgs& sa = prob.scat;
        // this thread's partial sums (device-scope stores) have completed
        // before any row of the item is counted
        wait_vmcnt<0>();
        __syncthreads();
        const int ncb = (cur.N + C::BF - 1) / C::BF;
        const int cb = cur.n0 / C::BF;
        if (tid < C::BT) {
          int tok = -1;
          if (tid < cur.rows_valid) {
            int t = cur.seg ? cur.row_base + tid : sa.row_token[cur.row_base + tid];
            t = min(max(t, 0), sa.T - 1);
            const int before = atomicAdd(sa.cnt + static_cast<int64_t>(t) * ncb + cb, 1);
            if (before == sa.target - 1) tok = t;
          }
          s_scat[tid] = tok;
        }
        __syncthreads();
        // the completed tokens' partial sums, read at device scope (every one
        // was stored before its row was counted)
        const int64_t A = static_cast<int64_t>(sa.T) * sa.k;
        for (int r = wave; r < cur.rows_valid; r += C::NW) {
          const int t = s_scat[r];
          if (t < 0) continue;
          for (int c = lane; c < C::BF; c += kWave) {
            const int col = cur.n0 + c;
            if (col >= cur.N) break;
            float a = 0.f;
            for (int j = 0; j < sa.k; ++j) {
              int p = sa.row_dest[static_cast<int64_t>(t) * sa.k + j];
              p = p < 0 ? 0 : (p >= A ? static_cast<int>(A - 1) : p);
              const float w = sa.topk_w ? sa.topk_w[static_cast<int64_t>(t) * sa.k + j] : 1.0f;
              const float* yp = sa.y + static_cast<int64_t>(p) * cur.N + col;
              float v = load_device(yp);
              for (int sl = 1; sl < sa.y_slices; ++sl) v += load_device(yp + sl * sa.y_slice_stride);
              a += w * v;
            }
            if (sa.y_sh) {
              const float sg =
                  sa.gate_logits ? 1.0f / (1.0f + expf(-sa.gate_logits[t])) : 1.0f;
              const float* yp = sa.y_sh + static_cast<int64_t>(t) * cur.N + col;
              float v = load_device(yp);
              for (int sl = 1; sl < sa.ysh_slices; ++sl)
                v += load_device(yp + sl * sa.ysh_slice_stride);
              a += sg * v;
            }
            sa.out[static_cast<int64_t>(t) * cur.N + col] = f32_to_bf16(a);
          }
        }
        wait_vmcnt<0>();  // the next item's ring waits count its own loads only
        __syncthreads();  // s_scat is rewritten by the next item
      }
    }
    primed = chain;
  }
  // no LDS DMA may land after the workgroup ends (its LDS may be reassigned)
  wait_vmcnt<0>();
}

// ---- register-streaming gate/up for decode-size groups ----
// Packed bf16 or fp8 weights. Each wave owns 16 output columns of a 16-row x
// 64-column item (4 waves per workgroup) and streams its weight fragments
// straight from global memory into registers: in the packed layouts a
// lane's MFMA operand (8 K-consecutive values of one column) is one 16-byte
// load (bf16) or one 8-byte load of codes widened in registers (fp8, the
// column scales applied in the epilogue), and the 16 columns of a wave
// read one contiguous run.
// No LDS and no barriers: every wave keeps kRsD K-steps (64 deep) of loads
// in flight in a ring of registers, and its step sequence runs across its
// items without draining (the loads of the next item start while the
// current one is finished). The compiler's own waits (vmcnt, in load order)
// hold each step back until its loads have landed. Activations (16 rows of
// the item) are read the same way; they are small and come from L2.
int device_cu_count();

constexpr int kRsWaves = 4;
constexpr int kRsThreads = kRsWaves * kWave;
constexpr int kRsD = 6;      // K-steps in flight per wave
constexpr int kRsBT = 16;    // rows per item
constexpr int kRsBF = 64;    // columns per item (16 per wave)

template <int WBITS>
__global__ __launch_bounds__(kRsThreads) void rs_gateup_kernel(GemmProblem prob) {
  static_assert(WBITS == 16 || WBITS == 8, "bf16 or fp8 weights");
  constexpr bool FP8 = WBITS == 8;
  // bytes of a 64 x 64 weight block and of one 32-deep half of it
  constexpr int BLK = 64 * 64 * WBITS / 8, HALF = BLK / 2;
  extern __shared__ __attribute__((aligned(16))) int s_pref[];
  __shared__ int s_wave_total[kRsWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g16 = lane >> 4, i16 = lane & 15;

  // item prefix over all groups of both segments (as in grouped_gemm_kernel)
  const int NG = prob.seg[0].ngroups + (prob.nseg > 1 ? prob.seg[1].ngroups : 0);
  int2* const s_rows = reinterpret_cast<int2*>(s_pref + ((NG + 2) & ~1));
  constexpr int GPT = (kMaxGroups + kRsThreads - 1) / kRsThreads;
  int cnt[GPT];
  int my_sum = 0;
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    cnt[i] = 0;
    if (g < NG) {
      const GroupView v = group_view(prob, g);
      const GemmSegment& S = v.seg ? prob.seg[1] : prob.seg[0];
      cnt[i] = ((v.M + kRsBT - 1) / kRsBT) * ((S.N + kRsBF - 1) / kRsBF);
      s_rows[g] = int2{v.r0, v.M};
    }
    my_sum += cnt[i];
  }
  const int incl = wave_inclusive_scan(my_sum);
  if (lane == kWave - 1) s_wave_total[wave] = incl;
  __syncthreads();
  int run = incl - my_sum;
  for (int w = 0; w < wave; ++w) run += s_wave_total[w];
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    if (g <= NG) s_pref[g] = run;
    run += cnt[i];
  }
  __syncthreads();
  const int total = s_pref[NG];
  if (total == 0) return;
  // balanced persistent slots, XCD-contiguous (as in grouped_gemm_kernel)
  const int G = gridDim.x;
  int slot, stride;
  if (G % 8 == 0) {
    const int rounds = (total + G - 1) / G;
    const int per_xcd = ((total + rounds - 1) / rounds + 7) / 8;
    if (static_cast<int>(blockIdx.x / 8) >= per_xcd) return;
    slot = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    stride = 8 * per_xcd;
  } else {
    slot = blockIdx.x;
    stride = G;
  }
  if (slot >= total) return;
  const int K = prob.seg[0].K;           // one K for both segments (host-checked)
  const int nk = (K + 63) / 64;
  const int kblk = nk;
  const int nitems = (total - slot + stride - 1) / stride;
  const int nsteps = nitems * nk;

  struct Cur {
    const char* w0;      // the item's 64-column block row (bytes)
    const char* w1;
    const bf16_t* x;     // the item's first activation row
    bf16_t* out;
    const float* sc0;    // fp8: the group's column scales (gate, up)
    const float* sc1;
    int N, n0, row_base, rows_valid;
  };
  auto item_info = [&](int item) INL {
    int lo = 0, hi = NG;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= item) lo = mid; else hi = mid;
    }
    const int segi = lo < prob.seg[0].ngroups ? 0 : 1;
    const int local_g = segi ? lo - prob.seg[0].ngroups : lo;
    const GemmSegment& S = segi ? prob.seg[1] : prob.seg[0];
    const int2 rows = s_rows[lo];
    const int mtiles = (rows.y + kRsBT - 1) / kRsBT;
    const int local = item - s_pref[lo];
    const int mt = local % mtiles;
    Cur c;
    c.N = S.N;
    c.n0 = (local / mtiles) * kRsBF;
    c.row_base = rows.x + mt * kRsBT;
    c.rows_valid = min(kRsBT, rows.y - mt * kRsBT);
    const int64_t blk0 = static_cast<int64_t>(c.n0 / 64) * kblk * BLK;  // first K-block
    c.w0 = uniform(reinterpret_cast<const char*>(S.w0 + static_cast<int64_t>(local_g) * S.w_stride) + blk0);
    c.w1 = uniform(reinterpret_cast<const char*>(S.w1 + static_cast<int64_t>(local_g) * S.w_stride) + blk0);
    c.x = uniform(S.act + static_cast<int64_t>(c.row_base) * K);
    c.out = uniform(static_cast<bf16_t*>(S.out));
    c.sc0 = c.sc1 = nullptr;
    if constexpr (FP8) {
      c.sc0 = uniform(static_cast<const float*>(S.scale0) + static_cast<int64_t>(local_g) * S.N);
      c.sc1 = uniform(static_cast<const float*>(S.scale1) + static_cast<int64_t>(local_g) * S.N);
    }
    c.N = __builtin_amdgcn_readfirstlane(c.N);
    c.n0 = __builtin_amdgcn_readfirstlane(c.n0);
    c.row_base = __builtin_amdgcn_readfirstlane(c.row_base);
    c.rows_valid = __builtin_amdgcn_readfirstlane(c.rows_valid);
    return c;
  };

  // the lane's offsets inside a K-block: column c of the wave's 16, chunk
  // g16 of each 32-deep half at its swizzled place; activation row i16
  // (bf16: 16 bytes at chunk g16 ^ ((c >> 1) & 3) of the column's 64-byte
  // row; fp8: 8 bytes at chunk g16 ^ ((c >> 2) & 3) of its 32 bytes)
  const int col = wave * 16 + i16;
  const uint32_t woff = static_cast<uint32_t>(
      FP8 ? col * 32 + ((g16 ^ ((col >> 2) & 3)) << 3)
          : (col * 32 + ((g16 ^ ((col >> 1) & 3)) << 3)) * 2);
  typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
  typedef typename std::conditional<FP8, u32x2v_t, bf16x8>::type wvec_t;
  struct Slot {
    wvec_t w[2][2];   // [matrix][half]: the lane's weights (fp8: codes)
    bf16x8 x[2];      // [half]
  };
  // loads through the global address space (not flat: a flat load also
  // counts as an LDS access, and its waits would drain every load in flight)
  typedef __attribute__((address_space(1))) const bf16x8 gvec_t;
  typedef __attribute__((address_space(1))) const wvec_t gw_t;
  auto gload = [](const bf16_t* p) INL { return *(gvec_t*)(p); };
  auto wload = [](const char* p) INL { return *(gw_t*)(p); };
  Slot ring[kRsD];
  // issue cursor
  int is_item = slot, is_k = 0, is_n = 0;
  Cur ic = item_info(is_item);
  auto issue = [&](Slot& sl) INL {
    // steps past the wave's last one re-load its last step
    const int kb = is_k;
    const char* wb0 = ic.w0 + static_cast<int64_t>(kb) * BLK;
    const char* wb1 = ic.w1 + static_cast<int64_t>(kb) * BLK;
    const int xrow = min(i16, ic.rows_valid - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sl.w[0][h] = wload(wb0 + h * HALF + woff);
      sl.w[1][h] = wload(wb1 + h * HALF + woff);
      const int k = min(kb * 64 + h * 32 + g16 * 8, K - 8);  // past K: weights are zero
      sl.x[h] = gload(ic.x + static_cast<int64_t>(xrow) * K + k);
    }
    if (is_n + 1 < nsteps) {
      ++is_n;
      if (++is_k == nk) {
        is_k = 0;
        is_item += stride;
        ic = item_info(is_item);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < kRsD; ++i) issue(ring[i]);

  floatx4 acc[2];
  acc[0] = acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
  int c_item = slot, c_k = 0;
  Cur cc = item_info(c_item);
  // fp8: the current item's column scales of the lane's 4 columns (powers
  // of two, exact on the fp32 sums). The wave's 16 columns' scales are
  // wave-uniform, so they are read with scalar loads (a separate counter):
  // a vector load here would make the epilogue wait, in load order, for the
  // whole weight stream in flight. Each lane then picks its 4 of the 16.
  f32x4_t csc0 = f32x4_t{1.f, 1.f, 1.f, 1.f}, csc1 = csc0;
  auto load_scales = [&]() INL {
    if constexpr (FP8) {
      typedef __attribute__((address_space(4))) const f32x4_t cf4_t;
      // columns n0 + 16 wave .. +15, clamped inside the group's N scales
      const int c0 = min(cc.n0 + wave * 16, cc.N - 16);
      const int sel = cc.n0 + wave * 16 + 4 * g16 - c0;   // 0, 4, 8 or 12 (or less near N)
      f32x4_t a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = *(cf4_t*)(cc.sc0 + c0 + 4 * q);
        b[q] = *(cf4_t*)(cc.sc1 + c0 + 4 * q);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // element sel + r of the 16, chosen without dynamic register indexing
        const int e = min(sel + r, 15);
        float x = a[0][0], y = b[0][0];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (e == q) x = a[q / 4][q % 4], y = b[q / 4][q % 4];
        csc0[r] = x;
        csc1[r] = y;
      }
    }
  };
  load_scales();
  auto wfrag = [&](const Slot& sl, int m, int h) INL {
    if constexpr (FP8) {
      return fp8x8_to_bf16(uint2{sl.w[m][h].x, sl.w[m][h].y});
    } else {
      return sl.w[m][h];
    }
  };
  auto step = [&](Slot& sl) INL {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag(sl, m, h), sl.x[h], acc[m], 0, 0, 0);
    issue(sl);
    if (++c_k == nk) {
      // epilogue: lane holds columns 4*g16 .. +3 of token i16
      const int f = cc.n0 + col - i16 + 4 * g16;
      if (i16 < cc.rows_valid && f < cc.N) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gt = FP8 ? acc[0][r] * csc0[r] : acc[0][r];
          const float up = FP8 ? acc[1][r] * csc1[r] : acc[1][r];
          v[r] = gt * sigmoid_rcp(gt) * up;
        }
        store4(cc.out + static_cast<int64_t>(cc.row_base + i16) * cc.N + f, v);
      }
      acc[0] = acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
      c_k = 0;
      c_item += stride;
      if (c_item < total) {
        cc = item_info(c_item);
        load_scales();
      }
    }
  };
  int s0 = 0;
  for (; s0 + kRsD <= nsteps; s0 += kRsD)
    static_for<kRsD>([&](auto I) INL { step(ring[decltype(I)::value]); });
  static_for<kRsD - 1>([&](auto I) INL {
    if (s0 + decltype(I)::value < nsteps) step(ring[decltype(I)::value]);
  });
}

template <int WBITS>
int rs_blocks_per_cu(size_t dyn) {
  static int cached_n[64] = {0};
  static size_t cached_dyn[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached_n[dev] == 0 || cached_dyn[dev] != dyn) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(rs_gateup_kernel<WBITS>), kRsThreads, dyn) !=
                hipSuccess ||
        n <= 0)
      n = 1;
    cached_n[dev] = n;
    cached_dyn[dev] = dyn;
  }
  return cached_n[dev];
}

template <int WBITS>
hipError_t launch_rs_gateup(const GemmProblem& p, hipStream_t stream) {
  int groups = 0;
  int64_t bound = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    groups += S.ngroups;
    bound += ((S.rows + kRsBT - 1) / kRsBT + (S.offsets ? S.ngroups : 0)) *
             static_cast<int64_t>((S.N + kRsBF - 1) / kRsBF);
  }
  if (bound <= 0) return hipSuccess;
  const size_t dyn = static_cast<size_t>((groups + 2) & ~1) * sizeof(int) +
                     static_cast<size_t>(groups) * sizeof(int2);
  int64_t grid = static_cast<int64_t>(device_cu_count()) * rs_blocks_per_cu<WBITS>(dyn);
  if (bound < grid) grid = bound;
  grid = (grid + 7) / 8 * 8;
  MOE_TRACE_LAUNCH("rs_gateup_kernel", dim3(static_cast<unsigned>(grid)), dim3(kRsThreads), dyn,
                   "tile=%dx%d wbits=%d segments=%d groups=%d items<=%lld", kRsBT, kRsBF, WBITS,
                   p.nseg, groups, static_cast<long long>(bound));
  hipLaunchKernelGGL((rs_gateup_kernel<WBITS>), dim3(static_cast<unsigned>(grid)),
                     dim3(kRsThreads), dyn, stream, p);
  return hipGetLastError();
}

// Tile shapes (BT tokens x BF columns, BK per stage, waves, ring depth).
// Large batch: 256 tokens x 128 columns (gated: 128 columns each of gate and
// up; down: 256 columns), 8 waves (2 per SIMD) as 4 along tokens x 2 along
// columns, 128 accumulators per lane, a 4-deep ring of 32-deep, 32 KB stages
// (three stages of look-ahead), on the ping-pong schedule (the ring schedule
// of the other tiles was 12-16 % slower at 8192 tokens of the Mixtral-shaped
// layer). Its time is set by the direct-to-LDS stream: the same launch with
// the MFMAs and fragment reads removed takes about 80 % of the full time,
// with the DMA removed about 65 %, and the DMA time halves with half the
// bytes.
// Small batch (decode): gate/up 16 tokens x 64 columns on 2 waves with a
// 4-deep ring of 18 KB stages (2 workgroups and ~108 KB of weights in flight
// per CU); down 32 tokens x 64 columns on 4 waves, 4-deep ring of 12 KB
// stages (3 workgroups per CU); both read the next stage's fragments while
// the current stage's MFMAs run (the large tiles have no registers to spare
// for a second fragment set). Mid (gate/up at 16..63 rows per group):
// 32 tokens x 64 columns, 2 waves, 3-deep ring of 20 KB, 64-deep stages
// (2 workgroups per CU, all stages in flight): half the row tiles per expert
// of the small tile (9 % faster than a 4-deep ring of 32-deep stages at the
// Mixtral-shaped layer's 128 tokens).
// Large128 (64..191 rows per group, where a 256-row tile would be about half
// padding): 128 tokens x 128 (gated) or 256 columns, 8 waves of 32 tokens, a
// 3-deep ring of 64-deep, 48 KB stages, one workgroup per CU, reading the
// next stage's fragments during the current MFMAs, so that all three stages
// are in flight (measured against 32-deep stages with two workgroups per CU:
// the DeepSeek-V3-shaped layer at 4096 tokens 8.6 % faster, the
// Mixtral-shaped one at 512 tokens 3 %).
using GateUpLarge = TileCfg<256, 128, 32, 4, 2, 4, true, false, 1, 16, true>;
using GateUpLarge128 = TileCfg<128, 128, 64, 4, 2, 3, true, true, 2>;
using DownLarge128 = TileCfg<128, 256, 64, 4, 2, 3, false, true, 2>;
using GateUpSmall = TileCfg<16, 64, 64, 1, 2, 4, true, true>;
using GateUpMid = TileCfg<32, 64, 64, 1, 2, 3, true, true>;
using DownLarge = TileCfg<256, 256, 32, 4, 2, 4, false, false, 1, 16, true>;
using DownSmall = TileCfg<32, 64, 64, 1, 4, 4, false, true>;
// Row-major weights at decode sizes. A stage of a row-major tile reads 128
// contiguous bytes of each weight row per 64 columns, and consecutive rows
// lie a whole matrix width apart, so a wider tile reads longer runs of every
// row: 32 rows x 128 or 256 columns (gate/up) and 32 x 128 (down) instead of
// 16 x 64 and 32 x 64 (Mixtral-shaped layer at T = 32 on row-major weights:
// gate/up 393 -> 342 us at 128 columns and 316 us at 256, down 198 ->
// 169 us). Wider tiles make fewer items, so the widest is taken whose
// expected items still fill the chip (rowmajor_decode_width).
using GateUpSmallRM128 = TileCfg<32, 128, 64, 1, 4, 3, true, true>;
using GateUpSmallRM256 = TileCfg<32, 256, 32, 1, 2, 3, true, true>;
using DownSmallRM = TileCfg<32, 128, 64, 1, 4, 4, false, true>;

// Column width (64, 128 or 256) of the decode-size tile on row-major
// weights: 256 when the expected items fill 1.5 per CU, else 128 when they
// fill half of the CUs (at the Mixtral-shaped T = 1, two experts' 224 items
// of 128 columns still beat 448 of 64: gate/up 104 -> 91 us, but 112 items
// of 256 columns took 112 us), else 64. A group of G with R routed rows
// touches G (1 - (1 - 1/G)^R) groups on average.
inline int rowmajor_decode_width(const GemmProblem& p, int max_width) {
  double items128 = 0, items256 = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    const double g = S.ngroups > 0 ? S.ngroups : 1;
    const double touched = g > 1 ? g * (1.0 - std::pow(1.0 - 1.0 / g, S.rows)) : 1.0;
    const double tiles = (touched + S.rows / 32) * (S.ksplit > 0 ? S.ksplit : 1);
    items128 += tiles * ((S.N + 127) / 128);
    items256 += tiles * ((S.N + 255) / 256);
  }
  const double cus = device_cu_count();
  if (max_width >= 256 && items256 >= 1.5 * cus) return 256;
  if (items128 >= 0.5 * cus) return 128;
  return 64;
}
// FP8 weights: the same tile shapes with half the weight bytes per stage,
// hence deeper rings in about the same LDS. The 128- and 256-row tiles run
// the ping-pong schedule with 32-deep stages and widen each stage's codes
// once into a bf16 tile (5-deep rings: two steps of look-ahead); against
// per-wave widening on the prefetching 128-row ring this made the
// DeepSeek-V3-shaped layer at 4096 tokens 10 % faster (the bf16 128-row
// tile measured no gain from ping-pong).
using GateUpLarge8 = TileCfg<256, 128, 32, 4, 2, 5, true, false, 1, 8, true>;
using GateUpLarge128_8 = TileCfg<128, 128, 32, 4, 2, 5, true, false, 1, 8, true>;
using DownLarge128_8 = TileCfg<128, 256, 32, 4, 2, 5, false, false, 1, 8, true>;
using GateUpSmall8 = TileCfg<16, 64, 64, 1, 2, 4, true, true, 1, 8>;
using GateUpMid8 = TileCfg<32, 64, 64, 1, 2, 4, true, true, 1, 8>;
using DownLarge8 = TileCfg<256, 256, 32, 4, 2, 5, false, false, 1, 8, true>;
using DownSmall8 = TileCfg<32, 64, 64, 1, 4, 4, false, true, 1, 8>;
// MXFP4 weights: a quarter of the bf16 weight bytes per stage plus the
// scale bytes, 64-deep stages wherever a 32-deep one would not give every
// wave a whole number of 1 KB DMA instructions. The decode tiles widen every
// weight fragment with VALU work, so they run as many waves per SIMD as
// their LDS allows: the gate/up tiles' 4-stage rings (27 and 35 KB a
// workgroup of two waves) fit five and four workgroups per CU (2-3 and 2
// waves per SIMD), the down tile's (19 KB) eight (4 waves per SIMD). Their
// registers are bounded for four waves per SIMD all the same (so that the
// register file is never the limit; the compiler reports the LDS-bound
// occupancy below that target): bounding the gate/up tiles for the two
// waves their LDS allows let them take 160-200 registers and measured no
// faster (DeepSeek-V3-shaped T = 128 gate/up 0.61 -> 0.62 ms, Mixtral-
// shaped T = 128 layer 0.323 -> 0.327 ms). With 8-stage rings and one wave
// per SIMD the Mixtral-shaped layer at 32 tokens took 17 % longer. The down tile has 16 rows (half the
// activation bytes of a 32-row one at decode; the K-split plan, made for
// 32-row tiles, stays valid for any tile). The 128-row tiles keep
// one fragment set (prefetching fragments of 64-deep stages spill) and read
// each weight fragment just before its MFMAs; they also serve the 256-row
// class (a 256-row tile with 64-deep stages spills even so; the down
// projection's K-split plan is valid for any tile, only tuned for another).
using GateUpSmall4 = TileCfg<16, 64, 64, 1, 2, 4, true, true, 4, 4>;
// At up to 4 rows per group (the stream is almost all weight codes), a
// 32 x 128 gate/up tile on 4 waves, twice the codes per stage: same box,
// A/B, Mixtral-shaped T = 1 0.090 -> 0.084 ms (gate/up 52 -> 47 us),
// DeepSeek-V3-shaped T = 128 1.02 -> 1.00 ms, Qwen2-shaped T = 16 0.083 ->
// 0.081 ms; at 8 rows per group (Mixtral-shaped T = 32) it was slower
// (0.210 -> 0.219 ms), which keeps the 16 x 64 tile.
using GateUpSmall4W = TileCfg<32, 128, 64, 1, 4, 4, true, true, 4, 4>;
using GateUpMid4 = TileCfg<32, 64, 64, 1, 2, 4, true, true, 4, 4>;
using DownSmall4 = TileCfg<16, 64, 64, 1, 2, 4, false, true, 4, 4>;
// ... and the fused layer's down projection (fp32 K-slices) likewise:
// Qwen2-shaped T = 16 0.081 -> 0.079 ms, DeepSeek-V3-shaped T = 128 1.028 ->
// 1.013 ms (same box, A/B; the K-split plan, made for 64 columns, holds for
// any width)
using DownSmall4W = TileCfg<32, 128, 64, 1, 4, 4, false, true, 4, 4>;
using GateUpLarge128_4 = TileCfg<128, 128, 64, 4, 2, 4, true, false, 2, 4>;
using DownLarge128_4 = TileCfg<128, 256, 64, 4, 2, 4, false, false, 2, 4>;
// ... and, for the 128- and 256-row classes, FP8's widen-once ping-pong
// schedule on 32-deep stages. 4-bit codes fill a 1 KB DMA instruction per
// wave only with twice the columns: 128 rows x 256 columns (gated, each
// matrix) or 512 columns (down), waves 2 along tokens x 4 along columns
// (the same 64 x 64 per wave, accumulators and fragments as the 256 x 128
// tiles), two widening units per thread. The down tile's 512 columns differ
// from the bf16 tile's 256; the K-split plan (made for 256) is valid for
// any tile.
using GateUpLarge_4W = TileCfg<128, 256, 32, 2, 4, 5, true, false, 1, 4, true>;
using DownLarge_4W = TileCfg<128, 512, 32, 2, 4, 5, false, false, 1, 4, true>;
// MXFP8 weights (E4M3 codes with a scale byte per 32 K-values of a column):
// the fp8 tiles' shapes with the mxfp4 tiles' scale handling. The 128- and
// 256-row tiles widen each 32-deep stage once, as for fp8; a stage's 32
// K-values are one scale block, so the stage carries one scale byte per
// column and matrix (256 bytes behind the operands).
using GateUpSmallM8 = TileCfg<16, 64, 64, 1, 2, 4, true, true, 1, 8, false, true>;
// At up to 4 rows per group, as for mxfp4: a 32 x 128 gate/up tile (4 waves,
// 3-deep ring): Mixtral-shaped T = 1 layer 0.100 -> 0.094 ms, Qwen2-shaped
// T = 16 0.118 -> 0.112 ms (same box, A/B).
using GateUpSmallM8W = TileCfg<32, 128, 64, 1, 4, 3, true, true, 1, 8, false, true>;
using GateUpMidM8 = TileCfg<32, 64, 64, 1, 2, 4, true, true, 1, 8, false, true>;
using DownSmallM8 = TileCfg<32, 64, 64, 1, 4, 4, false, true, 1, 8, false, true>;
// ... and its fp32-output down tile likewise (DeepSeek-V3-shaped T = 128
// layer 1.485 -> 1.440 ms, Qwen2-shaped T = 16 0.111 -> 0.107 ms)
using DownSmallM8W = TileCfg<32, 128, 64, 1, 4, 4, false, true, 1, 8, false, true>;
using GateUpLargeM8 = TileCfg<256, 128, 32, 4, 2, 5, true, false, 1, 8, true, true>;
using GateUpLarge128_M8 = TileCfg<128, 128, 32, 4, 2, 5, true, false, 1, 8, true, true>;
using DownLarge128_M8 = TileCfg<128, 256, 32, 4, 2, 5, false, false, 1, 8, true, true>;
using DownLargeM8 = TileCfg<256, 256, 32, 4, 2, 5, false, false, 1, 8, true, true>;
static_assert(DownLarge128_M8::BT == DownLarge128::BT && DownLarge128_M8::BF == DownLarge128::BF &&
                  DownLargeM8::BT == DownLarge::BT && DownLargeM8::BF == DownLarge::BF &&
                  DownSmallM8::BT == DownSmall::BT && DownSmallM8::BF == DownSmall::BF,
              "mxfp8 tiles share the bf16 tiles' shapes (the split-K plan and tile classes)");
static_assert(DownLarge128_4::BT == DownLarge128::BT &&
                  DownLarge128_4::BF == DownLarge128::BF && DownSmall4::BF == DownSmall::BF,
              "mxfp4 tiles share the bf16 tiles' shapes (the split-K plan and tile classes)");
static_assert(DownLarge8::BT == DownLarge::BT && DownLarge8::BF == DownLarge::BF &&
                  DownLarge128_8::BT == DownLarge128::BT &&
                  DownLarge128_8::BF == DownLarge128::BF && DownSmall8::BT == DownSmall::BT &&
                  DownSmall8::BF == DownSmall::BF,
              "fp8 tiles share the bf16 tiles' shapes (the split-K plan and tile classes)");

int device_cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Resident workgroups per CU for a launch with `dyn` bytes of dynamic LDS.
template <class C, typename OutT, bool KTAIL, bool PACKED, bool TRANSW>
int blocks_per_cu(size_t dyn) {
  static int cached_n[64] = {0};
  static size_t cached_dyn[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached_n[dev] == 0 || cached_dyn[dev] != dyn) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(grouped_gemm_kernel<C, OutT, KTAIL, PACKED, TRANSW>),
            C::kThreads, dyn) != hipSuccess || n <= 0)
      n = 1;
    cached_n[dev] = n;
    cached_dyn[dev] = dyn;
  }
  return cached_n[dev];
}

// The most groups whose item table (dynamic LDS: 12 bytes a group, 8 more)
// fits beside a tile's static LDS (its ring stages and widened tiles, each
// array aligned to 1 KB, plus 1 KB for the rest) in the CU's 160 KB.
template <class C>
constexpr int max_groups_in_lds() {
  constexpr int up = (C::STAGE_BYTES + 1023) / 1024 * 1024;
  constexpr int wide = C::WIDEN ? 2 * ((C::WW_BYTES + 1023) / 1024 * 1024) : 0;
  return (160 * 1024 - C::STAGES * up - wide - 1024 - 8) / 12;
}

template <class C>
int64_t item_bound(const GemmProblem& p) {
  // upper bound on items: every group may leave one partial M-tile
  int64_t bound = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    const int64_t mt = (S.rows + C::BT - 1) / C::BT + (S.offsets ? S.ngroups : 0);
    bound += mt * ((S.N + C::BF - 1) / C::BF) * S.ksplit;
  }
  return bound;
}

template <class C, typename OutT, bool KTAIL, bool PACKED, bool TRANSW = false>
hipError_t launch_tail(const GemmProblem& p, int64_t bound, hipStream_t stream) {
  int groups = 0;
  for (int s = 0; s < p.nseg; ++s) groups += p.seg[s].ngroups;
  const size_t dyn = static_cast<size_t>((groups + 2) & ~1) * sizeof(int) +
                    static_cast<size_t>(groups) * sizeof(int2);
  int64_t grid =
      static_cast<int64_t>(device_cu_count()) * blocks_per_cu<C, OutT, KTAIL, PACKED, TRANSW>(dyn);
  if (bound < grid) grid = bound;
  grid = (grid + 7) / 8 * 8;
  MOE_TRACE_LAUNCH("grouped_gemm_kernel", dim3(static_cast<unsigned>(grid)), dim3(C::kThreads),
                   dyn,
                   "tile=%dx%dx%d stages=%d schedule=%s wbits=%d%s gated=%d out=%s ktail=%d "
                   "layout=%d segments=%d groups=%d items<=%lld ksplit=%d combine=%d",
                   C::BT, C::BF, C::BK, C::STAGES,
                   C::PP ? (C::WIDEN ? "pingpong-widen" : "pingpong")
                         : (C::PREFETCH ? "ring-prefetch" : "ring"),
                   C::WBITS, C::MX ? "+mx" : "", C::GATED ? 1 : 0,
                   sizeof(OutT) == 4 ? "f32" : "bf16", KTAIL ? 1 : 0,
                   TRANSW ? kWeightsTransposed : p.seg[0].packed, p.nseg, groups,
                   static_cast<long long>(bound), p.seg[0].ksplit, p.scat.cnt ? 1 : 0);
  hipLaunchKernelGGL((grouped_gemm_kernel<C, OutT, KTAIL, PACKED, TRANSW>),
                     dim3(static_cast<unsigned>(grid)), dim3(C::kThreads), dyn, stream, p);
  return hipGetLastError();
}

template <class C, typename OutT>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  const int64_t bound = item_bound<C>(p);
  if (bound <= 0) return hipSuccess;
  bool ktail = false;
  for (int s = 0; s < p.nseg; ++s) ktail = ktail || (p.seg[s].K % C::BK != 0);
  const int layout = p.seg[0].packed;
  for (int s = 1; s < p.nseg; ++s)
    if (p.seg[s].packed != layout) return hipErrorInvalidValue;  // one layout per launch
  if constexpr (C::MX) {
    if (layout != (C::WBITS == 4 ? 3 : 5)) return hipErrorInvalidValue;
    return ktail ? launch_tail<C, OutT, true, true>(p, bound, stream)
                 : launch_tail<C, OutT, false, true>(p, bound, stream);
  } else if constexpr (C::WBITS == 8) {
    if (layout != 2) return hipErrorInvalidValue;
    return ktail ? launch_tail<C, OutT, true, true>(p, bound, stream)
                 : launch_tail<C, OutT, false, true>(p, bound, stream);
  } else {
    if (layout == kWeightsTransposed) {
      if constexpr (!C::GATED)
        return ktail ? launch_tail<C, OutT, true, false, true>(p, bound, stream)
                     : launch_tail<C, OutT, false, false, true>(p, bound, stream);
      return hipErrorInvalidValue;
    }
    if (layout >= 2) return hipErrorInvalidValue;
    if (layout == 1)
      return ktail ? launch_tail<C, OutT, true, true>(p, bound, stream)
                   : launch_tail<C, OutT, false, true>(p, bound, stream);
    return ktail ? launch_tail<C, OutT, true, false>(p, bound, stream)
                 : launch_tail<C, OutT, false, false>(p, bound, stream);
  }
}

}  // namespace

// Tile class by typical rows per group (chosen in grouped_gemm.hip).
enum TileClass { kSmall = 0, kMid = 1, kLarge128 = 2, kLarge = 3 };

// One family of tiles each (grouped_gemm_<family>.hip): bf16 weights
// (row-major, packed or transposed) gated, plain with fp32 output and plain
// with bf16 output; fp8 and mxfp4 codes; the register-streaming gate/up.
hipError_t launch_bf16_gated(const GemmProblem& p, int tc, hipStream_t stream);
hipError_t launch_bf16_plain_f32(const GemmProblem& p, int tc, hipStream_t stream);
hipError_t launch_bf16_plain_bf16(const GemmProblem& p, int tc, hipStream_t stream);
hipError_t launch_fp8(const GemmProblem& p, int tc, hipStream_t stream);
hipError_t launch_mxfp4(const GemmProblem& p, int tc, hipStream_t stream);
hipError_t launch_mxfp8(const GemmProblem& p, int tc, hipStream_t stream);
hipError_t launch_rs(const GemmProblem& p, hipStream_t stream);

}  // namespace moe
