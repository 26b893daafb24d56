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
// layouts (weights [BK][BF] N-contiguous, activations [BT][BK] K-contiguous)
// with an XOR swizzle of 16-byte chunks chosen on the global side. The
// weight operand needs K-consecutive values per lane, which the N-contiguous
// layout does not give; the transposing LDS read ds_read_b64_tr_b16 delivers
// them. MFMA: v_mfma_f32_16x16x32_bf16, fp32 accumulation.
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxGroups = kMaxExperts + 1;  // routed experts + one shared

typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Transposing LDS read: within each 16-lane group, lane i receives element
// i%4 of the 8-byte chunks read by lanes 4r + i/4, r = 0..3.
__device__ __forceinline__ short4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maximum, i.e. not waited for).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int BT_, int BF_, int BK_, int WT_, int WF_, int STAGES_, bool GATED_,
          bool PREFETCH_>
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
  static constexpr int NW = WT * WF;
  static constexpr int kThreads = NW * kWave;
  static constexpr int NMAT = GATED ? 2 : 1;
  static constexpr int TF = BF / WF;  // columns per wave
  static constexpr int TT = BT / WT;  // tokens per wave
  static constexpr int FF = TF / 16;  // MFMA blocks per wave (columns)
  static constexpr int FT = TT / 16;  // MFMA blocks per wave (tokens)
  static constexpr int W_BYTES = BK * BF * 2;  // one weight matrix per stage
  static constexpr int X_BYTES = BT * BK * 2;
  static constexpr int STAGE_BYTES = NMAT * W_BYTES + X_BYTES;
  static constexpr int INSTR = STAGE_BYTES / 1024;  // 1 KB DMA instructions
  static constexpr int IPW = INSTR / NW;            // per wave per stage
  static constexpr int W_INSTR = NMAT * W_BYTES / 1024;
  static_assert(BF % (16 * WF) == 0 && BT % (16 * WT) == 0, "wave tiling");
  static_assert((BK == 32 || BK % 64 == 0) && BF % 64 == 0, "swizzle geometry");
  static_assert(W_BYTES % 1024 == 0 && X_BYTES % 1024 == 0, "1 KB DMA granules");
  static_assert(INSTR % NW == 0, "equal DMA share per wave");
  static_assert(STAGES == 4, "the pipeline is written for a 4-deep ring");
};

// 16-byte chunk swizzles (chunk index within a row), chosen by measuring
// LDS throughput of each access pattern on gfx950.
// Weights: the 4 rows a 16-lane transpose read touches land in 4 distinct
// chunk pairs (XOR 2*(row%4)), and the row groups 8 apart that other lanes of
// the same instruction read land on the other bank half (XOR 8 for rows of
// >= 256 bytes, XOR 2 for 128-byte rows). Rows r and r+4, read by one lane,
// share the swizzle. Activations: 8 consecutive token rows at the same K
// chunk land in 8 distinct 16-byte bank groups: with rows of >= 128 bytes the
// chunk is XORed with row % 8; with 64-byte rows (BK = 32) two rows share a
// 128-byte window, so row % 2 picks the half and (row / 2) % 4 is XORed in.
template <int BF>
__device__ __forceinline__ int swz_w(int row, int chunk) {
  return chunk ^ ((row & 3) << 1) ^ (((row >> 3) & 1) << (BF >= 128 ? 3 : 1));
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

__device__ __forceinline__ void store4(bf16_t* p, const float v[4]) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
}

template <class C, typename OutT, bool KTAIL>
__global__ __launch_bounds__(C::kThreads) void grouped_gemm_kernel(GemmProblem prob) {
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st3[C::STAGE_BYTES];
  extern __shared__ int s_pref[];  // [groups + 1], sized at launch
  __shared__ int s_wave_total[C::NW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wf = wave % C::WF;
  const int wt = wave / C::WF;
  const int g16 = lane >> 4;   // k-group of the lane in an MFMA operand
  const int i16 = lane & 15;   // row/column of the lane in an MFMA operand
  const int ksplit = prob.ksplit;

  // ---- prologue: item prefix over all groups of both segments ----
  const int NG = prob.seg[0].ngroups + (prob.nseg > 1 ? prob.seg[1].ngroups : 0);
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
      cnt[i] = ((v.M + C::BT - 1) / C::BT) * ((s.N + C::BF - 1) / C::BF) * ksplit;
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

  for (int item = slot; item < total; item += stride) {
    // group owning the item: the largest g with s_pref[g] <= item
    int lo = 0, hi = NG;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= item) lo = mid; else hi = mid;
    }
    const GroupView v = group_view(prob, lo);
    const GemmSegment& S = v.seg ? prob.seg[1] : prob.seg[0];
    const int K = S.K, N = S.N;
    const int mtiles = (v.M + C::BT - 1) / C::BT;
    int local = item - s_pref[lo];
    const int ks = local % ksplit;
    local /= ksplit;
    const int mt = local % mtiles;
    const int n0 = (local / mtiles) * C::BF;
    const int row_base = v.r0 + mt * C::BT;
    const int rows_valid = min(C::BT, v.M - mt * C::BT);
    // K range of this slice: whole stages (the last stage of K may be short)
    const int nk_all = (K + C::BK - 1) / C::BK;
    const int per = (nk_all + ksplit - 1) / ksplit;
    const int kt_begin = ks * per;
    const int nk = min(nk_all, kt_begin + per) - kt_begin;

    // ---- DMA of one K-step into one ring buffer ----
    // Instruction i of this wave fills 16-byte slots 64*j .. 64*j+63 of the
    // stage, j = wave*IPW + i (wave-uniform). The lane's slot is a tile
    // (row, physical chunk); the swizzle gives the logical chunk, hence the
    // global source. Rows and columns are clamped to the valid range: clamped
    // lanes fetch finite in-bounds data whose products only reach masked
    // outputs or the zeroed K-tail rows.
    const bf16_t* const wsrc0 = S.w0 + static_cast<int64_t>(v.local) * S.w_stride;
    const bf16_t* const wsrc1 = C::GATED ? S.w1 + static_cast<int64_t>(v.local) * S.w_stride : wsrc0;
    const bf16_t* const xsrc = S.act;
    constexpr int W_PER_MAT = C::W_BYTES / 1024;   // instructions per weight matrix
    constexpr int RPI_W = 1024 / (C::BF * 2);      // weight rows per instruction
    constexpr int RPI_X = 1024 / (C::BK * 2);      // activation rows per instruction
    auto issue = [&](int kt, char* buf) {
      const int k0 = kt * C::BK;
#pragma unroll
      for (int i = 0; i < C::IPW; ++i) {
        const int j = wave * C::IPW + i;
        const bf16_t* src;
        if (j < C::W_INSTR) {
          const int mat = j / W_PER_MAT;
          const int r = (j - mat * W_PER_MAT) * RPI_W + lane / (C::BF / 8);
          const int col = min(n0 + swz_w<C::BF>(r, lane % (C::BF / 8)) * 8, N - 8);
          src = (mat ? wsrc1 : wsrc0) + static_cast<int64_t>(min(k0 + r, K - 1)) * N + col;
        } else {
          const int r = (j - C::W_INSTR) * RPI_X + lane / (C::BK / 8);
          const int kc = min(k0 + swz_x<C::BK>(r, lane % (C::BK / 8)) * 8, K - 8);
          src = xsrc + static_cast<int64_t>(row_base + min(r, rows_valid - 1)) * K + kc;
        }
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + j * 1024), 16, 0, 0);
      }
    };

    floatx4 acc[C::NMAT][C::FF][C::FT];
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
      for (int a = 0; a < C::FF; ++a)
#pragma unroll
        for (int b = 0; b < C::FT; ++b) acc[m][a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    // MFMA operand fragments of one stage (all its 32-deep substeps)
    struct Frags {
      bf16x8 a[C::BK / 32][C::NMAT][C::FF];
      bf16x8 b[C::BK / 32][C::FT];
    };
    auto load_frags = [&](const char* buf, Frags& F) {
#pragma unroll
      for (int s = 0; s < C::BK / 32; ++s) {
#pragma unroll
        for (int ti = 0; ti < C::FT; ++ti) {
          const int tok = wt * C::TT + ti * 16 + i16;
          const int chunk = swz_x<C::BK>(tok, s * 4 + g16);
          F.b[s][ti] = *reinterpret_cast<const bf16x8*>(buf + C::NMAT * C::W_BYTES +
                                                         tok * (C::BK * 2) + chunk * 16);
        }
#pragma unroll
        for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m) {
            const int row = s * 32 + 8 * g16 + (i16 >> 2);          // k within the stage
            const int col = wf * C::TF + fi * 16 + 4 * (i16 & 3);   // column within the tile
            const int chunk = swz_w<C::BF>(row, col >> 3);           // rows row, row+4 share it
            const char* p = buf + m * C::W_BYTES + row * (C::BF * 2) + chunk * 16 + (col & 7) * 2;
            const short4_t lo4 = lds_read_tr16(p);
            const short4_t hi4 = lds_read_tr16(p + 4 * C::BF * 2);
            typedef short short8_t __attribute__((ext_vector_type(8)));
            const short8_t s8 = {lo4[0], lo4[1], lo4[2], lo4[3],
                                 hi4[0], hi4[1], hi4[2], hi4[3]};
            F.a[s][m][fi] = __builtin_bit_cast(bf16x8, s8);
          }
      }
    };
    auto mfma = [&](const Frags& F) {
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
    };

    // Weight rows past K (only in the last stage of K when K % BK != 0; the
    // KTAIL instantiation) are zeroed once they have landed and before their
    // fragments are read, so the clamped activation columns there contribute
    // exactly 0. The __syncthreads also drains the DMA issued just before;
    // only the tail step pays for it.
    auto zero_k_tail = [&](int kt, char* buf) {
      const int kvalid = K - kt * C::BK;
      if (kvalid >= C::BK) return;
      const int nrow = C::BK - kvalid;
      constexpr int per_row = C::BF * 2 / 16;
      for (int i = tid; i < C::NMAT * nrow * per_row; i += C::kThreads) {
        const int m = i / (nrow * per_row);
        const int rem = i - m * nrow * per_row;
        const int r = kvalid + rem / per_row;
        const int c = rem - (rem / per_row) * per_row;
        *reinterpret_cast<uint4*>(buf + m * C::W_BYTES + r * (C::BF * 2) + c * 16) =
            uint4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    };

    // Pipeline, ring of 4 stages. Refills are issued even past the end of
    // the item's K range (clamped in bounds; their rows are cached), so the
    // number of stages in flight, hence every wait count, is a constant.
    //
    // PREFETCH: step t waits for stage t+1, refills the buffer stage t-1 used
    // with stage t+3, then reads stage t+1's fragments while the MFMAs of
    // stage t (read during step t-1) run.
    // Otherwise: step t waits for stage t, refills the buffer of stage t-1
    // with stage t+3, then reads and multiplies stage t.
    Frags fa, fb;
    auto step_pf = [&](int t, char* next, char* refill, const Frags& cur, Frags& nxt) {
      wait_vmcnt<C::IPW>();
      __builtin_amdgcn_s_barrier();
      issue(kt_begin + t + 3, refill);
      if (KTAIL && kt_begin + t + 1 == nk_all - 1) zero_k_tail(kt_begin + t + 1, next);
      load_frags(next, nxt);
      mfma(cur);
    };
    // Without prefetch, the gated kernel interleaves the weight-fragment
    // reads column block by column block with the MFMAs that use them; the
    // plain kernel reads all fragments first (each order measured faster for
    // its kernel).
    auto compute_interleaved = [&](const char* buf) {
#pragma unroll
      for (int s = 0; s < C::BK / 32; ++s) {
        bf16x8 b[C::FT];
#pragma unroll
        for (int ti = 0; ti < C::FT; ++ti) {
          const int tok = wt * C::TT + ti * 16 + i16;
          const int chunk = swz_x<C::BK>(tok, s * 4 + g16);
          b[ti] = *reinterpret_cast<const bf16x8*>(buf + C::NMAT * C::W_BYTES +
                                                    tok * (C::BK * 2) + chunk * 16);
        }
#pragma unroll
        for (int fi = 0; fi < C::FF; ++fi) {
          bf16x8 a[C::NMAT];
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m) {
            const int row = s * 32 + 8 * g16 + (i16 >> 2);
            const int col = wf * C::TF + fi * 16 + 4 * (i16 & 3);
            const int chunk = swz_w<C::BF>(row, col >> 3);
            const char* p = buf + m * C::W_BYTES + row * (C::BF * 2) + chunk * 16 + (col & 7) * 2;
            const short4_t lo4 = lds_read_tr16(p);
            const short4_t hi4 = lds_read_tr16(p + 4 * C::BF * 2);
            typedef short short8_t __attribute__((ext_vector_type(8)));
            const short8_t s8 = {lo4[0], lo4[1], lo4[2], lo4[3],
                                 hi4[0], hi4[1], hi4[2], hi4[3]};
            a[m] = __builtin_bit_cast(bf16x8, s8);
          }
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int ti = 0; ti < C::FT; ++ti)
              acc[m][fi][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  a[m], b[ti], acc[m][fi][ti], 0, 0, 0);
        }
      }
    };
    auto step_np = [&](int t, char* cur, char* refill) {
      wait_vmcnt<2 * C::IPW>();
      __builtin_amdgcn_s_barrier();
      issue(kt_begin + t + 3, refill);
      if (KTAIL && kt_begin + t == nk_all - 1) zero_k_tail(kt_begin + t, cur);
      if (C::GATED) {
        compute_interleaved(cur);
      } else {
        load_frags(cur, fa);
        mfma(fa);
      }
    };

    wait_vmcnt<0>();               // every DMA into the ring has landed and
    __builtin_amdgcn_s_barrier();  // every wave is done with the last item
    issue(kt_begin + 0, st0);
    issue(kt_begin + 1, st1);
    issue(kt_begin + 2, st2);
    if (C::PREFETCH) {
      wait_vmcnt<2 * C::IPW>();
      __builtin_amdgcn_s_barrier();  // stage 0 has landed
      if (KTAIL && kt_begin == nk_all - 1) zero_k_tail(kt_begin, st0);
      load_frags(st0, fa);
    }
    // whole turns of the ring, then the remaining steps (no early exits
    // inside the loop: they would keep the accumulators from being updated
    // in place and double their registers)
    {
      const int full = nk / 4;
      int t = 0;
      for (int it = 0; it < full; ++it, t += 4) {
        if (C::PREFETCH) {
          step_pf(t, st1, st3, fa, fb);
          step_pf(t + 1, st2, st0, fb, fa);
          step_pf(t + 2, st3, st1, fa, fb);
          step_pf(t + 3, st0, st2, fb, fa);
        } else {
          step_np(t, st0, st3);
          step_np(t + 1, st1, st0);
          step_np(t + 2, st2, st1);
          step_np(t + 3, st3, st2);
        }
      }
      const int rem = nk - t;
      if (C::PREFETCH) {
        if (rem > 0) step_pf(t, st1, st3, fa, fb);
        if (rem > 1) step_pf(t + 1, st2, st0, fb, fa);
        if (rem > 2) step_pf(t + 2, st3, st1, fa, fb);
      } else {
        if (rem > 0) step_np(t, st0, st3);
        if (rem > 1) step_np(t + 1, st1, st0);
        if (rem > 2) step_np(t + 2, st2, st1);
      }
    }

    // ---- epilogue: lane holds columns 4*g16..+3 of one token per block ----
    // (bf16 stores round to nearest even; fp32 stores keep the accumulator)
    OutT* __restrict__ out =
        static_cast<OutT*>(S.out) + static_cast<int64_t>(ks) * S.slice_stride;
#pragma unroll
    for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
      for (int ti = 0; ti < C::FT; ++ti) {
        const int tok = wt * C::TT + ti * 16 + i16;
        const int f = n0 + wf * C::TF + fi * 16 + 4 * g16;
        if (tok < rows_valid && f < N) {
          float vals[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (C::GATED) {
              const float gt = acc[0][fi][ti][r];
              const float up = acc[C::NMAT - 1][fi][ti][r];
              vals[r] = gt / (1.0f + __expf(-gt)) * up;
            } else {
              vals[r] = acc[0][fi][ti][r];
            }
          }
          store4(out + static_cast<int64_t>(row_base + tok) * N + f, vals);
        }
      }
  }
  // no LDS DMA may land after the workgroup ends (its LDS may be reassigned)
  wait_vmcnt<0>();
}

// Tile shapes (BT tokens x BF columns, BK per stage, waves, ring depth).
// Large batch: 256 tokens x 128 columns (gated: 128 columns each of gate and
// up; down: 256 columns), 8 waves (2 per SIMD) as 4 along tokens x 2 along
// columns, 128 accumulators per lane, a 4-deep ring of 32-deep, 32 KB stages
// (three stages of look-ahead).
// Small batch (decode): gate/up 16 tokens x 64 columns on 2 waves with a
// 4-deep ring of 18 KB stages (2 workgroups and ~108 KB of weights in flight
// per CU); down 32 tokens x 64 columns on 4 waves, 4-deep ring of 12 KB
// stages (3 workgroups per CU); both read the next stage's fragments while
// the current stage's MFMAs run (the large tiles have no registers to spare
// for a second fragment set). Mid (gate/up at 16..63 rows per group):
// 32 tokens x 64 columns, 2 waves, 4-deep ring of 10 KB, 32-deep stages
// (3 workgroups per CU): half the row tiles per expert of the small tile.
using GateUpLarge = TileCfg<256, 128, 32, 4, 2, 4, true, false>;
using GateUpSmall = TileCfg<16, 64, 64, 1, 2, 4, true, true>;
using GateUpMid = TileCfg<32, 64, 32, 1, 2, 4, true, true>;
using DownLarge = TileCfg<256, 256, 32, 4, 2, 4, false, false>;
using DownSmall = TileCfg<32, 64, 64, 1, 4, 4, false, true>;

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
template <class C, typename OutT, bool KTAIL>
int blocks_per_cu(size_t dyn) {
  static int cached_n[64] = {0};
  static size_t cached_dyn[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached_n[dev] == 0 || cached_dyn[dev] != dyn) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(grouped_gemm_kernel<C, OutT, KTAIL>), C::kThreads,
            dyn) != hipSuccess || n <= 0)
      n = 1;
    cached_n[dev] = n;
    cached_dyn[dev] = dyn;
  }
  return cached_n[dev];
}

template <class C>
int64_t item_bound(const GemmProblem& p) {
  // upper bound on items: every group may leave one partial M-tile
  int64_t bound = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    const int64_t mt = (S.rows + C::BT - 1) / C::BT + (S.offsets ? S.ngroups : 0);
    bound += mt * ((S.N + C::BF - 1) / C::BF) * p.ksplit;
  }
  return bound;
}

template <class C, typename OutT, bool KTAIL>
hipError_t launch_tail(const GemmProblem& p, int64_t bound, hipStream_t stream) {
  int groups = 0;
  for (int s = 0; s < p.nseg; ++s) groups += p.seg[s].ngroups;
  const size_t dyn = static_cast<size_t>(groups + 1) * sizeof(int);
  int64_t grid = static_cast<int64_t>(device_cu_count()) * blocks_per_cu<C, OutT, KTAIL>(dyn);
  if (bound < grid) grid = bound;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((grouped_gemm_kernel<C, OutT, KTAIL>), dim3(static_cast<unsigned>(grid)),
                     dim3(C::kThreads), dyn, stream, p);
  return hipGetLastError();
}

template <class C, typename OutT>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  const int64_t bound = item_bound<C>(p);
  if (bound <= 0) return hipSuccess;
  bool ktail = false;
  for (int s = 0; s < p.nseg; ++s) ktail = ktail || (p.seg[s].K % C::BK != 0);
  return ktail ? launch_tail<C, OutT, true>(p, bound, stream)
               : launch_tail<C, OutT, false>(p, bound, stream);
}

}  // namespace

// Tile shape by typical rows per group: fewer than 64 -> small, else large.
// MOE_TILE=small|large overrides the choice (for tile sweeps).
// Tile class by typical rows per group: < 16 small, < 64 mid (gate/up only;
// the down projection keeps the small tile), else large. MOE_TILE=small|mid|
// large overrides the choice (for tile sweeps).
enum TileClass { kSmall = 0, kMid = 1, kLarge = 2 };

int tile_class(const GemmProblem& p) {
  static int forced = -2;
  if (forced == -2) {
    const char* e = getenv("MOE_TILE");
    forced = !e ? -1 : (!strcmp(e, "small") ? kSmall : !strcmp(e, "mid") ? kMid
                        : !strcmp(e, "large") ? kLarge : -1);
  }
  if (forced >= 0) return forced;
  return p.rows_hint < 16 ? kSmall : (p.rows_hint < 64 ? kMid : kLarge);
}

bool grouped_gemm_uses_large_tiles(const GemmProblem& p) { return tile_class(p) == kLarge; }

int grouped_gemm_ksplit_hint(const GemmProblem& p, int cus) {
  // Split K only where the unsplit item count cannot fill the chip: down
  // projections (fp32 partial outputs) with few touched experts or few
  // row tiles.
  if (p.gated || !p.out_f32) return 1;
  const bool large = grouped_gemm_uses_large_tiles(p);
  const int BT = large ? DownLarge::BT : DownSmall::BT;
  const int BF = large ? DownLarge::BF : DownSmall::BF;
  const int BK = large ? DownLarge::BK : DownSmall::BK;
  int64_t items = 0;
  int min_k = 1 << 30;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    // expected row tiles: one partial tile per touched group plus full ones
    const int64_t touched = S.ngroups > 1 ? (S.rows < S.ngroups ? S.rows : S.ngroups) : 1;
    const int64_t mt = touched + S.rows / BT;
    items += mt * ((S.N + BF - 1) / BF);
    min_k = S.K < min_k ? S.K : min_k;
  }
  const int64_t want = 2 * static_cast<int64_t>(cus);
  int split = 1;
  while (split < kMaxKSplit && items * split * 2 <= want && min_k / (split * 2) >= 256 &&
         min_k / (split * 2) >= 4 * BK)
    split *= 2;
  return split;
}

int grouped_gemm_device_cus() { return device_cu_count(); }

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
  const int tc = tile_class(p);
  const bool large = tc == kLarge;
  if (p.gated)
    return large ? launch_cfg<GateUpLarge, bf16_t>(p, stream)
                 : tc == kMid ? launch_cfg<GateUpMid, bf16_t>(p, stream)
                              : launch_cfg<GateUpSmall, bf16_t>(p, stream);
  if (p.out_f32)
    return large ? launch_cfg<DownLarge, float>(p, stream)
                 : launch_cfg<DownSmall, float>(p, stream);
  return large ? launch_cfg<DownLarge, bf16_t>(p, stream)
               : launch_cfg<DownSmall, bf16_t>(p, stream);
}

}  // namespace moe
