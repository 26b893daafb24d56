// Persistent, block-scheduled grouped GEMM for the MoE expert layer (gfx950).
//
// One launch computes, for every group g (an expert, or the shared expert),
//   out[rows of g] = epilogue( act[rows of g] * W[g] ),
// where W[g] is [K][N] with N contiguous and the epilogue is either a plain
// store (bf16, or fp32 for the fused layer's down projection, whose output
// feeds the combine without a bf16 rounding) or, in the gated form, SwiGLU
// over two weight
// matrices: out = silu(act*W_gate) * (act*W_up). In the gated form the gate
// and up products only ever live in accumulator registers, so the SwiGLU
// input never reaches memory (the dispatch-kernel post (lumeric.app),
// summary paragraph). Grouping many independent GEMMs into one persistent
// launch follows the grouped-GEMM news page (meineki.news); block scheduling
// over variable expert batch sizes follows the Triton MoE page (setupai.cc),
// key points.
//
// Work items and scheduling. An item is one (group, M-tile, N-tile): BT
// activation rows by BF output columns over the whole K. Every item has the
// same cost within a segment, so a static round-robin over a persistent grid
// stays balanced however skewed the expert counts are. Each workgroup
// rebuilds the per-group item prefix from the device-side expert offsets in
// its prologue: there is no host synchronisation. Items are numbered group by
// group, N-tile by N-tile, with the M-tile fastest, and the workgroup ->
// item-slot map gives every XCD a contiguous run of items (workgroups are
// dispatched round-robin over the 8 XCDs), so the M-tiles sharing one weight
// tile run together under one L2.
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
// Data path per K-step: global -> VGPR (16-byte loads, prefetched one step
// ahead) -> LDS in the tensors' own layouts (weights [BK][BF] N-contiguous,
// activations [BT][BK] K-contiguous, rows padded against bank conflicts) ->
// MFMA operands. The weight operand needs K-consecutive values per lane,
// which the N-contiguous layout does not give; gfx950's transposing LDS read
// (ds_read_b64_tr_b16) delivers them directly. MFMA: v_mfma_f32_16x16x32_bf16,
// fp32 accumulation.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxGroups = kMaxExperts + 1;  // routed experts + one shared

typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// Transposing LDS read: within each 16-lane group, lane i receives element
// i%4 of the 8-byte chunks read by lanes 4r + i/4, r = 0..3.
__device__ __forceinline__ short4_t lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

template <int BT_, int BF_, int BK_, int WT_, int WF_, bool GATED_>
struct TileCfg {
  static constexpr int BT = BT_;  // activation rows (tokens) per tile
  static constexpr int BF = BF_;  // output columns per tile
  static constexpr int BK = BK_;  // K per pipeline step
  static constexpr int WT = WT_;  // waves along tokens
  static constexpr int WF = WF_;  // waves along output columns
  static constexpr bool GATED = GATED_;
  static constexpr int kThreads = WT * WF * kWave;
  static constexpr int NMAT = GATED ? 2 : 1;
  static constexpr int TF = BF / WF;  // columns per wave
  static constexpr int TT = BT / WT;  // tokens per wave
  static constexpr int FF = TF / 16;  // MFMA blocks per wave (columns)
  static constexpr int FT = TT / 16;  // MFMA blocks per wave (tokens)
  static constexpr int WP = BF + 16;  // LDS pitch of a weight row (elements)
  static constexpr int XP = BK + 8;   // LDS pitch of an activation row
  static constexpr int W_CHUNKS = NMAT * BK * BF / 8;  // 16-byte chunks
  static constexpr int X_CHUNKS = BT * BK / 8;
  static constexpr int WCPT = (W_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int XCPT = (X_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int LDS_W = NMAT * BK * WP;
  static constexpr int LDS_X = BT * XP;
  static_assert(BF % (16 * WF) == 0 && BT % (16 * WT) == 0, "wave tiling");
  static_assert(BK % 32 == 0, "BK must be a multiple of the MFMA K");
};

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

template <class C, typename OutT>
__global__ __launch_bounds__(C::kThreads) void grouped_gemm_kernel(GemmProblem prob) {
  __shared__ __attribute__((aligned(16))) bf16_t sW[C::LDS_W];
  __shared__ __attribute__((aligned(16))) bf16_t sX[C::LDS_X];
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_wave_total[C::kThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wf = wave % C::WF;
  const int wt = wave / C::WF;
  const int g16 = lane >> 4;   // k-group of the lane in an MFMA operand
  const int i16 = lane & 15;   // row/column of the lane in an MFMA operand

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
      cnt[i] = ((v.M + C::BT - 1) / C::BT) * ((s.N + C::BF - 1) / C::BF);
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

  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8
                                : blockIdx.x;

  for (int item = slot; item < total; item += G) {
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
    const int local = item - s_pref[lo];
    const int mt = local % mtiles;
    const int n0 = (local / mtiles) * C::BF;
    const int row_base = v.r0 + mt * C::BT;
    const int rows_valid = min(C::BT, v.M - mt * C::BT);
    const bf16_t* __restrict__ act = S.act;
    const bf16_t* wmat[C::NMAT];
    wmat[0] = S.w0 + static_cast<int64_t>(v.local) * S.w_stride;
    if (C::GATED) wmat[C::NMAT - 1] = S.w1 + static_cast<int64_t>(v.local) * S.w_stride;

    floatx4 acc[C::NMAT][C::FF][C::FT];
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
      for (int a = 0; a < C::FF; ++a)
#pragma unroll
        for (int b = 0; b < C::FT; ++b) acc[m][a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    uint4 wreg[C::WCPT];
    uint4 xreg[C::XCPT];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < C::WCPT; ++i) {
        const int c = tid + i * C::kThreads;
        wreg[i] = uint4{0u, 0u, 0u, 0u};
        if (c < C::W_CHUNKS) {
          const int mat = c / (C::BK * C::BF / 8);
          const int rem = c - mat * (C::BK * C::BF / 8);
          const int kr = rem / (C::BF / 8);
          const int cc = rem - kr * (C::BF / 8);
          const int kg = k0 + kr, ng = n0 + cc * 8;
          if (kg < K && ng < N)
            wreg[i] = *reinterpret_cast<const uint4*>(
                wmat[mat] + static_cast<int64_t>(kg) * N + ng);
        }
      }
#pragma unroll
      for (int i = 0; i < C::XCPT; ++i) {
        const int c = tid + i * C::kThreads;
        xreg[i] = uint4{0u, 0u, 0u, 0u};
        if (c < C::X_CHUNKS) {
          const int r = c / (C::BK / 8);
          const int cc = c - r * (C::BK / 8);
          const int kg = k0 + cc * 8;
          if (r < rows_valid && kg < K)
            xreg[i] = *reinterpret_cast<const uint4*>(
                act + static_cast<int64_t>(row_base + r) * K + kg);
        }
      }
    };
    auto sstore = [&]() {
#pragma unroll
      for (int i = 0; i < C::WCPT; ++i) {
        const int c = tid + i * C::kThreads;
        if (c < C::W_CHUNKS) {
          const int mat = c / (C::BK * C::BF / 8);
          const int rem = c - mat * (C::BK * C::BF / 8);
          const int kr = rem / (C::BF / 8);
          const int cc = rem - kr * (C::BF / 8);
          *reinterpret_cast<uint4*>(&sW[(mat * C::BK + kr) * C::WP + cc * 8]) = wreg[i];
        }
      }
#pragma unroll
      for (int i = 0; i < C::XCPT; ++i) {
        const int c = tid + i * C::kThreads;
        if (c < C::X_CHUNKS) {
          const int r = c / (C::BK / 8);
          const int cc = c - r * (C::BK / 8);
          *reinterpret_cast<uint4*>(&sX[r * C::XP + cc * 8]) = xreg[i];
        }
      }
    };

    const int nk = (K + C::BK - 1) / C::BK;
    gload(0);
    for (int kt = 0; kt < nk; ++kt) {
      __syncthreads();  // every wave has finished reading the previous step
      sstore();
      __syncthreads();
      if (kt + 1 < nk) gload((kt + 1) * C::BK);  // in flight during the MFMAs
#pragma unroll
      for (int s = 0; s < C::BK / 32; ++s) {
        bf16x8 a[C::NMAT][C::FF];
        bf16x8 b[C::FT];
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
          for (int fi = 0; fi < C::FF; ++fi) {
            const int col = wf * C::TF + fi * 16 + 4 * (i16 & 3);
            const int row = m * C::BK + s * 32 + 8 * g16 + (i16 >> 2);
            const short4_t lo4 = lds_read_tr16(&sW[row * C::WP + col]);
            const short4_t hi4 = lds_read_tr16(&sW[(row + 4) * C::WP + col]);
            typedef short short8_t __attribute__((ext_vector_type(8)));
            const short8_t s8 = {lo4[0], lo4[1], lo4[2], lo4[3],
                                 hi4[0], hi4[1], hi4[2], hi4[3]};
            a[m][fi] = __builtin_bit_cast(bf16x8, s8);
          }
#pragma unroll
        for (int ti = 0; ti < C::FT; ++ti) {
          const int tok = wt * C::TT + ti * 16 + i16;
          b[ti] = *reinterpret_cast<const bf16x8*>(&sX[tok * C::XP + s * 32 + 8 * g16]);
        }
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
          for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
            for (int ti = 0; ti < C::FT; ++ti)
              acc[m][fi][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  a[m][fi], b[ti], acc[m][fi][ti], 0, 0, 0);
      }
    }

    // ---- epilogue: lane holds columns 4*g16..+3 of one token per block ----
    // (bf16 stores round to nearest even; fp32 stores keep the accumulator)
    OutT* __restrict__ out = static_cast<OutT*>(S.out);
#pragma unroll
    for (int fi = 0; fi < C::FF; ++fi)
#pragma unroll
      for (int ti = 0; ti < C::FT; ++ti) {
        const int tok = wt * C::TT + ti * 16 + i16;
        const int f = n0 + wf * C::TF + fi * 16 + 4 * g16;
        if (tok < rows_valid && f < N) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (C::GATED) {
              const float gt = acc[0][fi][ti][r];
              const float up = acc[C::NMAT - 1][fi][ti][r];
              v[r] = gt / (1.0f + __expf(-gt)) * up;
            } else {
              v[r] = acc[0][fi][ti][r];
            }
          }
          store4(out + static_cast<int64_t>(row_base + tok) * N + f, v);
        }
      }
  }
}

// Tile shapes. Large: 128 tokens x 128 columns, 2x2 waves of 64x64.
// Small (decode): 16 tokens x 64 columns, 4 waves of 16 columns each, long
// K steps so each workgroup keeps many weight bytes in flight.
using GateUpLarge = TileCfg<128, 128, 64, 2, 2, true>;
using GateUpSmall = TileCfg<16, 64, 128, 1, 4, true>;
using DownLarge = TileCfg<128, 128, 64, 2, 2, false>;
using DownSmall = TileCfg<16, 64, 256, 1, 4, false>;

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

template <class C, typename OutT>
int blocks_per_cu() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(grouped_gemm_kernel<C, OutT>), C::kThreads, 0) != hipSuccess || n <= 0)
      n = 1;
    cached[dev] = n;
  }
  return cached[dev];
}

template <class C, typename OutT>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  // upper bound on items: every group may leave one partial M-tile
  int64_t bound = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    const int64_t mt = (S.rows + C::BT - 1) / C::BT + (S.offsets ? S.ngroups : 0);
    bound += mt * ((S.N + C::BF - 1) / C::BF);
  }
  if (bound <= 0) return hipSuccess;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * blocks_per_cu<C, OutT>();
  if (bound < grid) grid = bound;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((grouped_gemm_kernel<C, OutT>), dim3(static_cast<unsigned>(grid)),
                     dim3(C::kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
  const bool large = p.rows_hint >= 64;
  if (p.gated)
    return large ? launch_cfg<GateUpLarge, bf16_t>(p, stream)
                 : launch_cfg<GateUpSmall, bf16_t>(p, stream);
  if (p.out_f32)
    return large ? launch_cfg<DownLarge, float>(p, stream)
                 : launch_cfg<DownSmall, float>(p, stream);
  return large ? launch_cfg<DownLarge, bf16_t>(p, stream)
               : launch_cfg<DownSmall, bf16_t>(p, stream);
}

}  // namespace moe
