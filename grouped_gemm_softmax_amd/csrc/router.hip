// Router GEMM fused with the routing step: the router logits
//   logits[t,e] = sum_h x[t,h] * w_router[e,h]
// (bf16 products, exact in fp32, summed in fp32) are computed here and
// ranked without a round trip of the logits through HBM when one block holds
// all of a token's experts. The routing on them is the library's S1 (top-k,
// ties to the lower expert index, softmax over the k chosen logits).
// Routing inside the kernel with no host round trip follows the Triton MoE
// page (setupai.cc), technical deep-dive; the router projection itself is not
// on the pages (it is the step upstream of the routing they describe).
//
// router_gemm_kernel<NB, NT>: a block owns 16*NT tokens x 16*NB experts over
// one K-slice of H. Its 4 waves split the slice by 64-wide K chunks (wave w
// takes chunks w, w+4, ...), so each wave reads whole 128-byte lines of the x
// and w rows and no operand is read twice inside the block. Experts fill the
// 16-wide MFMA M side and tokens the N side of v_mfma_f32_16x16x32_bf16; both
// operands come straight from global memory (x and w rows are K-contiguous:
// a lane's 8 consecutive K values are one 16-byte load). The 4 waves' tiles
// are then added in LDS in wave order. With one K-slice and one expert block
// the block ranks its tokens' experts at once; otherwise it writes its fp32
// tile to part[s][t][e] and router_finalize_kernel adds the slices in slice
// order and ranks. The result does not depend on timing.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterWaves = kRouterThreads / kWave;
constexpr int kRouterChunk = 64;  // K values per wave step (two MFMA K steps)

// A token's k best experts, one token per lane: 64-bit keys (the logit's
// order-preserving image above ~expert) pushed through a sorted list of KM
// slots (KM = the power of two >= k), so ties go to the lower expert and the
// list is exact whatever the push order.
template <int KM>
struct TopK {
  uint64_t key[KM];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int j = 0; j < KM; ++j) key[j] = 0;
  }
  __device__ __forceinline__ void push(uint64_t v) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const bool gt = v > key[j];
      const uint64_t hi = gt ? v : key[j];
      v = gt ? key[j] : v;
      key[j] = hi;
    }
  }
  // ids and softmax weights of the first k slots. The routing kernel sums
  // the k exponentials with a butterfly over a lane group (lanes past k add
  // exact zeros), which is the pairwise tree below with stride KM/2 first;
  // with its max subtraction, expf and division the weights are bit-equal.
  __device__ __forceinline__ void write(int k, int64_t t, int32_t* topk_ids,
                                        float* topk_w) const {
    float ex[KM];
    const float m = key_to_float(static_cast<uint32_t>(key[0] >> 32));
#pragma unroll
    for (int j = 0; j < KM; ++j)
      ex[j] = j < k ? expf(key_to_float(static_cast<uint32_t>(key[j] >> 32)) - m) : 0.f;
    float sum[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) sum[j] = ex[j];
#pragma unroll
    for (int st = KM / 2; st >= 1; st /= 2)
#pragma unroll
      for (int j = 0; j < st; ++j) sum[j] += sum[j + st];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) {
        topk_ids[t * k + j] = static_cast<int>(0xffffffffu - static_cast<uint32_t>(key[j]));
        topk_w[t * k + j] = ex[j] / sum[0];
      }
  }
};

__device__ __forceinline__ uint64_t make_key(float logit, int e) {
  return (static_cast<uint64_t>(order_key(logit)) << 32) |
         static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(e));
}

template <int NB, int NT>
__global__ __launch_bounds__(kRouterThreads) void router_gemm_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int H, int E, int k,
    int kslice /* K values per slice, a multiple of kRouterChunk */, bool rank,
    float* __restrict__ logits_out, float* __restrict__ part,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  constexpr int BT = 16 * NT;  // tokens of the block
  constexpr int BE = 16 * NB;  // experts of the block
  __shared__ float s_tile[BT][BE + 1];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;
  const int t0 = blockIdx.x * BT;
  const int e0 = blockIdx.y * BE;
  const int s = blockIdx.z;
  const int kb0 = s * kslice;
  const int kb1 = min(H, kb0 + kslice);

  const bf16_t* xrow[NT];
  bool t_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = t0 + 16 * nt + i16;
    t_ok[nt] = t < T;
    xrow[nt] = x + static_cast<int64_t>(t_ok[nt] ? t : 0) * H;
  }
  const bf16_t* wrow[NB];
  bool e_ok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = e0 + 16 * nb + i16;
    e_ok[nb] = e < E;
    wrow[nb] = w + static_cast<int64_t>(e_ok[nb] ? e : 0) * H;
  }
  floatx4 acc[NB][NT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nb][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- this wave's chunks of the slice, two register buffers (up to 32 x 64
  // tiles): the loads of the next chunk are in flight while the current one
  // is multiplied.
  // H % 8 == 0, so a lane's 8 values are all in range or all out.
  bf16x8 a[2][2][NB], b[2][2][NT];  // [buffer][K half][tile]
  auto load = [&](int buf, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = kc + 32 * h + 8 * g16;
      const bool k_ok = kk < kb1;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        b[buf][h][nt] = (k_ok && t_ok[nt]) ? *reinterpret_cast<const bf16x8*>(xrow[nt] + kk)
                                           : bf16x8{};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        a[buf][h][nb] = (k_ok && e_ok[nb]) ? *reinterpret_cast<const bf16x8*>(wrow[nb] + kk)
                                           : bf16x8{};
    }
  };
  auto mul = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[buf][h][nb], b[buf][h][nt],
                                                                acc[nb][nt], 0, 0, 0);
  };
  const int nch = (kb1 - kb0 + kRouterChunk - 1) / kRouterChunk;
  auto chunk_k = [&](int j) __attribute__((always_inline)) { return kb0 + j * kRouterChunk; };
  int j = wave;
  if constexpr (NB * NT <= 8) {
    if (j < nch) load(0, chunk_k(j));
    for (; j < nch; j += 2 * kRouterWaves) {
      const bool more = j + kRouterWaves < nch;
      if (more) load(1, chunk_k(j + kRouterWaves));
      mul(0);
      if (!more) break;
      if (j + 2 * kRouterWaves < nch) load(0, chunk_k(j + 2 * kRouterWaves));
      mul(1);
    }
  } else {
    // the 64 x 64 tile: one buffer (its 64 accumulators and 16 loads per
    // lane leave no room for a second at 3 waves per SIMD)
    for (; j < nch; j += kRouterWaves) {
      load(0, chunk_k(j));
      mul(0);
    }
  }

  // ---- the 4 waves' tiles added in wave order; lane holds experts
  // 16nb + 4*g16 + r of token 16nt + i16
  for (int ww = 0; ww < kRouterWaves; ++ww) {
    if (wave == ww) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float& dst = s_tile[16 * nt + i16][16 * nb + 4 * g16 + r];
            dst = ww == 0 ? acc[nb][nt][r] : dst + acc[nb][nt][r];
          }
    }
    __syncthreads();
  }

  if (!rank) {
    // fp32 tile of slice s to part[s][t][e], experts innermost
    float* dst = part + static_cast<int64_t>(s) * T * E;
    for (int i = tid; i < BT * BE; i += kRouterThreads) {
      const int tl = i / BE, el = i % BE;
      const int t = t0 + tl, e = e0 + el;
      if (t < T && e < E) dst[static_cast<int64_t>(t) * E + e] = s_tile[tl][el];
    }
    return;
  }

  // ---- one slice, all experts in the block: rank here, a token per lane of
  // wave 0 (the block's experts are e0 = 0 .. E-1)
  if (wave != 0) return;
  const int t = t0 + lane;
  if (logits_out)
    for (int i = tid; i < BT * BE; i += kWave) {
      const int tl = i / BE, el = i % BE;
      if (t0 + tl < T && el < E) logits_out[static_cast<int64_t>(t0 + tl) * E + el] = s_tile[tl][el];
    }
  if (lane >= BT || t >= T) return;
  auto rank_token = [&](auto top) __attribute__((always_inline)) {
    top.clear();
    for (int e = 0; e < E; ++e) top.push(make_key(s_tile[lane][e], e));
    top.write(k, t, topk_ids, topk_w);
  };
  if (k <= 1) rank_token(TopK<1>{});
  else if (k <= 2) rank_token(TopK<2>{});
  else if (k <= 4) rank_token(TopK<4>{});
  else if (k <= 8) rank_token(TopK<8>{});
  else rank_token(TopK<16>{});
}

// Adds the K-slices of each logit in slice order and ranks the token's
// experts: one wave per token, expert e = lane + 64q for q < NQ (coalesced
// loads; J slices of all NQ experts in flight before they are added). The
// k rounds of a wave-wide maximum over the 64-bit keys give the same list
// as the per-lane lists of the one-slice path, and the softmax below is the
// routing kernel's (butterfly sum over the wave, lanes past k add zeros).
template <int NQ>
__global__ __launch_bounds__(kRouterThreads) void router_finalize_kernel(
    const float* __restrict__ part, int nslices, int T, int E, int k,
    float* __restrict__ logits_out, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouterWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const int64_t slice = static_cast<int64_t>(T) * E;
  const float* p = part + static_cast<int64_t>(t) * E + lane;
  constexpr int J = NQ >= 16 ? 1 : 16 / NQ;
  float v[NQ];
  for (int s0 = 0; s0 < nslices; s0 += J) {
    float tmp[J][NQ];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        tmp[j][q] = (s0 + j < nslices && lane + q * kWave < E)
                        ? p[(s0 + j) * slice + q * kWave]
                        : 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (s0 + j < nslices) v[q] = s0 + j == 0 ? tmp[j][q] : v[q] + tmp[j][q];
  }
  uint64_t key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + q * kWave;
    key[q] = 0;
    if (e < E) {
      if (logits_out) logits_out[static_cast<int64_t>(t) * E + e] = v[q];
      key[q] = make_key(v[q], e);
    }
  }
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) best = key[q] > best ? key[q] : best;
    best = group_max_u64<kWave>(best);
#pragma unroll
    for (int q = 0; q < NQ; ++q) key[q] = (key[q] == best) ? 0 : key[q];
    if (lane == j) mine = best;
  }
  const float lg = key_to_float(static_cast<uint32_t>(mine >> 32));
  const float m = __shfl(lg, 0, kWave);
  const float ex = lane < k ? expf(lg - m) : 0.f;
  const float ssum = group_sum<kWave>(ex);
  if (lane < k) {
    topk_ids[static_cast<int64_t>(t) * k + lane] =
        static_cast<int>(0xffffffffu - static_cast<uint32_t>(mine));
    topk_w[static_cast<int64_t>(t) * k + lane] = ex / ssum;
  }
}

template <int NB, int NT>
void launch_gemm(const RouterPlan& p, const bf16_t* x, const bf16_t* w, int T, int H, int E,
                 int k, float* logits_out, float* part, int32_t* ids, float* tw,
                 hipStream_t stream) {
  const dim3 grid((T + 16 * NT - 1) / (16 * NT), (E + 16 * NB - 1) / (16 * NB), p.nslices);
  MOE_TRACE_LAUNCH("router_gemm_kernel", grid, dim3(kRouterThreads), 0,
                   "tile=%dx%d T=%d H=%d E=%d k=%d kslices=%d fused=%d", 16 * NT, 16 * NB, T, H,
                   E, k, p.nslices, p.fused ? 1 : 0);
  hipLaunchKernelGGL((router_gemm_kernel<NB, NT>), grid, dim3(kRouterThreads), 0, stream, x,
                     w, T, H, E, k, p.kslice, p.fused, logits_out, part, ids, tw);
}

template <int NB>
void launch_gemm_nt(const RouterPlan& p, const bf16_t* x, const bf16_t* w, int T, int H,
                    int E, int k, float* logits_out, float* part, int32_t* ids, float* tw,
                    hipStream_t stream) {
  switch (p.nt) {
    case 1: launch_gemm<NB, 1>(p, x, w, T, H, E, k, logits_out, part, ids, tw, stream); break;
    case 2: launch_gemm<NB, 2>(p, x, w, T, H, E, k, logits_out, part, ids, tw, stream); break;
    default: launch_gemm<NB, 4>(p, x, w, T, H, E, k, logits_out, part, ids, tw, stream); break;
  }
}

}  // namespace

// Tile and K-split of the router GEMM. Tokens and experts per block grow to
// 64 each (a 64 x 64 fp32 tile per wave, which bounds the re-reads of x and
// w at large T). A wave's chunk loop waits on memory at each chunk, so the
// time follows the chunks per wave: while the blocks cannot fill the chip,
// H is cut into slices of at least 4 chunks (one per wave), up to 3 blocks
// per compute unit (the 64 x 64 tile's occupancy). When all experts fit one
// block and the tiles alone give a block per compute unit, one slice is
// kept: the ranking then happens in the GEMM kernel and the second launch
// and its fp32 round trip go away.
RouterPlan router_plan(int T, int H, int E, int cus) {
  RouterPlan p;
  p.nb = E <= 16 ? 1 : E <= 32 ? 2 : 4;
  p.nt = T <= 16 ? 1 : T <= 32 ? 2 : 4;
  const int tiles = ((T + 16 * p.nt - 1) / (16 * p.nt)) * ((E + 16 * p.nb - 1) / (16 * p.nb));
  const int chunks = (H + kRouterChunk - 1) / kRouterChunk;
  const int max_slices = (chunks + kRouterWaves - 1) / kRouterWaves;
  int S = (3 * cus + tiles - 1) / tiles;
  if (E <= 16 * p.nb && tiles >= cus) S = 1;
  S = S < 1 ? 1 : S > max_slices ? max_slices : S;
  // slice width in whole chunks, then the slices that width needs
  const int per = (chunks + S - 1) / S;
  p.kslice = per * kRouterChunk;
  p.nslices = (chunks + per - 1) / per;
  p.fused = p.nslices == 1 && E <= 16 * p.nb;
  return p;
}

size_t router_part_elems(const RouterPlan& p, int T, int E) {
  if (p.fused) return 0;
  return static_cast<size_t>(p.nslices) * T * E;
}

hipError_t launch_router(const RouterPlan& p, const bf16_t* x, const bf16_t* w, int T, int H,
                         int E, int k, float* logits_out, float* part, int32_t* topk_ids,
                         float* topk_w, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  switch (p.nb) {
    case 1: launch_gemm_nt<1>(p, x, w, T, H, E, k, logits_out, part, topk_ids, topk_w, stream); break;
    case 2: launch_gemm_nt<2>(p, x, w, T, H, E, k, logits_out, part, topk_ids, topk_w, stream); break;
    default: launch_gemm_nt<4>(p, x, w, T, H, E, k, logits_out, part, topk_ids, topk_w, stream); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.fused) return err;
  const dim3 grid2((T + kRouterWaves - 1) / kRouterWaves);
  auto fin = [&](auto kernel) {
    MOE_TRACE_LAUNCH("router_finalize_kernel", grid2, dim3(kRouterThreads), 0,
                     "T=%d E=%d k=%d kslices=%d", T, E, k, p.nslices);
    hipLaunchKernelGGL(kernel, grid2, dim3(kRouterThreads), 0, stream, part, p.nslices, T, E,
                       k, logits_out, topk_ids, topk_w);
  };
  if (E <= 64) fin(router_finalize_kernel<1>);
  else if (E <= 256) fin(router_finalize_kernel<4>);
  else fin(router_finalize_kernel<16>);
  return hipGetLastError();
}

}  // namespace moe
