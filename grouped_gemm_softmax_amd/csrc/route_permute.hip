// Routing and permutation kernels of the MoE expert layer.
//
// route_kernel: a group of L lanes per token (L = next power of two >= E,
// clamped to 8..64). Each lane holds the logits of experts e = lane%L + L*q
// as 64-bit keys (order-preserving integer image of the fp32 logit in the
// high word, ~e in the low word), so k rounds of a group-wide max give the k
// largest logits with equal logits in ascending expert order. Top-k routing inside the kernel, with no host round trip,
// follows the Triton MoE page (setupai.cc), technical deep-dive; the tie rule
// and the softmax over the k chosen logits are this library's definition.
// The same kernel optionally counts, per chunk of tokens, how many
// assignments each expert received (the histogram for the permutation).
//
// permute_kernel: a stable counting sort of the assignments (t, j) by expert.
// Each block owns a few consecutive routing chunks: it derives each expert's
// first free row for each of them from the per-chunk histogram table
// (exclusive scan over experts of the totals, plus the counts of earlier
// chunks), ranks its assignments in (t, j) order within their chunk, writes
// the row maps and copies its tokens' rows of x into x_perm. Per-expert contiguous activations as in the
// DeepGEMM article (itsolotime.com), section 3.1; re-arrangement before the
// grouped GEMM as in the HPC-Ops article (ntfzh.com), FusedMoE paragraph.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRouteThreads = 256;
// The routing kernel's blocks: 16 waves, so that a 32-token chunk of a
// layer with more than 32 experts (one token per wave and pass) takes two
// passes instead of eight (DeepSeek-V3-shaped T = 4096: 35.5 -> 18.8 us,
// Qwen2-shaped T = 16384 23.6 -> 18.6 us, T = 1024 6.3 -> 4.8 us).
constexpr int kRouteBlock = 1024;

// L lanes per token (L = the power of two >= E, at least 8, at most 64), so
// a wave routes 64/L tokens at once; each lane holds the logits of NQ
// experts, lane%L + L*q (NQ = the power of two >= E/L). The next token's
// logits are loaded before the current one is ranked, so at most one load
// latency per pass is exposed.
template <int L, int NQ, int NT>
__device__ void route_tokens(const float* __restrict__ logits, int T, int E, int k,
                             int t_begin, int t_end, int32_t* __restrict__ topk_ids,
                             float* __restrict__ topk_w, int* s_count) {
  constexpr int TPW = kWave / L;          // tokens per wave per pass
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane / L;               // token slot in the wave
  const int gl = lane % L;                // lane within the token group
  const int Q = (E + L - 1) / L;
  const int stride = (NT / kWave) * TPW;
  float cur[NQ];
  auto load = [&](int t, float* dst) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = gl + q * L;
      dst[q] = (t < t_end && q < Q && e < E) ? logits[static_cast<int64_t>(t) * E + e] : 0.f;
    }
  };
  int t = t_begin + wave * TPW + sub;
  load(t, cur);
  for (; t - sub < t_end; t += stride) {
    float nxt[NQ];
    load(t + stride, nxt);
    uint64_t key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = gl + q * L;
      key[q] = 0;  // below every real key: never chosen while k <= E
      if (q < Q && e < E)
        key[q] = (static_cast<uint64_t>(order_key(cur[q])) << 32) |
                 static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(e));
    }
    int my_id = 0;
    float my_logit = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int q = 0; q < NQ; ++q) best = key[q] > best ? key[q] : best;
      best = group_max_u64<L>(best);
#pragma unroll
      for (int q = 0; q < NQ; ++q) key[q] = (key[q] == best) ? 0 : key[q];
      if (gl == j) {
        my_id = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
        my_logit = key_to_float(static_cast<uint32_t>(best >> 32));
      }
    }
    // softmax over the k chosen logits; slot 0 of the group holds the largest
    const float m = __shfl(my_logit, lane - gl, kWave);
    const float ex = (gl < k) ? expf(my_logit - m) : 0.f;
    const float ssum = group_sum<L>(ex);
    if (t < t_end && gl < k) {
      topk_ids[static_cast<int64_t>(t) * k + gl] = my_id;
      topk_w[static_cast<int64_t>(t) * k + gl] = ex / ssum;
      if (s_count) atomicAdd(&s_count[min(max(my_id, 0), E - 1)], 1);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) cur[q] = nxt[q];
  }
}

// Tokens [t_begin, t_end) of an NT-thread block, with the lane group sized to
// E (E <= 64 * MAXQ).
template <int NT, int MAXQ = 16>
__device__ __forceinline__ void route_range(const float* logits, int T, int E, int k,
                                            int t_begin, int t_end, int32_t* ids, float* w,
                                            int* cnt) {
  if (E <= 8) route_tokens<8, 1, NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
  else if (E <= 16) route_tokens<16, 1, NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
  else if (E <= 32) route_tokens<32, 1, NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
  else if (E <= 64) route_tokens<64, 1, NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
  else if (E <= 128) route_tokens<64, 2, NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
  else if (MAXQ <= 4 || E <= 256) route_tokens<64, 4, NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
  else if (MAXQ <= 8 || E <= 512) route_tokens<64, (MAXQ < 8 ? MAXQ : 8), NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
  else route_tokens<64, MAXQ, NT>(logits, T, E, k, t_begin, t_end, ids, w, cnt);
}

__global__ __launch_bounds__(kRouteBlock) void route_kernel(
    const float* __restrict__ logits, int T, int E, int k, int chunk_tokens,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist /* [nchunks][E] or null */) {
  __shared__ int s_count[kMaxExperts];
  if (hist)
    for (int e = threadIdx.x; e < E; e += kRouteBlock) s_count[e] = 0;
  __syncthreads();
  const int t_begin = blockIdx.x * chunk_tokens;
  const int t_end = min(T, t_begin + chunk_tokens);
  route_range<kRouteBlock>(logits, T, E, k, t_begin, t_end, topk_ids, topk_w,
                             hist ? s_count : nullptr);
  if (hist) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouteBlock)
      hist[static_cast<int64_t>(blockIdx.x) * E + e] = s_count[e];
  }
}

// Per-chunk expert histogram from existing ids (moe_permute's first pass).
__global__ __launch_bounds__(kRouteThreads) void hist_kernel(
    const int32_t* __restrict__ topk_ids, int T, int E, int k,
    int chunk_tokens, int32_t* __restrict__ hist) {
  __shared__ int s_count[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) s_count[e] = 0;
  __syncthreads();
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * chunk_tokens * k;
  const int64_t a1 = min(static_cast<int64_t>(T) * k, a0 + static_cast<int64_t>(chunk_tokens) * k);
  for (int64_t a = a0 + threadIdx.x; a < a1; a += kRouteThreads) {
    int e = topk_ids[a];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);  // keep out-of-contract ids in bounds
    atomicAdd(&s_count[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads)
    hist[static_cast<int64_t>(blockIdx.x) * E + e] = s_count[e];
}

constexpr int kPermThreads = 256;

// Zeroes clear[0, nclear) across the whole grid (one int per thread and
// pass): the arrival counters of a down projection that combines in its
// epilogue, cleared by the launch before it in the stream.
__device__ __forceinline__ void clear_range(int32_t* clear, int64_t nclear) {
  if (!clear) return;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * gridDim.y * blockDim.x;
  const int64_t first =
      (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = first; i < nclear; i += nthreads) clear[i] = 0;
}

// One block per group of `cpb` (<= kPermChunks) routing chunks (and per column slice of
// x). Steps:
//  1. One coalesced pass over the [nchunks][E] histogram gives each expert's
//     total (hence, by an exclusive scan over experts, expert_offsets) and the
//     counts of the chunks before this block; then the first free row of
//     every expert for each of the block's routing chunks.
//  2. Each assignment's row: that base plus its stable rank among the
//     assignments of its own routing chunk with the same expert.
//  3. The block copies its column slice of the assigned rows of x.
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ topk_ids, int T,
    int H, int E, int k, int chunk_tokens, int nchunks, int cpb, int slice_cols,
    const int32_t* __restrict__ hist, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_dest,
    bf16_t* __restrict__ x_perm, int32_t* __restrict__ clear, int64_t nclear) {
  __shared__ int s_total[kMaxExperts];
  __shared__ int s_base[kPermChunks][kMaxExperts];
  __shared__ int s_wave_total[kPermThreads / kWave];
  __shared__ int s_ids[kPermChunks * kMaxChunkAssign];
  __shared__ int s_dest[kPermChunks * kMaxChunkAssign];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c0 = blockIdx.x * cpb;                       // first routing chunk
  const int nc = min(cpb, nchunks - c0);                 // routing chunks here
  clear_range(clear, nclear);

  // 1a. totals and counts before this block (integer LDS atomics: exact and
  //     order-independent)
  for (int e = tid; e < E; e += kPermThreads) {
    s_total[e] = 0;
    for (int r = 0; r < kPermChunks; ++r) s_base[r][e] = 0;
  }
  __syncthreads();
  const int ncell = nchunks * E;
  constexpr int U = 8;
  for (int i0 = tid; i0 < ncell; i0 += kPermThreads * U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kPermThreads;
      v[u] = i < ncell ? hist[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kPermThreads;
      if (i < ncell && v[u] != 0) {
        const int c = i / E, e = i - c * E;
        atomicAdd(&s_total[e], v[u]);
        // chunks before the block count into every row of s_base; chunk
        // c0 + r counts into rows r+1 .. nc-1
        if (c < c0) atomicAdd(&s_base[0][e], v[u]);
        else if (c < c0 + nc - 1) atomicAdd(&s_base[c - c0 + 1][e], v[u]);
      }
    }
  }
  __syncthreads();
  // 1b. exclusive scan of the totals over experts (4 experts per thread,
  //     thread-major), then the per-chunk bases
  constexpr int EPT = kMaxExperts / kPermThreads;
  int tot[EPT];
  int my_sum = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid * EPT + i;
    tot[i] = e < E ? s_total[e] : 0;
    my_sum += tot[i];
  }
  const int incl = wave_inclusive_scan(my_sum);
  if (lane == kWave - 1) s_wave_total[wave] = incl;
  __syncthreads();
  int run = incl - my_sum;
  for (int w = 0; w < wave; ++w) run += s_wave_total[w];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid * EPT + i;
    if (e < E) {
      if (blockIdx.x == 0 && blockIdx.y == 0) expert_offsets[e] = run;
      int b = run;
      for (int r = 0; r < nc; ++r) {  // running prefix over the block's chunks
        b += s_base[r][e];
        s_base[r][e] = b;
      }
    }
    run += tot[i];
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) expert_offsets[E] = T * k;

  // 2. stable rank inside each routing chunk, in (t, j) order
  const int t0 = c0 * chunk_tokens;
  const int ntok = min(T - t0, nc * chunk_tokens);
  const int n = ntok * k;
  const int64_t a0 = static_cast<int64_t>(t0) * k;
  const int per_chunk = chunk_tokens * k;
  for (int i = tid; i < n; i += kPermThreads) {
    int e = topk_ids[a0 + i];
    s_ids[i] = e < 0 ? 0 : (e >= E ? E - 1 : e);
  }
  __syncthreads();
  for (int i = tid; i < n; i += kPermThreads) {
    const int e = s_ids[i];
    const int r = i / per_chunk;
    // the earlier assignments of the chunk with the same expert, eight LDS
    // reads in flight at a time (a read-compare loop waits for each read)
    int rank = 0;
    int i2 = r * per_chunk;
    for (; i2 + 8 <= i; i2 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = s_ids[i2 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) rank += (v[u] == e);
    }
    for (; i2 < i; ++i2) rank += (s_ids[i2] == e);
    int p = s_base[r][e] + rank;
    p = p < T * k ? p : T * k - 1;  // in bounds even for out-of-contract ids
    s_dest[i] = p;
    if (blockIdx.y == 0) {
      row_dest[a0 + i] = p;
      row_token[p] = t0 + i / k;
    }
  }
  __syncthreads();

  // 3. copy this block's column slice of each assigned row: x_perm[p] = x[t]
  //    (8 independent 16-byte loads in flight per thread before the stores);
  //    skipped when the consumer gathers the rows of x itself
  if (!x_perm) return;
  const int c_begin = blockIdx.y * slice_cols;
  const int c_end = min(H, c_begin + slice_cols);
  const int vec_per_row = (c_end - c_begin) / 8;  // 16-byte vectors
  const int nvec = n * vec_per_row;
  for (int v0 = tid; v0 < nvec; v0 += kPermThreads * U) {
    uint4 val[U];
    const uint4* src[U];
    uint4* dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // out-of-range slots repeat the last vector (same source, same target)
      const int v = min(v0 + u * kPermThreads, nvec - 1);
      const int i = v / vec_per_row;
      const int c = c_begin + (v - i * vec_per_row) * 8;
      src[u] = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t0 + i / k) * H + c);
      dst[u] = reinterpret_cast<uint4*>(x_perm + static_cast<int64_t>(s_dest[i]) * H + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) val[u] = *src[u];
#pragma unroll
    for (int u = 0; u < U; ++u) *dst[u] = val[u];
  }
}

// Small batches (all T*k <= kMaxChunkAssign / 2 assignments in one routing
// chunk): routing and the permutation in one launch. Every block routes all
// T tokens into LDS (block 0 also writes the routing result, the offsets
// and the row maps), scans the expert counts, ranks the assignments in
// (t, j) order and copies its own column slice of the assigned rows of x.
// 16 waves, so that one pass routes up to 16 tokens (E > 32) to 128 (E <= 8);
// E <= kSmallMaxExperts. The rank of assignment i (its position among the
// earlier assignments of its expert) comes from the wave holding it: the
// lanes with the same expert are found with one ballot per bit of the id,
// the earlier lanes among them counted, and the first wave's per-expert
// counts added for the second (instead of each lane scanning all earlier
// assignments in LDS, up to 127 dependent reads).
constexpr int kSmallThreads = 1024;
constexpr int kSmallMaxExperts = 256;
__global__ __launch_bounds__(kSmallThreads) void route_permute_small_kernel(
    const float* __restrict__ logits, const bf16_t* __restrict__ x, int T, int H, int E,
    int k, int slice_cols, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_dest, bf16_t* __restrict__ x_perm, int32_t* __restrict__ clear,
    int64_t nclear) {
  __shared__ int s_count[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_ids[kMaxChunkAssign];
  __shared__ float s_w[kMaxChunkAssign];
  __shared__ int s_dest[kMaxChunkAssign];
  __shared__ int s_wave_total[kSmallThreads / kWave];
  __shared__ int s_first_wave[kSmallMaxExperts];  // wave 0's assignments per expert
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const bool lead = blockIdx.x == 0;
  const int n = T * k;
  clear_range(clear, nclear);
  for (int e = tid; e < E; e += kSmallThreads) {
    s_count[e] = 0;
    s_first_wave[e] = 0;
  }
  __syncthreads();
  route_range<kSmallThreads, 4>(logits, T, E, k, 0, T, s_ids, s_w, s_count);
  __syncthreads();
  if (lead)
    for (int i = tid; i < n; i += kSmallThreads) {
      topk_ids[i] = s_ids[i];
      topk_w[i] = s_w[i];
    }
  // exclusive scan of the expert counts (one expert per thread)
  constexpr int EPT = kMaxExperts / kSmallThreads;
  int cnt[EPT];
  int my_sum = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid * EPT + i;
    cnt[i] = e < E ? s_count[e] : 0;
    my_sum += cnt[i];
  }
  const int incl = wave_inclusive_scan(my_sum);
  if (lane == kWave - 1) s_wave_total[wave] = incl;
  __syncthreads();
  // (only the waves holding experts: E <= 256 of them, so waves 0-3)
  if (wave * kWave * EPT < E) {
    int run = incl - my_sum;
    for (int w = 0; w < wave; ++w) run += s_wave_total[w];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      if (e < E) {
        s_off[e] = run;
        if (lead) expert_offsets[e] = run;
      }
      run += cnt[i];
    }
  }
  if (lead && tid == 0) expert_offsets[E] = n;
  __syncthreads();
  // stable rank of each assignment among the earlier ones with its expert
  // (n <= 128: the assignments are lanes of waves 0 and 1)
  const bool valid = wave < 2 && tid < n;
  const int e = valid ? min(max(s_ids[tid], 0), E - 1) : 0;
  int rank = 0;
  if (wave < 2) {
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {  // E <= 256: ids have 8 bits
      const bool bit = (e >> b) & 1;
      const uint64_t set = __ballot(valid && bit);
      same &= bit ? set : ~set;
    }
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    rank = __popcll(same & below);
    // the last lane of each expert in wave 0 records the wave's count
    if (wave == 0 && valid && (same >> lane) == 1ull) s_first_wave[e] = rank + 1;
  }
  __syncthreads();
  if (valid) {
    if (wave == 1) rank += s_first_wave[e];
    const int p = min(s_off[e] + rank, n - 1);
    s_dest[tid] = p;
    if (lead) {
      row_dest[tid] = p;
      row_token[p] = tid / k;
    }
  }
  __syncthreads();
  // this block's column slice of every assigned row: x_perm[p] = x[t]
  // (8 independent 16-byte loads in flight per thread before the stores)
  const int c_begin = blockIdx.x * slice_cols;
  const int c_end = min(H, c_begin + slice_cols);
  const int vec_per_row = (c_end - c_begin) / 8;  // 16-byte vectors
  const int nvec = n * vec_per_row;
  constexpr int U = 4;
  for (int v0 = tid; v0 < nvec; v0 += kSmallThreads * U) {
    uint4 val[U];
    int64_t dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // out-of-range slots repeat the last vector (same source, same target)
      const int v = min(v0 + u * kSmallThreads, nvec - 1);
      const int i = v / vec_per_row;
      const int c = c_begin + (v - i * vec_per_row) * 8;
      val[u] = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(i / k) * H + c);
      dst[u] = static_cast<int64_t>(s_dest[i]) * H + c;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) *reinterpret_cast<uint4*>(x_perm + dst[u]) = val[u];
  }
}

}  // namespace

// Measured: one launch wins up to 128 assignments (Mixtral-shaped T = 1 and
// 32, Qwen2-shaped T = 16); at 256 (Mixtral T = 128) the 16 blocks' row copy
// makes it slower than the two kernels.
bool route_permute_fits_one_launch(int T, int E, int k) {
  return static_cast<int64_t>(T) * k <= kMaxChunkAssign / 2 && E <= kSmallMaxExperts;
}

hipError_t launch_route_permute_small(const float* logits, const bf16_t* x, int T, int H,
                                      int E, int k, int32_t* topk_ids, float* topk_w,
                                      int32_t* expert_offsets, int32_t* row_token,
                                      int32_t* row_dest, bf16_t* x_perm, hipStream_t stream,
                                      int32_t* clear, int64_t nclear) {
  if (T <= 0) return hipSuccess;
  const int slice = kPermuteSliceCols;
  const int nslices = (H + slice - 1) / slice;
  MOE_TRACE_LAUNCH("route_permute_small_kernel", dim3(nslices), dim3(kSmallThreads), 0,
                   "T=%d H=%d E=%d k=%d", T, H, E, k);
  hipLaunchKernelGGL(route_permute_small_kernel, dim3(nslices), dim3(kSmallThreads), 0, stream,
                     logits, x, T, H, E, k, slice, topk_ids, topk_w, expert_offsets, row_token,
                     row_dest, x_perm, clear, nclear);
  return hipGetLastError();
}

// Tokens per routing chunk (one histogram row, one routing block): at most
// 32 and kMaxChunkAssign / k; small batches use chunks of down to 4 tokens
// (one pass of a block at one token per wave) so that more blocks share the
// routing and the permutation.
int route_chunk_tokens(int T, int k) {
  int c = kMaxChunkAssign / k;
  c = c < 32 ? c : 32;
  int want = (T + 127) / 128;  // about 128 chunks while T is small
  want = want < 4 ? 4 : want;
  return want < c ? want : c;
}

int route_num_chunks(int T, int k) {
  const int c = route_chunk_tokens(T, k);
  return (T + c - 1) / c;
}

hipError_t launch_route(const float* logits, int T, int E, int k,
                        int32_t* topk_ids, float* topk_w, int32_t* hist,
                        hipStream_t stream) {
  const int chunk = route_chunk_tokens(T, k);
  const int nchunks = route_num_chunks(T, k);
  MOE_TRACE_LAUNCH("route_kernel", dim3(nchunks), dim3(kRouteBlock), 0,
                   "T=%d E=%d k=%d chunk=%d hist=%d", T, E, k, chunk, hist ? 1 : 0);
  hipLaunchKernelGGL(route_kernel, dim3(nchunks), dim3(kRouteBlock), 0,
                     stream, logits, T, E, k, chunk, topk_ids, topk_w, hist);
  return hipGetLastError();
}

hipError_t launch_hist(const int32_t* topk_ids, int T, int E, int k,
                       int32_t* hist, hipStream_t stream) {
  const int chunk = route_chunk_tokens(T, k);
  const int nchunks = route_num_chunks(T, k);
  MOE_TRACE_LAUNCH("hist_kernel", dim3(nchunks), dim3(kRouteThreads), 0, "T=%d E=%d k=%d chunk=%d",
                   T, E, k, chunk);
  hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(kRouteThreads), 0,
                     stream, topk_ids, T, E, k, chunk, hist);
  return hipGetLastError();
}

hipError_t launch_permute(const bf16_t* x, const int32_t* topk_ids, int T,
                          int H, int E, int k, const int32_t* hist,
                          int32_t* expert_offsets, int32_t* row_token,
                          int32_t* row_dest, bf16_t* x_perm,
                          hipStream_t stream, int32_t* clear, int64_t nclear) {
  const int chunk = route_chunk_tokens(T, k);
  const int nchunks = route_num_chunks(T, k);
  const int slice = kPermuteSliceCols;
  const int nslices = x_perm ? (H + slice - 1) / slice : 1;
  // with a row copy, a block amortises its pass over the histogram over
  // kPermChunks chunks; without one (maps only) it takes a single chunk, so
  // that more blocks share the passes
  const int cpb = x_perm ? kPermChunks : 1;
  const int nblocks = (nchunks + cpb - 1) / cpb;
  MOE_TRACE_LAUNCH("permute_kernel", dim3(nblocks, nslices), dim3(kPermThreads), 0,
                   "T=%d H=%d E=%d k=%d chunk=%d copy=%d", T, H, E, k, chunk, x_perm ? 1 : 0);
  hipLaunchKernelGGL(permute_kernel, dim3(nblocks, nslices), dim3(kPermThreads),
                     0, stream, x, topk_ids, T, H, E, k, chunk, nchunks, cpb, slice,
                     hist, expert_offsets, row_token, row_dest, x_perm, clear, nclear);
  return hipGetLastError();
}

}  // namespace moe
