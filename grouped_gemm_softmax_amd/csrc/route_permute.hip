// Routing and permutation kernels of the MoE expert layer.
//
// route_kernel: one wavefront per token. Each lane holds the logits of the
// experts e = lane + 64*q as 64-bit keys (order-preserving integer image of
// the fp32 logit in the high word, ~e in the low word), so k rounds of a
// wave-wide max give the k largest logits with equal logits in ascending
// expert order. Top-k routing inside the kernel, with no host round trip,
// follows the Triton MoE page (setupai.cc), technical deep-dive; the tie rule
// and the softmax over the k chosen logits are this library's definition.
// The same kernel optionally counts, per chunk of tokens, how many
// assignments each expert received (the histogram for the permutation).
//
// permute_kernel: a stable counting sort of the assignments (t, j) by expert.
// Each block owns one chunk of tokens: it derives each expert's first free
// row for the chunk from the per-chunk histogram table (exclusive scan over
// experts of the totals, plus the counts of earlier chunks), ranks its own
// assignments in (t, j) order, writes the row maps and copies its tokens'
// rows of x into x_perm. Per-expert contiguous activations as in the
// DeepGEMM article (itsolotime.com), section 3.1; re-arrangement before the
// grouped GEMM as in the HPC-Ops article (ntfzh.com), FusedMoE paragraph.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kMaxQ = kMaxExperts / kWave;  // logits per lane

// Order-preserving map of an fp32 bit pattern to uint32 (larger float ->
// larger key); -0.0 is first canonicalised to +0.0 so the two tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ logits, int T, int E, int k, int chunk_tokens,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist /* [nchunks][E] or null */) {
  __shared__ int s_count[kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = kRouteThreads / kWave;
  if (hist)
    for (int e = threadIdx.x; e < E; e += kRouteThreads) s_count[e] = 0;
  __syncthreads();

  const int t_begin = blockIdx.x * chunk_tokens;
  const int t_end = min(T, t_begin + chunk_tokens);
  const int Q = (E + kWave - 1) / kWave;
  for (int t = t_begin + wave; t < t_end; t += nwaves) {
    const float* row = logits + static_cast<int64_t>(t) * E;
    uint64_t key[kMaxQ];
#pragma unroll
    for (int q = 0; q < kMaxQ; ++q) {
      const int e = lane + q * kWave;
      key[q] = 0;  // below every real key: never chosen while k <= E
      if (q < Q && e < E)
        key[q] = (static_cast<uint64_t>(order_key(row[e])) << 32) |
                 static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(e));
    }
    int my_id = 0;
    float my_logit = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int q = 0; q < kMaxQ; ++q) best = key[q] > best ? key[q] : best;
      best = wave_max_u64(best);
#pragma unroll
      for (int q = 0; q < kMaxQ; ++q) key[q] = (key[q] == best) ? 0 : key[q];
      if (lane == j) {
        my_id = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
        my_logit = key_to_float(static_cast<uint32_t>(best >> 32));
      }
    }
    // softmax over the k chosen logits; slot 0 (lane 0) holds the largest
    const float m = __shfl(my_logit, 0, kWave);
    const float ex = (lane < k) ? expf(my_logit - m) : 0.f;
    float s = ex;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
    if (lane < k) {
      topk_ids[static_cast<int64_t>(t) * k + lane] = my_id;
      topk_w[static_cast<int64_t>(t) * k + lane] = ex / s;
      if (hist) atomicAdd(&s_count[min(max(my_id, 0), E - 1)], 1);
    }
  }
  if (hist) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouteThreads)
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
constexpr int kExpPerThread = kMaxExperts / kPermThreads;  // 4

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ topk_ids, int T,
    int H, int E, int k, int chunk_tokens, int nchunks, int slice_cols,
    const int32_t* __restrict__ hist, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_dest,
    bf16_t* __restrict__ x_perm) {
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_wave_total[kPermThreads / kWave];
  __shared__ int s_ids[kMaxChunkAssign];
  __shared__ int s_dest[kMaxChunkAssign];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int chunk = blockIdx.x;

  // 1. first free row of each expert for this chunk
  int before[kExpPerThread], total[kExpPerThread];
  int my_sum = 0;
#pragma unroll
  for (int i = 0; i < kExpPerThread; ++i) {
    const int e = tid * kExpPerThread + i;
    int b = 0, a = 0;
    if (e < E) {
      for (int c = 0; c < nchunks; ++c) {
        const int v = hist[static_cast<int64_t>(c) * E + e];
        a += v;
        if (c < chunk) b += v;
      }
    }
    before[i] = b;
    total[i] = a;
    my_sum += a;
  }
  // exclusive scan over experts (thread-major order) of the totals
  int incl = wave_inclusive_scan(my_sum);
  if (lane == kWave - 1) s_wave_total[wave] = incl;
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < wave; ++w) wave_off += s_wave_total[w];
  int run = wave_off + incl - my_sum;
#pragma unroll
  for (int i = 0; i < kExpPerThread; ++i) {
    const int e = tid * kExpPerThread + i;
    if (e < E) {
      if (chunk == 0 && blockIdx.y == 0) expert_offsets[e] = run;
      s_base[e] = run + before[i];
    }
    run += total[i];
  }
  if (chunk == 0 && blockIdx.y == 0 && tid == 0)
    expert_offsets[E] = T * k;

  // 2. stable rank of this chunk's assignments in (t, j) order
  const int t0 = chunk * chunk_tokens;
  const int nt = min(T - t0, chunk_tokens);
  const int n = nt * k;
  const int64_t a0 = static_cast<int64_t>(t0) * k;
  for (int i = tid; i < n; i += kPermThreads) {
    int e = topk_ids[a0 + i];
    s_ids[i] = e < 0 ? 0 : (e >= E ? E - 1 : e);
  }
  __syncthreads();
  for (int i = tid; i < n; i += kPermThreads) {
    const int e = s_ids[i];
    int rank = 0;
    for (int i2 = 0; i2 < i; ++i2) rank += (s_ids[i2] == e);
    int p = s_base[e] + rank;
    p = p < T * k ? p : T * k - 1;  // in bounds even for out-of-contract ids
    s_dest[i] = p;
    if (blockIdx.y == 0) {
      row_dest[a0 + i] = p;
      row_token[p] = t0 + i / k;
    }
  }
  __syncthreads();

  // 3. copy this block's column slice of each assigned row: x_perm[p] = x[t]
  const int c_begin = blockIdx.y * slice_cols;
  const int c_end = min(H, c_begin + slice_cols);
  const int vec_per_row = (c_end - c_begin) / 8;  // 16-byte vectors
  for (int v = tid; v < n * vec_per_row; v += kPermThreads) {
    const int i = v / vec_per_row;
    const int c = c_begin + (v - i * vec_per_row) * 8;
    const int t = t0 + i / k;
    const uint4 val = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * H + c);
    *reinterpret_cast<uint4*>(x_perm + static_cast<int64_t>(s_dest[i]) * H + c) = val;
  }
}

}  // namespace

int route_chunk_tokens(int k) { return kMaxChunkAssign / k; }

int route_num_chunks(int T, int k) {
  const int c = route_chunk_tokens(k);
  return (T + c - 1) / c;
}

hipError_t launch_route(const float* logits, int T, int E, int k,
                        int32_t* topk_ids, float* topk_w, int32_t* hist,
                        hipStream_t stream) {
  const int chunk = route_chunk_tokens(k);
  const int nchunks = route_num_chunks(T, k);
  hipLaunchKernelGGL(route_kernel, dim3(nchunks), dim3(kRouteThreads), 0,
                     stream, logits, T, E, k, chunk, topk_ids, topk_w, hist);
  return hipGetLastError();
}

hipError_t launch_hist(const int32_t* topk_ids, int T, int E, int k,
                       int32_t* hist, hipStream_t stream) {
  const int chunk = route_chunk_tokens(k);
  const int nchunks = route_num_chunks(T, k);
  hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(kRouteThreads), 0,
                     stream, topk_ids, T, E, k, chunk, hist);
  return hipGetLastError();
}

hipError_t launch_permute(const bf16_t* x, const int32_t* topk_ids, int T,
                          int H, int E, int k, const int32_t* hist,
                          int32_t* expert_offsets, int32_t* row_token,
                          int32_t* row_dest, bf16_t* x_perm,
                          hipStream_t stream) {
  const int chunk = route_chunk_tokens(k);
  const int nchunks = route_num_chunks(T, k);
  const int slice = kPermuteSliceCols;
  const int nslices = (H + slice - 1) / slice;
  hipLaunchKernelGGL(permute_kernel, dim3(nchunks, nslices), dim3(kPermThreads),
                     0, stream, x, topk_ids, T, H, E, k, chunk, nchunks, slice,
                     hist, expert_offsets, row_token, row_dest, x_perm);
  return hipGetLastError();
}

}  // namespace moe
