// Training backward of the MoE expert layer: the kernels that are not the
// grouped GEMM itself (the grouped-GEMM news page, meineki.news, notes that
// the kernel serves training as well as inference; the pages give no
// backward, so these are the chain rule through the forward's steps).
//
//   preparation: per row p of (t,j), dy[p] = w[t,j] dout[t] (bf16, for
//     dW_down), dout[t] itself and w[t,j]; the dh product runs on the
//     unweighted dout, g = dout W_down^T, so that the routing-weight gradient
//     d_w[t,j] = <dout[t], y[p]> = <h[p], g[p]> comes out of its epilogue
//     (per-fragment partial sums, added in a fixed order) and the forward's
//     down projection need not be recomputed.
//   route backward: the softmax over the k selected logits,
//     d_logit[t, id_j] = w_j (d_w_j - sum_i w_i d_w_i), 0 elsewhere.
//   K-grouped GEMM: dW[e] = sum over the expert's rows p of a[p]^T b[p]
//     (the reduction runs over each expert's token segment, so K differs per
//     expert): dW_down = h^T dy, dW_gate = x^T dG, dW_up = x^T dU.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {

namespace {

// --- backward preparation -------------------------------------------------
// Per token (one block of 256 threads, 8 columns each per pass) and slot j,
// with p = row_dest[t,j]: dy[p] = bf16(w dout[t]) (for dW_down),
// dout_perm[p] = dout[t] (the unweighted operand of dh), wrow[p] = w.
constexpr int kPrepThreads = 256;

__global__ __launch_bounds__(kPrepThreads) void backward_prep_kernel(
    const bf16_t* __restrict__ dout, const int32_t* __restrict__ row_dest,
    const float* __restrict__ topk_w, int T, int H, int k, bf16_t* __restrict__ dy,
    bf16_t* __restrict__ dout_perm, float* __restrict__ wrow) {
  const int t = blockIdx.x;
  const int64_t A = static_cast<int64_t>(T) * k;
  for (int j = 0; j < k; ++j) {
    int p = row_dest[static_cast<int64_t>(t) * k + j];
    p = p < 0 ? 0 : (p >= A ? static_cast<int>(A - 1) : p);  // stay in bounds
    const float w = topk_w[static_cast<int64_t>(t) * k + j];
    if (threadIdx.x == 0) wrow[p] = w;
    for (int c = threadIdx.x * 8; c < H; c += kPrepThreads * 8) {
      const uint4 q = *reinterpret_cast<const uint4*>(dout + static_cast<int64_t>(t) * H + c);
      *reinterpret_cast<uint4*>(dout_perm + static_cast<int64_t>(p) * H + c) = q;
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
      float d[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d[2 * i] = bf16_to_f32(static_cast<bf16_t>(u[i] & 0xffffu));
        d[2 * i + 1] = bf16_to_f32(static_cast<bf16_t>(u[i] >> 16));
      }
      uint4 o;
      o.x = pack_bf16x2(w * d[0], w * d[1]);
      o.y = pack_bf16x2(w * d[2], w * d[3]);
      o.z = pack_bf16x2(w * d[4], w * d[5]);
      o.w = pack_bf16x2(w * d[6], w * d[7]);
      *reinterpret_cast<uint4*>(dy + static_cast<int64_t>(p) * H + c) = o;
    }
  }
}

// --- the shared expert's preparation ------------------------------------------
// Per token (one block): s = 1, or the logistic sigmoid of the gate logit
// (the forward's combine computes it the same way), wrow[t] = s and
// dy[t] = bf16(s dout[t]); block 0 also writes the single group's offsets.
__global__ __launch_bounds__(kPrepThreads) void shared_prep_kernel(
    const bf16_t* __restrict__ dout, const float* __restrict__ gate_logits, int T, int H,
    bf16_t* __restrict__ dy, float* __restrict__ wrow, int32_t* __restrict__ offsets) {
  const int t = blockIdx.x;
  const float s = gate_logits ? 1.0f / (1.0f + expf(-gate_logits[t])) : 1.0f;
  if (threadIdx.x == 0) {
    wrow[t] = s;
    if (t == 0) {
      offsets[0] = 0;
      offsets[1] = T;
    }
  }
  for (int c = threadIdx.x * 8; c < H; c += kPrepThreads * 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(dout + static_cast<int64_t>(t) * H + c);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
    float d[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[2 * i] = bf16_to_f32(static_cast<bf16_t>(u[i] & 0xffffu));
      d[2 * i + 1] = bf16_to_f32(static_cast<bf16_t>(u[i] >> 16));
    }
    uint4 o;
    o.x = pack_bf16x2(s * d[0], s * d[1]);
    o.y = pack_bf16x2(s * d[2], s * d[3]);
    o.z = pack_bf16x2(s * d[4], s * d[5]);
    o.w = pack_bf16x2(s * d[6], s * d[7]);
    *reinterpret_cast<uint4*>(dy + static_cast<int64_t>(t) * H + c) = o;
  }
}

// Gate-logit gradient of the shared expert: <dout[t], y_sh[t]> s (1 - s),
// the inner product being the sum of the dh product's per-fragment partial
// sums of row t (in order, then a fixed butterfly), one wave per token.
__global__ __launch_bounds__(256) void shared_gate_grad_kernel(
    const float* __restrict__ part, int nq, const float* __restrict__ gate_logits, int T,
    float* __restrict__ d_gate) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;  // whole waves
  const float* r = part + t * nq;
  float acc = 0.f;
  for (int q = lane; q < nq; q += kWave) acc += r[q];
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kWave);
  if (lane == 0) {
    const float s = 1.0f / (1.0f + expf(-gate_logits[t]));
    d_gate[t] = acc * s * (1.0f - s);
  }
}

// --- routing-weight gradient --------------------------------------------------
// d_topk_w[t,j] = <dout[t], y[p]> = <h[p], g[p]> (g = dout W_down^T), the sum
// of the dh GEMM's per-fragment partial sums of row p. One wave per
// assignment: lane l adds fragments l, l + 64, ... in order, then the lanes
// are added by a fixed butterfly, so the result does not depend on timing.
__global__ __launch_bounds__(256) void topk_w_grad_kernel(
    const float* __restrict__ part, int nq, const int32_t* __restrict__ row_dest, int64_t n,
    float* __restrict__ d_topk_w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (i >= n) return;  // whole waves
  int64_t p = row_dest[i];
  p = p < 0 ? 0 : (p >= n ? n - 1 : p);
  const float* r = part + p * nq;
  float s = 0.f;
  for (int q = lane; q < nq; q += kWave) s += r[q];
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, kWave);
  if (lane == 0) d_topk_w[i] = s;
}

// --- route backward -----------------------------------------------------
// One thread per (token, expert); each recomputes the token's sum over its
// k slots in slot order (k <= 16).
__global__ __launch_bounds__(256) void route_backward_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, const float* __restrict__ dw,
    int T, int E, int k, float* __restrict__ dl) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(T) * E) return;
  const int64_t t = idx / E;
  const int e = static_cast<int>(idx % E);
  const int32_t* id = ids + t * k;
  const float* wt = w + t * k;
  const float* dwt = dw + t * k;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += wt[j] * dwt[j];
  float v = 0.f;
  for (int j = 0; j < k; ++j)
    if (id[j] == e) v = wt[j] * (dwt[j] - s);
  dl[idx] = v;
}

// --- K-grouped GEMM -------------------------------------------------------
// out[e][i][j] = sum_{p in e} a[p][i] b[p][j]. A workgroup owns one
// (expert, 256-row i tile, 256-column j tile) and walks the expert's rows
// 32 at a time. Each step's operands are staged in LDS as [32 rows p][256
// columns] in four 64-column sub-blocks of 128-byte rows (16-byte chunks
// XOR-swizzled by 2*(p % 4) ^ 2*((p / 8) % 2)) by direct-to-LDS loads, in a
// 4-deep ring (up to three steps in flight). Rows past the expert load its last row and columns past M or N the
// last 8 columns, all in bounds: the a-fragments of rows past the expert
// are zeroed, and the outputs past M or N are not stored. The MFMA operands
// need 8 consecutive p per lane, which the transposing LDS read
// ds_read_b64_tr_b16 delivers from that layout. 8 waves as 4 (i) x 2 (j),
// each 64 x 128 (4 x 8 blocks of v_mfma_f32_16x16x32_bf16), on a ping-pong
// schedule (below): a 256 x 256 tile loads 32 KB per 32-row step for
// 4 MFLOP, twice the arithmetic per loaded byte of a 128 x 128 tile.
constexpr int kKgThreads = 512;
constexpr int kKgTile = 256;
constexpr int kKgBK = 32;
constexpr int kKgStages = 4;
constexpr int kKgSub = kKgBK * 128;               // bytes of one 64-column sub-block
constexpr int kKgOp = kKgTile / 64 * kKgSub;      // bytes of one operand's stage (16 KB)
constexpr int kKgStage = 2 * kKgOp;               // a then b
constexpr int kKgIpw = kKgStage / 1024 / (kKgThreads / kWave);  // DMA instructions per wave

__device__ __forceinline__ int kg_swz(int row, int chunk) {
  return chunk ^ ((row & 3) << 1) ^ (((row >> 3) & 1) << 1);
}

// Fragment of 16 columns (c0 .. c0+15) of a staged [32][256] operand: lane
// (i16, g16) gets rows 8*g16 .. 8*g16+7 of column c0 + i16 (the transposing
// read gives lane i of each 16-lane group element i % 4 of the 8-byte
// pieces read by lanes 4r + i / 4).
__device__ __forceinline__ bf16x8 kg_frag(const char* tile, int c0, int lane) {
  const int i16 = lane & 15, g16 = lane >> 4;
  const int row = 8 * g16 + (i16 >> 2);
  const int col = c0 + 4 * (i16 & 3);
  const int c64 = col & 63;
  const char* p = tile + (col >> 6) * kKgSub + row * 128 + kg_swz(row, c64 >> 3) * 16 +
                  (c64 & 7) * 2;
  const short4_t lo = lds_read_tr16(p);
  const short4_t hi = lds_read_tr16(p + 4 * 128);
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t s8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, s8);
}

__global__ __launch_bounds__(kKgThreads) void kgrouped_gemm_kernel(
    const bf16_t* __restrict__ a, const bf16_t* __restrict__ b,
    const int32_t* __restrict__ offsets, int E, int M, int N, int tiles_i, int tiles_j,
    float* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char ring[kKgStages][kKgStage];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wi = wave / 2, wj = wave % 2;
  const int tiles = tiles_i * tiles_j;
  const int e = blockIdx.x / tiles;
  const int i0 = (blockIdx.x % tiles) / tiles_j * kKgTile;
  const int j0 = (blockIdx.x % tiles) % tiles_j * kKgTile;
  const int rows = offsets ? max(0, offsets[e + 1] - offsets[e]) : 0;  // null: no rows
  const int64_t r0 = offsets ? offsets[e] : 0;
  const int nk = (rows + kKgBK - 1) / kKgBK;

  // DMA instruction j = wave + 8 i of a stage fills its 1 KB at j * 1024:
  // operand j / 16, sub-block (j % 16) / 4, rows 8 (j % 4) .. +7; the lane's
  // slot (row, physical chunk lane % 8) holds logical chunk kg_swz(row, .)
  int rrow[kKgIpw], rcol[kKgIpw];
#pragma unroll
  for (int i = 0; i < kKgIpw; ++i) {
    const int j = wave + (kKgThreads / kWave) * i;
    const int jj = j % 16;
    const int row = (jj % 4) * 8 + lane / 8;
    const int col = (j < 16 ? i0 : j0) + (jj / 4) * 64 + kg_swz(row, lane % 8) * 8;
    rrow[i] = row;
    rcol[i] = min(col, (j < 16 ? M : N) - 8);
  }
  auto issue = [&](int t) {
    // steps past the last re-load the last one (a fixed count in flight)
    const int kk = min(t, nk - 1) * kKgBK;
    char* const dst = ring[t % kKgStages];
#pragma unroll
    for (int i = 0; i < kKgIpw; ++i) {
      const int j = wave + (kKgThreads / kWave) * i;
      const bool is_a = j < 16;  // wave-uniform
      const int ld = is_a ? M : N;
      const bf16_t* base = (is_a ? a : b) + (r0 + kk) * ld;
      const int prow = min(rrow[i], rows - 1 - kk);
      dma16(base, static_cast<uint32_t>(prow * ld + rcol[i]) * 2u, dst + j * 1024);
    }
  };

  floatx4 acc[4][8];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) acc[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Ping-pong schedule: waves 0-3 and 4-7 (one of each per SIMD) alternate
  // between a memory phase M(t) (fragment reads of step t, the wait for the
  // wave's own loads of step t+1, the loads of step t+3) and a compute
  // phase C(t) (32 MFMAs), each closed by a workgroup barrier; waves 4-7
  // pass one extra barrier first, so in interval 2t waves 0-3 run M(t) while
  // waves 4-7 run C(t-1), and in 2t+1 the reverse: one wave of each SIMD
  // keeps the matrix core busy while the other moves data. Step t+1 is read
  // from interval 2t+2 on, after both groups have waited for their loads of
  // it (in 2t and 2t+1); the buffer refilled in M(t) held step t-1, whose
  // fragments both groups read in intervals 2t-2 and 2t-1.
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nk > 0) {
    const bool grp1 = wave >= 4;
    const int g16 = lane >> 4;
#pragma unroll
    for (int t = 0; t < kKgStages - 1; ++t) issue(t);
    wait_vmcnt<(kKgStages - 2) * kKgIpw>();  // this wave's loads of step 0 have landed
    barrier();                               // ... and every wave's
    if (grp1) barrier();
    bf16x8 fa[4], fb[8];
    for (int t = 0; t < nk; ++t) {
      const char* sa = ring[t % kKgStages];
      const char* sb = sa + kKgOp;
#pragma unroll
      for (int x = 0; x < 4; ++x) fa[x] = kg_frag(sa, wi * 64 + x * 16, lane);
#pragma unroll
      for (int y = 0; y < 8; ++y) fb[y] = kg_frag(sb, wj * 128 + y * 16, lane);
      wait_vmcnt<(kKgStages - 3) * kKgIpw>();  // this wave's loads of step t+1 have landed
      issue(t + kKgStages - 1);
      wait_vmcnt_lgkm0<63>();                  // fragments in registers
      const int left = rows - t * kKgBK - 8 * g16;  // valid rows among the lane's 8
      if (left < 8) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (r >= left) fa[x][r] = __bf16(0.0f);
      }
      barrier();
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
      barrier();
    }
    if (!grp1) barrier();
    // no LDS DMA may land after the workgroup ends
    wait_vmcnt<0>();
  }
  // lane (i16, g16) holds rows 4*g16 .. 4*g16+3 of column i16 of each block
  const int i16 = lane & 15, g16 = lane >> 4;
  float* oe = out + static_cast<int64_t>(e) * M * N;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      const int j = j0 + wj * 128 + y * 16 + i16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + wi * 64 + x * 16 + 4 * g16 + r;
        if (i < M && j < N) oe[static_cast<int64_t>(i) * N + j] = acc[x][y][r];
      }
    }
}

}  // namespace

hipError_t launch_backward_prep(const bf16_t* dout, const int32_t* row_dest,
                                const float* topk_w, int T, int H, int k, bf16_t* dy,
                                bf16_t* dout_perm, float* wrow, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  MOE_TRACE_LAUNCH("backward_prep_kernel", dim3(T), dim3(kPrepThreads), 0, "T=%d H=%d k=%d", T, H,
                   k);
  hipLaunchKernelGGL(backward_prep_kernel, dim3(T), dim3(kPrepThreads), 0, stream, dout,
                     row_dest, topk_w, T, H, k, dy, dout_perm, wrow);
  return hipGetLastError();
}

hipError_t launch_shared_prep(const bf16_t* dout, const float* gate_logits, int T, int H,
                              bf16_t* dy, float* wrow, int32_t* offsets, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  MOE_TRACE_LAUNCH("shared_prep_kernel", dim3(T), dim3(kPrepThreads), 0, "T=%d H=%d gated=%d", T,
                   H, gate_logits ? 1 : 0);
  hipLaunchKernelGGL(shared_prep_kernel, dim3(T), dim3(kPrepThreads), 0, stream, dout,
                     gate_logits, T, H, dy, wrow, offsets);
  return hipGetLastError();
}

hipError_t launch_shared_gate_grad(const float* part, int nq, const float* gate_logits, int T,
                                   float* d_gate, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((T + 3) / 4);
  MOE_TRACE_LAUNCH("shared_gate_grad_kernel", dim3(blocks), dim3(256), 0, "T=%d partials=%d", T,
                   nq);
  hipLaunchKernelGGL(shared_gate_grad_kernel, dim3(blocks), dim3(256), 0, stream, part, nq,
                     gate_logits, T, d_gate);
  return hipGetLastError();
}

hipError_t launch_topk_w_grad(const float* part, int nq, const int32_t* row_dest, int T, int k,
                              float* d_topk_w, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(T) * k;
  if (n <= 0) return hipSuccess;
  MOE_TRACE_LAUNCH("topk_w_grad_kernel", dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0,
                   "assignments=%lld partials=%d", static_cast<long long>(n), nq);
  hipLaunchKernelGGL(topk_w_grad_kernel, dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0,
                     stream, part, nq, row_dest, n, d_topk_w);
  return hipGetLastError();
}

hipError_t launch_route_backward(const int32_t* topk_ids, const float* topk_w,
                                 const float* d_topk_w, int T, int E, int k, float* d_logits,
                                 hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(T) * E;
  if (n <= 0) return hipSuccess;
  MOE_TRACE_LAUNCH("route_backward_kernel", dim3(static_cast<unsigned>((n + 255) / 256)),
                   dim3(256), 0, "T=%d E=%d k=%d", T, E, k);
  hipLaunchKernelGGL(route_backward_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, stream, topk_ids, topk_w, d_topk_w, T, E, k, d_logits);
  return hipGetLastError();
}

hipError_t launch_kgrouped_gemm(const bf16_t* a, const bf16_t* b, const int32_t* offsets,
                                int E, int M, int N, float* out, hipStream_t stream) {
  const int ti = (M + kKgTile - 1) / kKgTile, tj = (N + kKgTile - 1) / kKgTile;
  const int64_t blocks = static_cast<int64_t>(E) * ti * tj;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  MOE_TRACE_LAUNCH("kgrouped_gemm_kernel", dim3(static_cast<unsigned>(blocks)), dim3(kKgThreads),
                   0, "tile=%dx%d groups=%d M=%d N=%d", kKgTile, kKgTile, E, M, N);
  hipLaunchKernelGGL(kgrouped_gemm_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kKgThreads), 0, stream, a, b, offsets, E, M, N, ti, tj, out);
  return hipGetLastError();
}

}  // namespace moe
