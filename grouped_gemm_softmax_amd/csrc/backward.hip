// Training backward of the MoE expert layer: the kernels that are not the
// grouped GEMM itself (the grouped-GEMM news page, meineki.news, notes that
// the kernel serves training as well as inference; the pages give no
// backward, so these are the chain rule through the forward's steps).
//
//   combine backward: dy[row(t,j)] = w[t,j] dout[t], and the routing-weight
//     gradient d_w[t,j] = <dout[t], y[row(t,j)]>: a gather through the
//     inverse map with a deterministic block reduction.
//   route backward: the softmax over the k selected logits,
//     d_logit[t, id_j] = w_j (d_w_j - sum_i w_i d_w_i), 0 elsewhere.
//   K-grouped GEMM: dW[e] = sum over the expert's rows p of a[p]^T b[p]
//     (the reduction runs over each expert's token segment, so K differs per
//     expert): dW_down = h^T dy, dW_gate = x^T dG, dW_up = x^T dU.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// --- combine backward ---------------------------------------------------
// One block per token; 256 threads, 8 columns each per pass. The dot
// product is reduced per thread in column order, then across the block in a
// fixed tree: the result does not depend on timing.
constexpr int kCbThreads = 256;

__global__ __launch_bounds__(kCbThreads) void combine_backward_kernel(
    const bf16_t* __restrict__ dout, const float* __restrict__ y,
    const int32_t* __restrict__ row_dest, const float* __restrict__ topk_w, int T, int H, int k,
    bf16_t* __restrict__ dy, float* __restrict__ d_topk_w) {
  const int t = blockIdx.x;
  __shared__ float s_red[kCbThreads / kWave];
  const int64_t A = static_cast<int64_t>(T) * k;
  for (int j = 0; j < k; ++j) {
    int p = row_dest[static_cast<int64_t>(t) * k + j];
    p = p < 0 ? 0 : (p >= A ? static_cast<int>(A - 1) : p);  // stay in bounds
    const float w = topk_w[static_cast<int64_t>(t) * k + j];
    float dot = 0.f;
    for (int c = threadIdx.x * 8; c < H; c += kCbThreads * 8) {
      const uint4 q = *reinterpret_cast<const uint4*>(dout + static_cast<int64_t>(t) * H + c);
      const float4 ya = *reinterpret_cast<const float4*>(y + static_cast<int64_t>(p) * H + c);
      const float4 yb = *reinterpret_cast<const float4*>(y + static_cast<int64_t>(p) * H + c + 4);
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
      const float yv[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
      float d[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d[2 * i] = bf16_to_f32(static_cast<bf16_t>(u[i] & 0xffffu));
        d[2 * i + 1] = bf16_to_f32(static_cast<bf16_t>(u[i] >> 16));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += d[i] * yv[i];
      uint4 o;
      o.x = pack_bf16x2(w * d[0], w * d[1]);
      o.y = pack_bf16x2(w * d[2], w * d[3]);
      o.z = pack_bf16x2(w * d[4], w * d[5]);
      o.w = pack_bf16x2(w * d[6], w * d[7]);
      *reinterpret_cast<uint4*>(dy + static_cast<int64_t>(p) * H + c) = o;
    }
    // block sum: butterfly within each wave, then the waves in order
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s_red[threadIdx.x / kWave] = dot;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.f;
      for (int i = 0; i < kCbThreads / kWave; ++i) s += s_red[i];
      d_topk_w[static_cast<int64_t>(t) * k + j] = s;
    }
    __syncthreads();
  }
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
// (expert, 128-row i tile, 128-column j tile) and walks the expert's rows
// 32 at a time. Both operands are staged in LDS as [32 rows p][128 columns]
// in two 64-column sub-blocks of 128-byte rows (16-byte chunks XOR-swizzled
// by 2*(p % 4) ^ 2*((p / 8) % 2)), double-buffered with plain loads (rows
// past the expert and columns past M or N are zeros); the MFMA operands
// need 8 consecutive p per lane, which the transposing LDS read
// ds_read_b64_tr_b16 delivers from that layout. 4 waves as 2 x 2, each
// 64 x 64 (4 x 4 blocks of v_mfma_f32_16x16x32_bf16).
constexpr int kKgThreads = 256;
constexpr int kKgTile = 128;
constexpr int kKgBK = 32;

__device__ __forceinline__ int kg_swz(int row, int chunk) {
  return chunk ^ ((row & 3) << 1) ^ (((row >> 3) & 1) << 1);
}

__device__ __forceinline__ short4_t kg_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

// Fragment of 16 columns (c0 .. c0+15) of a staged [32][128] tile: lane
// (i16, g16) gets rows 8*g16 .. 8*g16+7 of column c0 + i16. Within each
// 16-lane group, lane i of a transposing read receives element i % 4 of the
// 8-byte pieces read by lanes 4r + i / 4.
__device__ __forceinline__ bf16x8 kg_frag(const char* tile, int c0, int lane) {
  const int i16 = lane & 15, g16 = lane >> 4;
  const int row = 8 * g16 + (i16 >> 2);
  const int col = c0 + 4 * (i16 & 3);
  const int c64 = col & 63;
  const char* p = tile + (col >> 6) * (kKgBK * 128) + row * 128 + kg_swz(row, c64 >> 3) * 16 +
                  (c64 & 7) * 2;
  const short4_t lo = kg_tr16(p);
  const short4_t hi = kg_tr16(p + 4 * 128);
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t s8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, s8);
}

__global__ __launch_bounds__(kKgThreads) void kgrouped_gemm_kernel(
    const bf16_t* __restrict__ a, const bf16_t* __restrict__ b,
    const int32_t* __restrict__ offsets, int E, int M, int N, int tiles_i, int tiles_j,
    float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char sa[2][kKgBK * kKgTile * 2];
  __shared__ __attribute__((aligned(16))) char sb[2][kKgBK * kKgTile * 2];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = tid / kWave, wi = wave / 2, wj = wave % 2;
  const int tiles = tiles_i * tiles_j;
  const int e = blockIdx.x / tiles;
  const int i0 = (blockIdx.x % tiles) / tiles_j * kKgTile;
  const int j0 = (blockIdx.x % tiles) % tiles_j * kKgTile;
  const int rows = offsets ? max(0, offsets[e + 1] - offsets[e]) : 0;  // null: no rows
  const int64_t r0 = offsets ? offsets[e] : 0;

  // this thread's 2 chunks of each operand per step: chunk q = tid + 256 s
  // -> sub-block q / 256, row (q / 8) % 32, logical column chunk q % 8.
  // The next step's chunks are loaded into registers before the current
  // step's MFMAs and written to the other LDS buffer after them.
  uint4 ra[2], rb[2];
  auto load = [&](int kk) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = tid + kKgThreads * s;
      const int sbk = q / 256, row = (q / 8) % 32, ch = q % 8;
      const int p = kk + row;
      const int ci = i0 + sbk * 64 + ch * 8;
      const int cj = j0 + sbk * 64 + ch * 8;
      ra[s] = uint4{0u, 0u, 0u, 0u};
      rb[s] = uint4{0u, 0u, 0u, 0u};
      if (p < rows) {
        if (ci < M) ra[s] = *reinterpret_cast<const uint4*>(a + (r0 + p) * M + ci);
        if (cj < N) rb[s] = *reinterpret_cast<const uint4*>(b + (r0 + p) * N + cj);
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = tid + kKgThreads * s;
      const int sbk = q / 256, row = (q / 8) % 32, ch = q % 8;
      const int off = sbk * (kKgBK * 128) + row * 128 + kg_swz(row, ch) * 16;
      *reinterpret_cast<uint4*>(sa[buf] + off) = ra[s];
      *reinterpret_cast<uint4*>(sb[buf] + off) = rb[s];
    }
  };

  floatx4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (rows + kKgBK - 1) / kKgBK;
  if (nk > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) load((s + 1) * kKgBK);
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) fa[x] = kg_frag(sa[buf], wi * 64 + x * 16, lane);
#pragma unroll
    for (int y = 0; y < 4; ++y) fb[y] = kg_frag(sb[buf], wj * 64 + y * 16, lane);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    if (s + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // lane (i16, g16) holds rows 4*g16 .. 4*g16+3 of column i16 of each block
  const int i16 = lane & 15, g16 = lane >> 4;
  float* oe = out + static_cast<int64_t>(e) * M * N;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = j0 + wj * 64 + y * 16 + i16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + wi * 64 + x * 16 + 4 * g16 + r;
        if (i < M && j < N) oe[static_cast<int64_t>(i) * N + j] = acc[x][y][r];
      }
    }
}

}  // namespace

hipError_t launch_combine_backward(const bf16_t* dout, const float* y, const int32_t* row_dest,
                                   const float* topk_w, int T, int H, int k, bf16_t* dy,
                                   float* d_topk_w, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_backward_kernel, dim3(T), dim3(kCbThreads), 0, stream, dout, y,
                     row_dest, topk_w, T, H, k, dy, d_topk_w);
  return hipGetLastError();
}

hipError_t launch_route_backward(const int32_t* topk_ids, const float* topk_w,
                                 const float* d_topk_w, int T, int E, int k, float* d_logits,
                                 hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(T) * E;
  if (n <= 0) return hipSuccess;
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
  hipLaunchKernelGGL(kgrouped_gemm_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kKgThreads), 0, stream, a, b, offsets, E, M, N, ti, tj, out);
  return hipGetLastError();
}

}  // namespace moe
