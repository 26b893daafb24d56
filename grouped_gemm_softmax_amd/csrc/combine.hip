// Combine / un-permute of the MoE expert layer:
//   out[t,c] = bf16( sum_{j<k} w[t,j] * y_perm[row_dest[t,j], c]
//                    + s_t * y_shared[t,c] )
// with fp32 accumulation in ascending j and the shared term added last.
// y_perm and y_shared are bf16 (the split ABI) or fp32 (inside the fused
// layer, where the down projection's output skips the bf16 rounding; there a
// decode-size down projection may come as K-slice partial sums, which are
// added here in slice order before the routing weight is applied).
// Semantically a scatter-add of the weighted expert rows back to their
// tokens; it is computed as a gather through the inverse map row_dest, so no
// floating-point atomics are used and the result is deterministic. The
// weighted reduce after the grouped GEMM follows the HPC-Ops article
// (ntfzh.com), FusedMoE paragraph; the combine stage of the DeepGEMM article
// (itsolotime.com), section 1.1, is the same step. s_t = 1 without gate
// logits, else the logistic sigmoid of the token's gate logit.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCombineThreads = 256;

// 8 consecutive values of a row as fp32.
__device__ __forceinline__ void load8(const bf16_t* p, float v[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(static_cast<bf16_t>(u[i] & 0xffffu));
    v[2 * i + 1] = bf16_to_f32(static_cast<bf16_t>(u[i] >> 16));
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One row as the sum of its K-slices, added in slice order; the loads of
// all slices are issued before the first add.
template <typename YT>
__device__ __forceinline__ void load8_sum(const YT* p, int nslices, int64_t stride, float v[8]) {
  float u[kMaxKSplit][8];
#pragma unroll
  for (int s = 0; s < kMaxKSplit; ++s)
    if (s < nslices) load8(p + s * stride, u[s]);
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = u[0][q];
#pragma unroll
  for (int s = 1; s < kMaxKSplit; ++s)
    if (s < nslices) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += u[s][q];
    }
}

template <typename YT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const YT* __restrict__ y_perm, int nslices, int64_t y_slice_stride,
    const int32_t* __restrict__ row_dest,
    const float* __restrict__ topk_w, int T, int H, int k,
    const YT* __restrict__ y_shared, int nslices_sh, int64_t ysh_slice_stride,
    const float* __restrict__ shared_gate, bf16_t* __restrict__ out) {
  // block (t, column block): 8 columns per thread
  const int t = blockIdx.x;
  __shared__ int s_row[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int64_t A = static_cast<int64_t>(T) * k;
  if (threadIdx.x < k) {
    int p = row_dest[static_cast<int64_t>(t) * k + threadIdx.x];
    p = p < 0 ? 0 : (p >= A ? static_cast<int>(A - 1) : p);  // stay in bounds
    s_row[threadIdx.x] = p;
    s_w[threadIdx.x] = topk_w ? topk_w[static_cast<int64_t>(t) * k + threadIdx.x] : 1.0f;
  }
  __syncthreads();
  float s = 1.0f;
  if (y_shared && shared_gate) s = 1.0f / (1.0f + expf(-shared_gate[t]));
  {
    const int c = (blockIdx.y * kCombineThreads + threadIdx.x) * 8;
    if (c >= H) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[8];
    for (int j = 0; j < k; ++j) {
      load8_sum(y_perm + static_cast<int64_t>(s_row[j]) * H + c, nslices, y_slice_stride, v);
      const float w = s_w[j];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += w * v[q];
    }
    if (y_shared) {
      load8_sum(y_shared + static_cast<int64_t>(t) * H + c, nslices_sh, ysh_slice_stride, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += s * v[q];
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + static_cast<int64_t>(t) * H + c) = o;
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, bool y_f32, int nslices,
                          int64_t y_slice_stride, const int32_t* row_dest,
                          const float* topk_w, int T, int H, int k,
                          const void* y_shared, int nslices_sh, int64_t ysh_slice_stride,
                          const float* shared_gate, bf16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(T, (H + kCombineThreads * 8 - 1) / (kCombineThreads * 8));
  MOE_TRACE_LAUNCH("combine_kernel", grid, dim3(kCombineThreads), 0,
                   "T=%d H=%d k=%d y=%s slices=%d shared=%d", T, H, k, y_f32 ? "f32" : "bf16",
                   nslices, y_shared ? 1 : 0);
  if (y_f32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(kCombineThreads), 0, stream,
                       static_cast<const float*>(y_perm), nslices, y_slice_stride, row_dest,
                       topk_w, T, H, k, static_cast<const float*>(y_shared), nslices_sh,
                       ysh_slice_stride, shared_gate, out);
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(kCombineThreads), 0, stream,
                       static_cast<const bf16_t*>(y_perm), 1, 0, row_dest, topk_w, T, H, k,
                       static_cast<const bf16_t*>(y_shared), 1, 0, shared_gate, out);
  return hipGetLastError();
}

}  // namespace moe
