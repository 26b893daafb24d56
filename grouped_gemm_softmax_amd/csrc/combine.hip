// Combine / un-permute of the MoE expert layer:
//   out[t,c] = bf16( sum_{j<k} w[t,j] * y_perm[row_dest[t,j], c]
//                    + s_t * y_shared[t,c] )
// with fp32 accumulation in ascending j and the shared term added last.
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

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const bf16_t* __restrict__ y_perm, const int32_t* __restrict__ row_dest,
    const float* __restrict__ topk_w, int T, int H, int k,
    const bf16_t* __restrict__ y_shared, const float* __restrict__ shared_gate,
    bf16_t* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int s_row[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int64_t A = static_cast<int64_t>(T) * k;
  if (threadIdx.x < k) {
    int p = row_dest[static_cast<int64_t>(t) * k + threadIdx.x];
    p = p < 0 ? 0 : (p >= A ? static_cast<int>(A - 1) : p);  // stay in bounds
    s_row[threadIdx.x] = p;
    s_w[threadIdx.x] = topk_w[static_cast<int64_t>(t) * k + threadIdx.x];
  }
  __syncthreads();
  float s = 1.0f;
  if (y_shared && shared_gate) s = 1.0f / (1.0f + expf(-shared_gate[t]));
  for (int c = threadIdx.x * 8; c < H; c += kCombineThreads * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(
          y_perm + static_cast<int64_t>(s_row[j]) * H + c);
      const float w = s_w[j];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w * bf16_to_f32(static_cast<bf16_t>(u[q] & 0xffffu));
        acc[2 * q + 1] += w * bf16_to_f32(static_cast<bf16_t>(u[q] >> 16));
      }
    }
    if (y_shared) {
      const uint4 v = *reinterpret_cast<const uint4*>(
          y_shared + static_cast<int64_t>(t) * H + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += s * bf16_to_f32(static_cast<bf16_t>(u[q] & 0xffffu));
        acc[2 * q + 1] += s * bf16_to_f32(static_cast<bf16_t>(u[q] >> 16));
      }
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

hipError_t launch_combine(const bf16_t* y_perm, const int32_t* row_dest,
                          const float* topk_w, int T, int H, int k,
                          const bf16_t* y_shared, const float* shared_gate,
                          bf16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(kCombineThreads), 0, stream,
                     y_perm, row_dest, topk_w, T, H, k, y_shared, shared_gate,
                     out);
  return hipGetLastError();
}

}  // namespace moe
