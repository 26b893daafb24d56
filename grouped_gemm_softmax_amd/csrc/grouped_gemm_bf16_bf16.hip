// Launch unit of the plain tiles on bf16 weights with bf16 output.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_bf16_plain_bf16(const GemmProblem& p, int tc, hipStream_t stream) {
  if (tc == kSmall && p.seg[0].packed == 0 && rowmajor_decode_width(p, 128) == 128)
    return launch_cfg<DownSmallRM, bf16_t>(p, stream);
  return tc == kLarge      ? launch_cfg<DownLarge, bf16_t>(p, stream)
         : tc == kLarge128 ? launch_cfg<DownLarge128, bf16_t>(p, stream)
                           : launch_cfg<DownSmall, bf16_t>(p, stream);
}

}  // namespace moe
