// Launch unit of the plain tiles on bf16 weights with fp32 output.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_bf16_plain_f32(const GemmProblem& p, int tc, hipStream_t stream) {
  if (tc == kSmall && p.seg[0].packed == 0 && rowmajor_decode_width(p, 128) == 128)
    return launch_cfg<DownSmallRM, float>(p, stream);
  return tc == kLarge      ? launch_cfg<DownLarge, float>(p, stream)
         : tc == kLarge128 ? launch_cfg<DownLarge128, float>(p, stream)
                           : launch_cfg<DownSmall, float>(p, stream);
}

}  // namespace moe
