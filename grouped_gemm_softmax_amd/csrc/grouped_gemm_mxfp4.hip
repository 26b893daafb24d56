// Launch unit of the tiles on mxfp4 (E2M1) weight codes.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_mxfp4(const GemmProblem& p, int tc, hipStream_t stream) {
  const bool big = tc == kLarge || tc == kLarge128;
  if (p.gated)
    return big ? launch_cfg<GateUpLarge128_4, bf16_t>(p, stream)
           : tc == kMid ? launch_cfg<GateUpMid4, bf16_t>(p, stream)
                        : launch_cfg<GateUpSmall4, bf16_t>(p, stream);
  if (p.out_f32)
    return big ? launch_cfg<DownLarge128_4, float>(p, stream)
               : launch_cfg<DownSmall4, float>(p, stream);
  return big ? launch_cfg<DownLarge128_4, bf16_t>(p, stream)
             : launch_cfg<DownSmall4, bf16_t>(p, stream);
}

}  // namespace moe
