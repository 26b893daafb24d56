// Launch unit of the tiles on mxfp8 (E4M3 codes with block scales) weights.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_mxfp8(const GemmProblem& p, int tc, hipStream_t stream) {
  const bool big = tc == kLarge || tc == kLarge128;
  if (p.gated)
    return big ? launch_cfg<GateUpLarge128_M8, bf16_t>(p, stream)
           : tc == kMid ? launch_cfg<GateUpMidM8, bf16_t>(p, stream)
                        : launch_cfg<GateUpSmallM8, bf16_t>(p, stream);
  if (p.out_f32)
    return big ? launch_cfg<DownLarge128_M8, float>(p, stream)
               : launch_cfg<DownSmallM8, float>(p, stream);
  return big ? launch_cfg<DownLarge128_M8, bf16_t>(p, stream)
             : launch_cfg<DownSmallM8, bf16_t>(p, stream);
}

}  // namespace moe
