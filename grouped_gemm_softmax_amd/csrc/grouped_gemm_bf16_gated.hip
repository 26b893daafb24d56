// Launch unit of the gated (gate/up + SwiGLU) tiles on bf16 weights.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_bf16_gated(const GemmProblem& p, int tc, hipStream_t stream) {
  if (tc == kSmall && p.seg[0].packed == 0) {
    const int w = rowmajor_decode_width(p, 256);
    if (w == 256) return launch_cfg<GateUpSmallRM256, bf16_t>(p, stream);
    if (w == 128) return launch_cfg<GateUpSmallRM128, bf16_t>(p, stream);
  }
  return tc == kLarge      ? launch_cfg<GateUpLarge, bf16_t>(p, stream)
         : tc == kLarge128 ? launch_cfg<GateUpLarge128, bf16_t>(p, stream)
         : tc == kMid      ? launch_cfg<GateUpMid, bf16_t>(p, stream)
                           : launch_cfg<GateUpSmall, bf16_t>(p, stream);
}

}  // namespace moe
