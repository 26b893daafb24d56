// Launch unit of the tiles on mxfp8 (E4M3 codes with block scales) weights.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_mxfp8(const GemmProblem& p, int tc, hipStream_t stream) {
  // the widening 256-row tiles leave ~2 KB of LDS for the per-group item
  // table: with more groups than fit, the 128-row tiles serve
  const int groups = p.seg[0].ngroups + (p.nseg > 1 ? p.seg[1].ngroups : 0);
  constexpr int kMaxGroups = std::min(max_groups_in_lds<GateUpLargeM8>(),
                                      max_groups_in_lds<DownLargeM8>());
  static_assert(kMaxGroups >= 128, "room for the item table of a 128-expert layer");
  const int tcm = (tc == kLarge && groups > kMaxGroups) ? static_cast<int>(kLarge128) : tc;
  if (p.gated)
    return tcm == kLarge      ? launch_cfg<GateUpLargeM8, bf16_t>(p, stream)
           : tcm == kLarge128 ? launch_cfg<GateUpLarge128_M8, bf16_t>(p, stream)
           : tcm == kMid      ? launch_cfg<GateUpMidM8, bf16_t>(p, stream)
           : p.rows_hint <= 4 ? launch_cfg<GateUpSmallM8W, bf16_t>(p, stream)
                              : launch_cfg<GateUpSmallM8, bf16_t>(p, stream);
  if (p.out_f32)
    return tcm == kLarge      ? launch_cfg<DownLargeM8, float>(p, stream)
           : tcm == kLarge128 ? launch_cfg<DownLarge128_M8, float>(p, stream)
           : p.rows_hint <= 4 ? launch_cfg<DownSmallM8W, float>(p, stream)
                              : launch_cfg<DownSmallM8, float>(p, stream);
  return tcm == kLarge      ? launch_cfg<DownLargeM8, bf16_t>(p, stream)
         : tcm == kLarge128 ? launch_cfg<DownLarge128_M8, bf16_t>(p, stream)
                            : launch_cfg<DownSmallM8, bf16_t>(p, stream);
}

}  // namespace moe
