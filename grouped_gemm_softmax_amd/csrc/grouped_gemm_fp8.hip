// Launch unit of the tiles on fp8 (E4M3) weight codes.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_fp8(const GemmProblem& p, int tc, hipStream_t stream) {
  // the widening 256-row tiles leave ~7 KB of LDS for the per-group item
  // table: with more groups than fit, the 128-row tiles serve
  const int groups = p.seg[0].ngroups + (p.nseg > 1 ? p.seg[1].ngroups : 0);
  constexpr int kMaxGroups = std::min(max_groups_in_lds<GateUpLarge8>(),
                                      max_groups_in_lds<DownLarge8>());
  static_assert(kMaxGroups >= 512, "room for the item table of a 512-expert layer");
  const int tc8 = (tc == kLarge && groups > kMaxGroups) ? static_cast<int>(kLarge128) : tc;
  if (p.gated)
    return tc8 == kLarge      ? launch_cfg<GateUpLarge8, bf16_t>(p, stream)
           : tc8 == kLarge128 ? launch_cfg<GateUpLarge128_8, bf16_t>(p, stream)
           : tc8 == kMid      ? launch_cfg<GateUpMid8, bf16_t>(p, stream)
                             : launch_cfg<GateUpSmall8, bf16_t>(p, stream);
  if (p.out_f32)
    return tc8 == kLarge      ? launch_cfg<DownLarge8, float>(p, stream)
           : tc8 == kLarge128 ? launch_cfg<DownLarge128_8, float>(p, stream)
                             : launch_cfg<DownSmall8, float>(p, stream);
  return tc8 == kLarge      ? launch_cfg<DownLarge8, bf16_t>(p, stream)
         : tc8 == kLarge128 ? launch_cfg<DownLarge128_8, bf16_t>(p, stream)
                           : launch_cfg<DownSmall8, bf16_t>(p, stream);
}

}  // namespace moe
