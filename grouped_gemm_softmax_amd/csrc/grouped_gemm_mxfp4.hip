// Launch unit of the tiles on mxfp4 (E2M1) weight codes.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_mxfp4(const GemmProblem& p, int tc, hipStream_t stream) {
  // the widening tiles leave ~10 KB of LDS for the per-group item table:
  // with more groups than fit, the 128-row tiles that decode per fragment
  const int groups = p.seg[0].ngroups + (p.nseg > 1 ? p.seg[1].ngroups : 0);
  constexpr int kMaxGroups = std::min(max_groups_in_lds<GateUpLarge_4W>(),
                                      max_groups_in_lds<DownLarge_4W>());
  static_assert(kMaxGroups >= 512, "room for the item table of a 512-expert layer");
  const bool big = tc == kLarge || tc == kLarge128;
  const bool wide = big && groups <= kMaxGroups;
  if (p.gated)
    return wide  ? launch_cfg<GateUpLarge_4W, bf16_t>(p, stream)
           : big ? launch_cfg<GateUpLarge128_4, bf16_t>(p, stream)
           : tc == kMid          ? launch_cfg<GateUpMid4, bf16_t>(p, stream)
           : p.rows_hint <= 4    ? launch_cfg<GateUpSmall4W, bf16_t>(p, stream)
                                 : launch_cfg<GateUpSmall4, bf16_t>(p, stream);
  if (p.out_f32)
    return wide  ? launch_cfg<DownLarge_4W, float>(p, stream)
           : big ? launch_cfg<DownLarge128_4, float>(p, stream)
           : p.rows_hint <= 4 ? launch_cfg<DownSmall4W, float>(p, stream)
                              : launch_cfg<DownSmall4, float>(p, stream);
  return wide  ? launch_cfg<DownLarge_4W, bf16_t>(p, stream)
         : big ? launch_cfg<DownLarge128_4, bf16_t>(p, stream)
               : launch_cfg<DownSmall4, bf16_t>(p, stream);
}

}  // namespace moe
