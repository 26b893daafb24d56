// Launch unit of the register-streaming decode gate/up kernel.
#include "grouped_gemm_kernel.h"

namespace moe {

hipError_t launch_rs(const GemmProblem& p, hipStream_t stream) {
  return p.seg[0].packed == 2 ? launch_rs_gateup<8>(p, stream)
                              : launch_rs_gateup<16>(p, stream);
}

}  // namespace moe
