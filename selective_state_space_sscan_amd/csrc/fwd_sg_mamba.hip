// State-group forward with the Mamba-style wrapper fused (softplus step, A = -exp(A_log),
// skip term).
#include "fwd_sg_kernel.h"

namespace sscan {

hipError_t launch_fwd_sg_mamba(int io, int DS, bool local_pass, const FwdParams& p, unsigned blocks, hipStream_t s) {
  switch (DS) {
    case 4:
      return io == 0 ? launch_fwd_sg_t<float, 4, kSgK, true>(local_pass, p, blocks, s)
                     : launch_fwd_sg_t<bf16_t, 4, kSgK, true>(local_pass, p, blocks, s);
    case 8:
      return io == 0 ? launch_fwd_sg_t<float, 8, kSgK, true>(local_pass, p, blocks, s)
                     : launch_fwd_sg_t<bf16_t, 8, kSgK, true>(local_pass, p, blocks, s);
    case 16:
      return io == 0 ? launch_fwd_sg_t<float, 16, kSgK, true>(local_pass, p, blocks, s)
                     : launch_fwd_sg_t<bf16_t, 16, kSgK, true>(local_pass, p, blocks, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace sscan
