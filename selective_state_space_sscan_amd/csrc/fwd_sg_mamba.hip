// State-group forward with the Mamba-style wrapper fused (softplus step, A = -exp(A_log),
// skip term).
#include "fwd_sg_kernel.h"

namespace sscan {

hipError_t launch_fwd_sg_mamba(int io, int DS, int cw, bool local_pass, const FwdParams& p, unsigned blocks,
                               hipStream_t s) {
  return launch_fwd_sg_io<true>(io, DS, cw, local_pass, p, blocks, s);
}

}  // namespace sscan
