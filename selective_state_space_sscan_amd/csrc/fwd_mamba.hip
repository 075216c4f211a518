// Forward kernels with the Mamba-style wrapper (softplus step, A = -exp(A_log), skip term),
// in a translation unit of their own so that the two variants compile in parallel.
#include "fwd_kernel.h"

namespace sscan {

hipError_t launch_fwd_mamba(int io, int DS, int lanes, bool local_pass, const FwdParams& p, unsigned grid,
                            hipStream_t s) {
  if (io == 0) return launch_fwd_io<float, true>(DS, lanes, local_pass, p, grid, s);
  return launch_fwd_io<bf16_t, true>(DS, lanes, local_pass, p, grid, s);
}

}  // namespace sscan
