// Backward kernels with the Mamba-style wrapper, in a translation unit of their own so that
// the two variants compile in parallel.
#include "bwd_kernel.h"

namespace sscan {

hipError_t launch_bwd_mamba(int io, int DS, int lanes, bool local_pass, const BwdParams& p, unsigned grid,
                            hipStream_t s) {
  if (io == 0) return launch_bwd_io<float, true, false>(DS, lanes, local_pass, p, grid, s);
  return launch_bwd_io<bf16_t, true, false>(DS, lanes, local_pass, p, grid, s);
}

}  // namespace sscan
