// The H-free backward sweep (states recomputed per tile from the forward's boundary
// states), with and without the Mamba-style wrapper, in a translation unit of its own.
#include "bwd_kernel.h"

namespace sscan {

hipError_t launch_bwd_hf(int io, int DS, int lanes, bool mamba, const BwdParams& p, unsigned grid, hipStream_t s) {
  if (io == 0)
    return mamba ? launch_bwd_io<float, true, true>(DS, lanes, false, p, grid, s)
                 : launch_bwd_io<float, false, true>(DS, lanes, false, p, grid, s);
  return mamba ? launch_bwd_io<bf16_t, true, true>(DS, lanes, false, p, grid, s)
               : launch_bwd_io<bf16_t, false, true>(DS, lanes, false, p, grid, s);
}

}  // namespace sscan
