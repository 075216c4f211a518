// State-group forward entry points without the wrapper, the b/c packing kernel, and the
// dispatch between the two instantiations.
#include "fwd_sg_kernel.h"

namespace sscan {

hipError_t launch_fwd_sg_plain(int io, int DS, int cw, bool local_pass, const FwdParams& p, unsigned blocks,
                               hipStream_t s) {
  return launch_fwd_sg_io<false>(io, DS, cw, local_pass, p, blocks, s);
}

hipError_t launch_fwd_sg(int io, int DS, int cw, bool local_pass, bool mamba, const FwdParams& p, unsigned blocks,
                         hipStream_t s) {
  return mamba ? launch_fwd_sg_mamba(io, DS, cw, local_pass, p, blocks, s)
               : launch_fwd_sg_plain(io, DS, cw, local_pass, p, blocks, s);
}

hipError_t launch_bc_pack(int io, int DS, const FwdParams& p, hipStream_t s) {
  switch (DS) {
    case 4: return io == 0 ? launch_bc_pack_t<float, 4, kSgK>(p, s) : launch_bc_pack_t<bf16_t, 4, kSgK>(p, s);
    case 8: return io == 0 ? launch_bc_pack_t<float, 8, kSgK>(p, s) : launch_bc_pack_t<bf16_t, 8, kSgK>(p, s);
    case 16: return io == 0 ? launch_bc_pack_t<float, 16, kSgK>(p, s) : launch_bc_pack_t<bf16_t, 16, kSgK>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sscan
