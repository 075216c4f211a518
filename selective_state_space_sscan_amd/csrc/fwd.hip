// Forward entry points without the wrapper, and the small fill kernel.
#include "fwd_kernel.h"

namespace sscan {
namespace {

__global__ __launch_bounds__(kThreads) void fill_kernel(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) dst[i] = src != nullptr ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_fwd_plain(int io, int DS, int lanes, bool local_pass, const FwdParams& p, unsigned grid,
                            hipStream_t s) {
  if (io == 0) return launch_fwd_io<float, false>(DS, lanes, local_pass, p, grid, s);
  return launch_fwd_io<bf16_t, false>(DS, lanes, local_pass, p, grid, s);
}

hipError_t launch_fwd(int io, int DS, int lanes, bool local_pass, bool mamba, const FwdParams& p, unsigned grid,
                      hipStream_t s) {
  return mamba ? launch_fwd_mamba(io, DS, lanes, local_pass, p, grid, s)
               : launch_fwd_plain(io, DS, lanes, local_pass, p, grid, s);
}

hipError_t launch_fill(float* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, dst, nullptr, n);
  return hipGetLastError();
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace sscan
