// Backward entry points without the wrapper, and the kernel of the backward that does not
// depend on it (fixed-order reduction of the partial sums).
#include "bwd_kernel.h"

namespace sscan {
namespace {

// src[0] + src[stride] + ... + src[(n-1) stride], added in that order, with eight loads
// in flight at a time.
__device__ __forceinline__ float ordered_sum(const float* src, int64_t stride, int n) {
  float s = 0.f;
  int k = 0;
  for (; k + 8 <= n; k += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = src[(int64_t)(k + q) * stride];
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
  for (; k < n; ++k) s += src[(int64_t)k * stride];
  return s;
}

// gb, gc: add the per-workgroup partials over channel tiles in ascending tile order.
// gA: add the per-(chunk, batch row) partials in ascending order (then, for the Mamba
// wrapper, scale by A = -exp(A_log): the gradient for A_log).  gDskip: likewise.
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(const ReduceParams p) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nbc = (int64_t)p.B * p.T * p.DS;
  const int64_t nA = (int64_t)p.D * p.DS;
  if (i < nbc) {
    const int64_t per_b = (int64_t)p.T * p.DS;
    const int64_t bb = i / per_b;
    const int64_t r = i - bb * per_b;
    // partials of one element lie B*T*DS float2 apart: issue eight loads at a time (the
    // sum stays in ascending order, so the result does not depend on the batching)
    const float2* src = p.part_bc + (int64_t)bb * per_b + r;
    const int64_t stride = (int64_t)p.B * per_b;
    float sb = 0.f, sc = 0.f;
    int k = 0;
    for (; k + 8 <= p.ntiles_d; k += 8) {
      float2 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = src[(int64_t)(k + q) * stride];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        sb += v[q].x;
        sc += v[q].y;
      }
    }
    for (; k < p.ntiles_d; ++k) {
      const float2 v = src[(int64_t)k * stride];
      sb += v.x;
      sc += v.y;
    }
    p.gb[i] = sb;
    p.gc[i] = sc;
  } else if (i < nbc + nA) {
    const int64_t e = i - nbc;
    float s = ordered_sum(p.part_A + e, nA, p.chunks * p.B);
    if (p.A_log != nullptr) s *= -expf(p.A_log[e]);
    p.gA[e] = s;
  } else if (p.gD != nullptr && i < nbc + nA + p.D) {
    const int64_t e = i - nbc - nA;
    p.gD[e] = ordered_sum(p.part_D + e, p.D, p.chunks * p.B);
  }
}

}  // namespace

hipError_t launch_bwd_plain(int io, int DS, int lanes, bool local_pass, const BwdParams& p, unsigned grid,
                            hipStream_t s) {
  if (io == 0) return launch_bwd_io<float, false, false>(DS, lanes, local_pass, p, grid, s);
  return launch_bwd_io<bf16_t, false, false>(DS, lanes, local_pass, p, grid, s);
}

hipError_t launch_bwd(int io, int DS, int lanes, bool local_pass, bool mamba, const BwdParams& p, unsigned grid,
                      hipStream_t s) {
  return mamba ? launch_bwd_mamba(io, DS, lanes, local_pass, p, grid, s)
               : launch_bwd_plain(io, DS, lanes, local_pass, p, grid, s);
}

hipError_t launch_bwd_reduce(const ReduceParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.T * p.DS + (int64_t)p.D * p.DS + (p.gD != nullptr ? p.D : 0);
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace sscan
