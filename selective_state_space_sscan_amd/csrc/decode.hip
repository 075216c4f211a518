// One-token decode step for gfx950.
//
// A single step of the recurrence ("pssa-100m/pssa_kernels.py" page, module docstring)
// applied to a state kept in device memory between calls, as the "ruDNN KDA chunk.rs"
// page does for one token (chunk_kda: a fused recurrent kernel on the resident state
// instead of the chunked path, inputs never mutated):
//   state'[b,d,n] = exp(delta[b,d] A[d,n]) state[b,d,n] + delta[b,d] x[b,d] b[b,n]
//   y[b,d]        = sum_n state'[b,d,n] c[b,n]
// The arithmetic is the forward kernel's for one step: exp2 of delta * (A log2 e), the
// injection (delta x) b, one fma, so a decode step and a one-step sscan_fwd agree bitwise
// up to the order of the readout sum.
//
// Latency-oriented layout: one lane per (b, d, n) state, so that a batch of B*D channels
// spreads over B*D*DS lanes; the readout is a DPP sum over the DS consecutive lanes of a
// channel.  Every access is a plain element load or store, and the state is read and then
// written by the same lane, so the output may be the input state itself.
#include "device_common.h"

namespace sscan {
namespace {

template <typename IO>
__device__ __forceinline__ float load_io(const void* p, int64_t i) {
  return to_f32(static_cast<const IO*>(p)[i]);
}

template <typename IO, int DS>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeParams p) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // state index over (b, d, n)
  const int64_t total = (int64_t)p.B * p.D * DS;
  const bool valid = i < total;
  const int n = static_cast<int>(i % DS);
  const int64_t bd = valid ? i / DS : 0;
  const int d = static_cast<int>(bd % p.D);
  const int64_t bb = bd / p.D;
  float h = 0.f, cv = 0.f;
  if (valid) {
    const float dl = load_io<IO>(p.delta, bb * p.x_bs + d);
    const float xv = load_io<IO>(p.x, bb * p.x_bs + d);
    const float bv = load_io<IO>(p.b, bb * p.bc_bs + n);
    cv = load_io<IO>(p.c, bb * p.bc_bs + n);
    const float a = exp2_hw(dl * (p.A[(int64_t)d * DS + n] * kLog2e));
    h = fmaf(a, p.state_in[i], (dl * xv) * bv);
    p.state_out[i] = h;
  }
  // every lane of the channel takes part in the sum, valid or not
  const float yv = group_sum<DS>(h * cv);
  if (valid && n == 0) static_cast<IO*>(p.y)[bb * p.y_bs + d] = from_f32<IO>(yv);
}

template <typename IO>
hipError_t launch_decode_io(int DS, const DecodeParams& p, unsigned blocks, hipStream_t s) {
  switch (DS) {
    case 1: hipLaunchKernelGGL((decode_kernel<IO, 1>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<IO, 2>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<IO, 4>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<IO, 8>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    case 16: hipLaunchKernelGGL((decode_kernel<IO, 16>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int io, int DS, const DecodeParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.D * DS;
  if (total <= 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((total + kThreads - 1) / kThreads);
  if (io == 0) return launch_decode_io<float>(DS, p, blocks, s);
  return launch_decode_io<bf16_t>(DS, p, blocks, s);
}

}  // namespace sscan
