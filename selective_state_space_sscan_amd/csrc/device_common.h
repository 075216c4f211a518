// Device helpers for the gfx950 kernels: element conversion, wave-level sums, exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sscan_internal.h"

namespace sscan {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(static_cast<uint32_t>(v.bits) << 16); }

template <typename IO>
__device__ __forceinline__ IO from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) {
  return v;
}
// Round to nearest even; gfx950 lowers this to v_cvt_pk_bf16_f32.
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  return r;
}

template <typename IO>
__device__ __forceinline__ float load_f32(const IO* p) {
  return to_f32(*p);
}

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float z) { return __builtin_amdgcn_exp2f(z); }

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm:[1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G consecutive lanes (G = 1,2,4,8,16); every lane of a
// group receives the group total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<kDppQuadXor1>(v);
  if constexpr (G >= 4) v += dpp<kDppQuadXor2>(v);
  if constexpr (G >= 8) v += dpp<kDppRowHalfMirror>(v);
  if constexpr (G >= 16) v += dpp<kDppRowMirror>(v);
  return v;
}

// Lanes are grouped L to a channel, 16/L channels to a 16-lane row.  Sum over the
// channels of a row for each position within the channel: lane i receives the total
// over lanes i, i+L, i+2L, ... (mod 16) of its row.  row_ror by 8, 4, 2, 1 doubles
// the covered set each step.
template <int L>
__device__ __forceinline__ float row_channel_sum(float v) {
  if constexpr (L <= 8) v += dpp<0x128>(v);  // row_ror:8
  if constexpr (L <= 4) v += dpp<0x124>(v);  // row_ror:4
  if constexpr (L <= 2) v += dpp<0x122>(v);  // row_ror:2
  if constexpr (L <= 1) v += dpp<0x121>(v);  // row_ror:1
  return v;
}

// Sum over the four 16-lane rows of the wave (lanes i, i+16, i+32, i+48); every lane
// receives the total.
__device__ __forceinline__ float cross_row_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace sscan
