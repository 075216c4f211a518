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

// ---- bounded buffer access --------------------------------------------------------
// A raw buffer resource covers [base, base + bytes).  Loads outside it return 0 and
// stores outside it are dropped by the hardware, so tails need no branches.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset beyond every resource this library builds
constexpr int kRsrcWord3 = 0x00020000;         // raw 32-bit data, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off, float*) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off, bf16_t*) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
}
// Load one element of type IO at byte offset `off` and widen it to fp32.
template <typename IO>
__device__ __forceinline__ float buf_load_elem(rsrc_t r, uint32_t off) {
  return buf_load_f32(r, off, static_cast<IO*>(nullptr));
}

// The raw bits of one element of type IO at byte offset `off` (a bf16 zero-extended), and
// their fp32 value.  Split so that a tile loaded ahead can stay in registers as loaded and
// be widened only where it is used: a widening next to the load makes the compiler wait
// for the load right there.
template <typename IO>
__device__ __forceinline__ uint32_t buf_load_bits(rsrc_t r, uint32_t off) {
  if constexpr (sizeof(IO) == 2) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
}
template <typename IO>
__device__ __forceinline__ float bits_to_f32(uint32_t v) {
  return sizeof(IO) == 2 ? __uint_as_float(v << 16) : __uint_as_float(v);
}

__device__ __forceinline__ void buf_store_elem(rsrc_t r, uint32_t off, float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_elem(rsrc_t r, uint32_t off, float v, bf16_t*) {
  __builtin_amdgcn_raw_buffer_store_b16(from_f32<bf16_t>(v).bits, r, off, 0, 0);
}
template <typename IO>
__device__ __forceinline__ void buf_store_io(rsrc_t r, uint32_t off, float v) {
  buf_store_elem(r, off, v, static_cast<IO*>(nullptr));
}

// Four consecutive elements of type IO at byte offset off (one 16-byte store for fp32,
// one 8-byte store for bf16); the caller keeps all four inside the row.
template <typename IO>
__device__ __forceinline__ void store4_io(rsrc_t r, uint32_t off, float4 v) {
  if constexpr (sizeof(IO) == 4) {
    __attribute__((ext_vector_type(4))) uint32_t t;
    t[0] = __float_as_uint(v.x); t[1] = __float_as_uint(v.y);
    t[2] = __float_as_uint(v.z); t[3] = __float_as_uint(v.w);
    __builtin_amdgcn_raw_buffer_store_b128(t, r, off, 0, 0);
  } else {
    __attribute__((ext_vector_type(2))) uint32_t t;
    t[0] = static_cast<uint32_t>(from_f32<bf16_t>(v.x).bits) | (static_cast<uint32_t>(from_f32<bf16_t>(v.y).bits) << 16);
    t[1] = static_cast<uint32_t>(from_f32<bf16_t>(v.z).bits) | (static_cast<uint32_t>(from_f32<bf16_t>(v.w).bits) << 16);
    __builtin_amdgcn_raw_buffer_store_b64(t, r, off, 0, 0);
  }
}

// Mamba-style step size: the softplus of a raw value in the thresholded form of the
// POPCORNBENCH page (the argument itself above 20, else log(1 + e^v)), and its
// derivative (1 above the threshold, else the logistic 1 / (1 + e^-v)).  Both use the
// hardware exp2 / log2 / reciprocal (about an ulp each): log(1 + e^v) is evaluated as
// max(v, 0) + log1p(e^-|v|), with log1p(u) = u log(w) / (w - 1), w = 1 + u (Kahan's
// formula: w - 1 is exact, and the ratio cancels the rounding of w), so the result stays
// within a few ulps for every v, including far below 0 where log(1 + e^v) ~ e^v.
constexpr float kSoftplusThreshold = 20.f;
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float softplus_th(float v) {
  const float u = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);  // e^-|v| in (0, 1]
  const float w = 1.f + u;
  const float l = (w == 1.f) ? u : __builtin_amdgcn_logf(w) * kLn2 * u * __builtin_amdgcn_rcpf(w - 1.f);
  return v > kSoftplusThreshold ? v : fmaxf(v, 0.f) + l;
}
__device__ __forceinline__ float softplus_th_grad(float v) {
  return v > kSoftplusThreshold ? 1.f : __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// K consecutive floats to global memory or LDS (16-byte stores when K is a multiple of 4).
template <int K>
__device__ __forceinline__ void store_state(float* __restrict__ p, const float (&v)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int q = 0; q < K / 4; ++q)
      reinterpret_cast<float4*>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else if constexpr (K == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
    p[0] = v[0];
  }
}

// Cache-policy operand of a buffer instruction with the non-temporal bit set: the data
// is streamed and not kept in the caches.  The materialised states are written once by the
// forward and read once by the backward, both with this policy: it raises the sustained
// HBM write rate of the forward markedly, and on the backward's side it keeps the 805 MB
// state stream from evicting the small per-step rows (x, delta, dy, gx, gdelta) from the
// last-level cache, which measured 215 -> 169 us for a memory-only kernel with the
// backward's access pattern at 8x2048x768x16.
constexpr int kNonTemporal = 2;

// K consecutive fp32 values at byte offset off.  AUX is the instruction's cache-policy
// operand (0: default).
template <int K, int AUX = 0>
__device__ __forceinline__ void buf_load_vec(rsrc_t r, uint32_t off, float (&v)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int q = 0; q < K / 4; ++q) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * q, 0, AUX);
      v[4 * q] = __uint_as_float(t[0]); v[4 * q + 1] = __uint_as_float(t[1]);
      v[4 * q + 2] = __uint_as_float(t[2]); v[4 * q + 3] = __uint_as_float(t[3]);
    }
  } else if constexpr (K == 2) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    v[0] = __uint_as_float(t[0]); v[1] = __uint_as_float(t[1]);
  } else {
    v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
  }
}

template <int K, int AUX = 0>
__device__ __forceinline__ void buf_store_vec(rsrc_t r, uint32_t off, const float (&v)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int q = 0; q < K / 4; ++q) {
      __attribute__((ext_vector_type(4))) uint32_t t;
      t[0] = __float_as_uint(v[4 * q]); t[1] = __float_as_uint(v[4 * q + 1]);
      t[2] = __float_as_uint(v[4 * q + 2]); t[3] = __float_as_uint(v[4 * q + 3]);
      __builtin_amdgcn_raw_buffer_store_b128(t, r, off + 16 * q, 0, AUX);
    }
  } else if constexpr (K == 2) {
    __attribute__((ext_vector_type(2))) uint32_t t;
    t[0] = __float_as_uint(v[0]); t[1] = __float_as_uint(v[1]);
    __builtin_amdgcn_raw_buffer_store_b64(t, r, off, 0, AUX);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, off, 0, AUX);
  }
}

// K consecutive fp32 values from LDS.
template <int K>
__device__ __forceinline__ void lds_load_vec(const float* p, float (&v)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int q = 0; q < K / 4; ++q) {
      const float4 t = reinterpret_cast<const float4*>(p)[q];
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
  } else if constexpr (K == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x; v[1] = t.y;
  } else {
    v[0] = p[0];
  }
}

// Rows of a tile that lie in [.., hi): clamp(hi - ts, 0, tb).  The value is uniform, but
// the compiler lowers this clamp to a vector med3; reading it back into a scalar register
// keeps the buffer resources built from it scalar (a vector resource would force a
// loop around every load that uses it).
__device__ __forceinline__ int tile_rows(int hi, int ts, int tb) {
  return __builtin_amdgcn_readfirstlane(max(0, min(tb, hi - ts)));
}

// ---- XCD-aware workgroup order -------------------------------------------------------
// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each XCD has its
// own L2.  Remap linear ids so that G consecutive logical tiles (which share 128-byte
// lines of x, delta and y) run on one XCD.  Bijective on [0, n).
__device__ __forceinline__ int xcd_grouped(int lin, int n, int G) {
  const int span = 8 * G;
  const int full = (n / span) * span;
  if (G <= 1 || lin >= full) return lin;
  const int base = lin - lin % span;
  const int r = lin - base;
  return base + (r % 8) * G + r / 8;
}

// v[0] + ... + v[N-1] as a balanced tree (N a power of two): the adds of each level are
// independent, and the rounding grows with log2(N) rather than N.
template <int N>
__device__ __forceinline__ float tree_sum(const float* v) {
  static_assert(N > 0 && (N & (N - 1)) == 0, "a power of two");
  if constexpr (N == 1) {
    return v[0];
  } else {
    return tree_sum<N / 2>(v) + tree_sum<N / 2>(v + N / 2);
  }
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
