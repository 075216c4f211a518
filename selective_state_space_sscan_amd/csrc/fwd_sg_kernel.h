// Forward selective scan, state-group layout, for gfx950 (the forward without the
// materialised states H: y, hT, the two-level scan's local pass, and the H-free path's
// boundary states).
//
// Recurrence ("pssa-100m/pssa_kernels.py" page, module docstring and scan_fwd):
//   h_t = exp(delta_t * A) * h_{t-1} + delta_t * b_t * x_t,   y_t = <h_t, c_t>.
//
// Work decomposition.  A workgroup owns one batch row and 64 consecutive channels: lane
// l of every wave is channel d0 + l, and wave w holds the K states n = wK .. wK+K-1 of
// all 64 channels (NW = DS/K waves).  Within a wave, b_t and c_t of its K states are the
// same for every lane.  A small packing kernel lays them out per (batch row, state
// group) as fp32, contiguous over steps; each 16-lane row of a wave loads the same block
// of them (lane p holds floats 4p .. 4p+3 of a 64-float block), and every use reads the
// value it needs from the lane that holds it with a DPP row broadcast folded into the
// multiply (row_newbcast), so b and c cost neither LDS traffic nor extra instructions.
// The workgroup stages (delta, delta*x) of a tile once in LDS (each element converted by
// one thread, the softplus of the wrapper applied there), and every wave reads its lane's
// channel from it.  Each wave leaves its partial sum over its K states of h * c per (step,
// channel) in LDS, and after the tile the workgroup adds the NW partials and stores y
// coalesced.  Per (step, state) a lane does one v_exp_f32 and four fp32 operations, with
// no other cross-lane traffic: about 5.6 instructions per state against 7 for the
// lane-split forward, which spends 1.5 on DPP sums over a channel's lanes.
//
// Steps past the end of the chunk load delta = 0 and b = c = 0 (buffer range checks),
// which leaves the state bit-for-bit unchanged.
#pragma once
#include "device_common.h"

namespace sscan {
namespace {

// Packed b/c: element (bb, w, t, e) at ((bb * NW + w) * tpad + t) * 2K + e holds
// b[bb, t, wK + e] for e < K and c[bb, t, wK + e - K] otherwise; zero for t >= T.  One
// thread per (bb, w, t) writes its 2K floats together; neighbouring threads take
// neighbouring steps, so the stores are contiguous.
template <typename IO, int DS, int K>
__global__ __launch_bounds__(kThreads) void bc_pack_kernel(const FwdParams p) {
  constexpr int NW = DS / K;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)p.B * NW * p.tpad;
  if (i >= total) return;
  const int t = static_cast<int>(i % p.tpad);
  const int64_t r = i / p.tpad;
  const int w = static_cast<int>(r % NW);
  const int64_t bb = r / NW;
  float v[2 * K];
#pragma unroll
  for (int e = 0; e < 2 * K; ++e) v[e] = 0.f;
  if (t < p.T) {
    const IO* b = static_cast<const IO*>(p.b) + bb * p.bc_bs + (int64_t)t * DS + w * K;
    const IO* c = static_cast<const IO*>(p.c) + bb * p.bc_bs + (int64_t)t * DS + w * K;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      v[e] = to_f32(b[e]);
      v[K + e] = to_f32(c[e]);
    }
  }
  store_state<2 * K>(p.bcp + i * 2 * K, v);
}

// Lane LANE of v's 16-lane row, for every lane of the row (DPP row_newbcast); the
// compiler folds it into the consuming multiply.
__device__ __forceinline__ float row_bcast(float v, int lane) {
  switch (lane) {
    case 0: return dpp<0x150>(v);  case 1: return dpp<0x151>(v);  case 2: return dpp<0x152>(v);
    case 3: return dpp<0x153>(v);  case 4: return dpp<0x154>(v);  case 5: return dpp<0x155>(v);
    case 6: return dpp<0x156>(v);  case 7: return dpp<0x157>(v);  case 8: return dpp<0x158>(v);
    case 9: return dpp<0x159>(v);  case 10: return dpp<0x15A>(v); case 11: return dpp<0x15B>(v);
    case 12: return dpp<0x15C>(v); case 13: return dpp<0x15D>(v); case 14: return dpp<0x15E>(v);
    default: return dpp<0x15F>(v);
  }
}

// acc += (lane LANE of c's row) * h as one v_fmac_f32 with a DPP row broadcast of c (the
// compiler does not fold a broadcast into an fma).  FIRST: acc = that product instead,
// after two wait states, which a DPP read of a register written by the previous vector
// instruction requires.
template <int LANE, bool FIRST>
__device__ __forceinline__ void fmac_bcast(float& acc, float c, float h) {
  if constexpr (FIRST) {
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "=v"(acc) : "v"(c), "v"(h), "i"(LANE));
  } else {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc) : "v"(c), "v"(h), "i"(LANE));
  }
}

// fmac_bcast with the lane and FIRST given at run time; every call site passes values
// that are constant once the step loops are unrolled, so the switch folds away.
__device__ __forceinline__ void fmac_bcast_rt(float& acc, float c, float h, int lane, bool first) {
#define SSCAN_FMAC_CASE(L) \
  case L:                  \
    if (first)             \
      fmac_bcast<L, true>(acc, c, h); \
    else                   \
      fmac_bcast<L, false>(acc, c, h); \
    break;
  switch (lane) {
    SSCAN_FMAC_CASE(0) SSCAN_FMAC_CASE(1) SSCAN_FMAC_CASE(2) SSCAN_FMAC_CASE(3)
    SSCAN_FMAC_CASE(4) SSCAN_FMAC_CASE(5) SSCAN_FMAC_CASE(6) SSCAN_FMAC_CASE(7)
    SSCAN_FMAC_CASE(8) SSCAN_FMAC_CASE(9) SSCAN_FMAC_CASE(10) SSCAN_FMAC_CASE(11)
    SSCAN_FMAC_CASE(12) SSCAN_FMAC_CASE(13) SSCAN_FMAC_CASE(14) default: SSCAN_FMAC_CASE(15)
  }
#undef SSCAN_FMAC_CASE
}

// MODE: 0 the two-level scan's local pass (only the chunk pair leaves the kernel), 1 y and
// hT, 2 y, hT and the H-free path's boundary states.
template <typename IO, int DS, int K, int MODE, bool MAMBA>
__global__ __launch_bounds__(64 * (DS / K)) void fwd_sg_kernel(const FwdParams p) {
  constexpr bool LOCAL = MODE == 0;
  constexpr int NW = DS / K;
  constexpr int NT = 64 * NW;
  constexpr int TB = kSgTile;
  constexpr int S = 4;  // steps per batch
  constexpr int E2 = 2 * K;
  constexpr uint32_t ES = sizeof(IO);
  constexpr int TILE = TB * 64;     // (step, channel) elements of a tile
  constexpr int PER = TILE / NT;    // elements each thread stages
  constexpr int GROUPS = TB * 16;   // (step, 4-channel group) items of a tile's readout
  constexpr int NB = TB * E2 / 64;  // 64-float blocks of packed b/c per tile
  static_assert(TILE % NT == 0 && TB % S == 0 && kCkptSteps % S == 0 && (TB * E2) % 64 == 0, "tile shape");

  // (delta, delta*x) at [step*64 + channel]; with the wrapper (delta, x), so that the
  // first wave can add the skip term Dskip * x to its partial sums
  __shared__ float2 s_dw[TILE];
  __shared__ float4 s_y[LOCAL ? 1 : NW * TB * 16];  // [w][step][channel / 4]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lin = blockIdx.x;
  const int dtile = lin % p.ntiles_d;
  const int rest = lin / p.ntiles_d;
  const int bb = rest % p.B;
  const int chunk = rest / p.B;
  const int D = p.D;
  const int d0 = dtile * 64;
  const int d = d0 + lane;
  const bool dvalid = d < D;
  const int t_begin = chunk * p.chunk_len;
  const int t_end = min(p.T, t_begin + p.chunk_len);

  const IO* xrow = static_cast<const IO*>(p.x) + (int64_t)bb * p.x_bs;
  const IO* drow = static_cast<const IO*>(p.delta) + (int64_t)bb * p.x_bs;
  IO* yrow = static_cast<IO*>(p.y) + (int64_t)bb * p.y_bs;
  // this wave's packed b/c row; lane p of each 16-lane row loads floats 4p .. 4p+3 of
  // every 64-float block
  const rsrc_t rBC = make_rsrc(p.bcp + ((int64_t)bb * NW + w) * p.tpad * E2, static_cast<uint32_t>(p.tpad) * E2 * 4u);
  const uint32_t bclane = static_cast<uint32_t>(lane & 15) * 16u;

  const int64_t nstate = (int64_t)p.B * D * DS;
  const int64_t soff = ((int64_t)bb * D + d) * DS + w * K;  // this lane's states in (B,D,DS)

  float A2[K], h[K];
  if (dvalid) {
    lds_load_vec<K>(p.A + (int64_t)d * DS + w * K, A2);
#pragma unroll
    for (int i = 0; i < K; ++i) A2[i] = (MAMBA ? -expf(A2[i]) : A2[i]) * kLog2e;
    if (LOCAL || (chunk == 0 && p.h0 == nullptr)) {
#pragma unroll
      for (int i = 0; i < K; ++i) h[i] = 0.f;
    } else if (chunk == 0) {
      lds_load_vec<K>(p.h0 + soff, h);
    } else {
      lds_load_vec<K>(p.hin + (int64_t)(chunk - 1) * nstate + soff, h);
    }
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) { A2[i] = 0.f; h[i] = 0.f; }
  }
  double dsum = 0.0;  // local pass: sum of delta over the chunk

  // staged elements: idx = tid + e*NT is (step idx / 64, channel idx % 64); columns past D
  // are forced out of range, rows past the chunk fall outside the resource
  uint32_t xoff[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid + e * NT;
    const int dd = d0 + (idx & 63);
    xoff[e] = dd < D ? static_cast<uint32_t>((idx >> 6) * D + dd) * ES : kOutOfRange;
  }
  // the skip weight of this lane's channel (used by the first wave)
  const float dskip = (MAMBA && !LOCAL && w == 0 && p.Dskip != nullptr && dvalid) ? p.Dskip[d] : 0.f;
  float rx[PER], rd[PER];
  int pend_rows = 0;
  auto load_tile = [&](int ts) {
    const int rows = tile_rows(t_end, ts, TB);
    pend_rows = rows;
    const rsrc_t rX = make_rsrc(xrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rD = make_rsrc(drow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      rx[e] = buf_load_elem<IO>(rX, xoff[e]);
      rd[e] = buf_load_elem<IO>(rD, xoff[e]);
    }
  };
  auto store_tile = [&]() {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      // padded steps and channels keep delta = 0 (a multiply by a 0/1 mask: a select
      // lets the compiler branch around the softplus)
      const float keep = (((tid + e * NT) >> 6) < pend_rows && xoff[e] != kOutOfRange) ? 1.f : 0.f;
      const float dl = MAMBA ? softplus_th(rd[e]) * keep : rd[e];
      s_dw[tid + e * NT] = make_float2(dl, MAMBA ? rx[e] : dl * rx[e]);
    }
  };
  float bcv[NB][4], bcw[NB][4];  // b/c blocks of this tile and of the next one
  auto load_bc = [&](int ts, float (&dst)[NB][4]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rBC, static_cast<uint32_t>(ts) * E2 * 4u + k * 256u + bclane, 0, 0);
      dst[k][0] = __uint_as_float(t[0]); dst[k][1] = __uint_as_float(t[1]);
      dst[k][2] = __uint_as_float(t[2]); dst[k][3] = __uint_as_float(t[3]);
    }
  };

  const int nsteps_total = t_end - t_begin;
  const int ntiles = nsteps_total > 0 ? (nsteps_total + TB - 1) / TB : 0;
  if (ntiles > 0) {
    load_tile(t_begin);
    load_bc(t_begin, bcw);
    store_tile();
  }

  for (int it = 0; it < ntiles; ++it) {
    const int ts = t_begin + it * TB;
    const int rows = min(TB, t_end - ts);
    __syncthreads();  // this tile's inputs are in LDS; the previous tile's partial sums are read
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q) bcv[k][q] = bcw[k][q];
    load_tile(ts + TB);  // zeros past the end of the chunk
    load_bc(ts + TB, bcw);

#pragma unroll
    for (int s0 = 0; s0 < TB; s0 += S) {
      if constexpr (MODE == 2) {
        if (dvalid && ts + s0 < t_end && ((ts + s0) % kCkptSteps) == 0)
          store_state<K>(p.hck + (((int64_t)bb * p.nck + (ts + s0) / kCkptSteps) * D + d) * DS + w * K, h);
      }
      float2 dw[S];
      float xs[S];  // with the wrapper: x of the step (dw[s].y becomes delta * x)
#pragma unroll
      for (int s = 0; s < S; ++s) {
        dw[s] = s_dw[(s0 + s) * 64 + lane];
        xs[s] = dw[s].y;
        if constexpr (MAMBA) dw[s].y *= dw[s].x;
      }
      (void)xs;
      float a[S][K], u[S][K];
#pragma unroll
      for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const int q = (s0 + s) * E2 + i;  // b_i of this step in the tile's packed floats
          a[s][i] = exp2_hw(dw[s].x * A2[i]);
          u[s][i] = dw[s].y * row_bcast(bcv[q / 64][q % 4], (q % 64) / 4);
        }
      }
#pragma unroll
      for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int i = 0; i < K; ++i) {
          h[i] = fmaf(a[s][i], h[i], u[s][i]);
          a[s][i] = h[i];
        }
      }
      if constexpr (LOCAL) {
        float dls[S];
#pragma unroll
        for (int s = 0; s < S; ++s) dls[s] = dw[s].x;
        dsum += static_cast<double>(tree_sum<S>(dls));
      } else {
        float* sy = reinterpret_cast<float*>(s_y) + (w * TB + s0) * 64 + lane;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          float yp;
#pragma unroll
          for (int i = 0; i < K; ++i) {
            const int q = (s0 + s) * E2 + K + i;  // c_i
            fmac_bcast_rt(yp, bcv[q / 64][q % 4], a[s][i], (q % 64) / 4, i == 0);
          }
          if constexpr (MAMBA) yp = fmaf(dskip, xs[s], yp);  // the skip term (dskip = 0 past the first wave)
          sy[s * 64] = yp;
        }
      }
    }

    __syncthreads();  // every wave is done with this tile's inputs and has left its partials
    if constexpr (!LOCAL) {
      const rsrc_t rY = make_rsrc(yrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
#pragma unroll
      for (int g0 = 0; g0 < GROUPS; g0 += NT) {
        // every thread stores (out of range when it has no group), so the number of
        // stores in flight does not depend on the thread
        const int g = g0 + tid;
        const bool act = GROUPS % NT == 0 || g < GROUPS;
        const int s = act ? (g >> 4) : 0;
        const int c4 = g & 15;
        float4 acc = s_y[s * 16 + c4];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
          const float4 v = s_y[(ww * TB + s) * 16 + c4];
          acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        // D is a multiple of 4 for this kernel: a group is wholly inside or outside
        const int dd = d0 + 4 * c4;
        store4_io<IO>(rY, (act && dd < D) ? static_cast<uint32_t>(s * D + dd) * ES : kOutOfRange, acc);
      }
    }
    store_tile();  // the next tile's inputs (zeros past the end of the chunk)
  }

  if (!dvalid) return;
  if constexpr (LOCAL) {
    float2* pr = p.pairs + (int64_t)chunk * nstate + soff;
#pragma unroll
    for (int i = 0; i < K; ++i)
      pr[i] = make_float2(exp2_hw(static_cast<float>(static_cast<double>(A2[i]) * dsum)), h[i]);
  } else {
    if (p.hT != nullptr && chunk == p.chunks - 1) store_state<K>(p.hT + soff, h);
  }
}

template <typename IO, int DS, int K>
hipError_t launch_bc_pack_t(const FwdParams& p, hipStream_t s) {
  constexpr int NW = DS / K;
  const int64_t npack = (int64_t)p.B * NW * p.tpad;
  if (npack > 0)
    hipLaunchKernelGGL((bc_pack_kernel<IO, DS, K>), dim3((unsigned)((npack + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int DS, int K, bool MAMBA>
hipError_t launch_fwd_sg_t(bool local_pass, const FwdParams& p, unsigned blocks, hipStream_t s) {
  constexpr int NW = DS / K;
  if (local_pass)
    hipLaunchKernelGGL((fwd_sg_kernel<IO, DS, K, 0, MAMBA>), dim3(blocks), dim3(64 * NW), 0, s, p);
  else if (p.hck != nullptr)
    hipLaunchKernelGGL((fwd_sg_kernel<IO, DS, K, 2, MAMBA>), dim3(blocks), dim3(64 * NW), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_sg_kernel<IO, DS, K, 1, MAMBA>), dim3(blocks), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace sscan
