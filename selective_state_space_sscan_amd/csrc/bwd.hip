// Backward selective scan kernels for gfx950.
//
// Reverse adjoint sweep over the materialised states ("pssa-100m/pssa_kernels.py"
// page, scan_bwd), for L = sum(dy*y) + sum(dhT*hT).  With G the adjoint carried into
// step t from step t+1 (G = dhT, or 0, before the last step) and a_t = exp(delta_t A):
//   g        = dy_t * c_t + G
//   gx_t     = delta_t * sum_n g b_t
//   gdelta_t = sum_n A (a_t g) h_{t-1} + x_t * sum_n g b_t
//   gb_t    += g * delta_t x_t            (summed over channels)
//   gc_t    += dy_t * h_t                 (summed over channels)
//   gA      += delta_t (a_t g) h_{t-1}    (summed over batch rows and steps)
//   G        = a_t g                      (so gh0 is the carry left after step 0)
// a_t is formed once per (step, state): the page recomputes exp(delta_{t+1} A) for the
// carry, which is the a_{t+1} the previous step already formed.
//
// Work decomposition.  As in the forward, a 256-thread workgroup owns one batch row
// and CPW = 256/L channels, L lanes per channel, K = DS/L states per lane.  The
// workgroup walks tiles of TB steps from the end of the sequence to the start; the
// x / delta / dy tiles and the b / c rows are loaded cooperatively one tile ahead and
// parked in LDS as fp32.  Each lane reads its own states H_{t-1} straight from HBM
// (coalesced: the lanes of a wave cover consecutive (channel, state) addresses) a
// sub-block ahead, and keeps H_t from the previous step.  Sums over a channel's states
// use DPP; sums over channels use DPP row rotations, the gfx950 row-swap permutes and
// one LDS slot per wave, and each workgroup writes one (gb, gc) partial per (step,
// state) and one gA partial per (batch row, channel, state).  A second kernel adds the
// partials in a fixed order: no float atomics, results are bitwise reproducible.
#include "device_common.h"

namespace sscan {
namespace {

template <int K>
__device__ __forceinline__ void load_k(const float* __restrict__ p, float (&v)[K]) {
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

// Steps of H per prefetch sub-block: at most 32 floats per lane, and at least two
// sub-blocks per tile so the two buffers alternate at compile-time positions.
template <int K, int TB>
__host__ __device__ constexpr int h_block_steps() {
  return (32 / K) < (TB / 2) ? (32 / K) : (TB / 2);
}

template <typename IO, int DS, int L>
__global__ __launch_bounds__(kThreads) void bwd_kernel(const BwdParams p) {
  constexpr int K = DS / L;
  constexpr int CPW = kThreads / L;
  constexpr int TB = bwd_tile_steps(L);
  constexpr int TILE = TB * CPW;
  constexpr int PER = TILE / kThreads;
  constexpr int BC = TB * DS;
  constexpr int PER_BC = (BC + kThreads - 1) / kThreads;
  constexpr int NWAVE = kThreads / 64;
  constexpr int HB = h_block_steps<K, TB>();
  constexpr int NSUB = TB / HB;
  static_assert(TILE % kThreads == 0 && TB % HB == 0, "tile shape");
  static_assert(NSUB % 2 == 0, "sub-blocks per tile must be even");

  __shared__ float4 s_in[TILE];         // (delta, x, dy, delta*x) at [step*CPW + channel]
  __shared__ float s_b[BC];
  __shared__ float s_c[BC];
  __shared__ float2 s_gxd[TILE];        // (gx, gdelta)
  __shared__ float2 s_red[NWAVE * BC];  // per-wave (gb, gc) sums at [wave*BC + step*DS + n]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ch = tid / L;
  const int j = tid % L;
  const int d0 = blockIdx.x * CPW;
  const int bb = blockIdx.y;
  const int D = p.D;
  const int T = p.T;
  const int d = d0 + ch;
  const bool dvalid = d < D;

  const IO* __restrict__ xg = static_cast<const IO*>(p.x) + (int64_t)bb * p.x_bs;
  const IO* __restrict__ dg = static_cast<const IO*>(p.delta) + (int64_t)bb * p.x_bs;
  const IO* __restrict__ yg = static_cast<const IO*>(p.dy) + (int64_t)bb * p.x_bs;
  const IO* __restrict__ bg = static_cast<const IO*>(p.b) + (int64_t)bb * p.bc_bs;
  const IO* __restrict__ cg = static_cast<const IO*>(p.c) + (int64_t)bb * p.bc_bs;
  // this lane's states of step t live at Hrow + t * (D*DS)
  const int64_t hstride = (int64_t)D * DS;
  const float* __restrict__ Hrow = p.H + (int64_t)bb * T * hstride + (int64_t)d * DS + j * K;
  const int64_t soff = ((int64_t)bb * D + d) * DS + j * K;

  float Av[K], A2[K], G[K], gA[K], hcur[K];
#pragma unroll
  for (int i = 0; i < K; ++i) { Av[i] = 0.f; G[i] = 0.f; gA[i] = 0.f; hcur[i] = 0.f; }
  if (dvalid) {
    load_k<K>(p.A + (int64_t)d * DS + j * K, Av);
    if (p.dhT != nullptr) load_k<K>(p.dhT + soff, G);
    if (T > 0) load_k<K>(Hrow + (int64_t)(T - 1) * hstride, hcur);
  }
#pragma unroll
  for (int i = 0; i < K; ++i) A2[i] = Av[i] * kLog2e;

  const int ntiles = (T + TB - 1) / TB;

  // ---- staged step inputs (one tile ahead) ----
  IO rx[PER], rd[PER], ry[PER], rb[PER_BC], rc[PER_BC];
  auto load_tile = [&](int ts) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + e * kThreads;
      const int t = ts + idx / CPW;
      const int dd = d0 + idx % CPW;
      if (t < T && dd < D) {
        const int64_t o = (int64_t)t * D + dd;
        rx[e] = xg[o];
        rd[e] = dg[o];
        ry[e] = yg[o];
      } else {
        rx[e] = IO{}; rd[e] = IO{}; ry[e] = IO{};
      }
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      const int idx = tid + e * kThreads;
      const int t = ts + idx / DS;
      if (idx < BC && t < T) {
        rb[e] = bg[(int64_t)t * DS + idx % DS];
        rc[e] = cg[(int64_t)t * DS + idx % DS];
      } else {
        rb[e] = IO{}; rc[e] = IO{};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float dl = to_f32(rd[e]);
      const float xv = to_f32(rx[e]);
      s_in[tid + e * kThreads] = make_float4(dl, xv, to_f32(ry[e]), dl * xv);
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      const int idx = tid + e * kThreads;
      if (idx < BC) {
        s_b[idx] = to_f32(rb[e]);
        s_c[idx] = to_f32(rc[e]);
      }
    }
  };

  // ---- H_{t-1} for one sub-block of HB steps, prefetched one sub-block ahead ----
  // Sub-block (tile it, sub s) covers steps ts + s*HB + [0, HB); its entry r holds H_{t-1}
  // for t = ts + s*HB + r, i.e. h0 for t = 0 and 0 for steps outside [1, T].
  float hbuf[2][HB][K];
  auto load_hblock = [&](float (&dst)[HB][K], int tfirst) {
#pragma unroll
    for (int r = 0; r < HB; ++r) {
      const int tp = tfirst + r - 1;  // index of the state to read
      if (dvalid && tp >= 0 && tp < T) {
        load_k<K>(Hrow + (int64_t)tp * hstride, dst[r]);
      } else if (dvalid && tp == -1 && p.h0 != nullptr) {
        load_k<K>(p.h0 + soff, dst[r]);
      } else {
#pragma unroll
        for (int i = 0; i < K; ++i) dst[r][i] = 0.f;
      }
    }
  };

  if (ntiles > 0) {
    const int ts_last = (ntiles - 1) * TB;
    load_tile(ts_last);
    load_hblock(hbuf[0], ts_last + (NSUB - 1) * HB);
  }

  for (int it = ntiles - 1; it >= 0; --it) {
    const int ts = it * TB;
    __syncthreads();  // previous tile's LDS users are done
    store_tile();
    __syncthreads();
    if (it > 0) load_tile(ts - TB);

#pragma unroll
    for (int s = NSUB - 1; s >= 0; --s) {
      // Sub-blocks are consumed in one global sequence; an even number precede each
      // tile, so the buffer roles depend only on s.
      float (&cur)[HB][K] = hbuf[(NSUB - 1 - s) & 1];
      float (&nxt)[HB][K] = hbuf[((NSUB - 1 - s) & 1) ^ 1];
      // prefetch the next sub-block in sweep order
      if (s > 0) {
        load_hblock(nxt, ts + (s - 1) * HB);
      } else if (it > 0) {
        load_hblock(nxt, ts - TB + (NSUB - 1) * HB);
      }

#pragma unroll
      for (int r = HB - 1; r >= 0; --r) {
        const int tt = s * HB + r;
        const float4 in = s_in[tt * CPW + ch];  // (delta, x, dy, delta*x)
        float bv[K], cv[K];
        load_k<K>(&s_b[tt * DS + j * K], bv);
        load_k<K>(&s_c[tt * DS + j * K], cv);
        float S = 0.f, gd = 0.f;
        float gbp[K], gcp[K];
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const float a = exp2_hw(in.x * A2[i]);
          const float g = fmaf(in.z, cv[i], G[i]);
          S = fmaf(g, bv[i], S);
          G[i] = a * g;
          const float q = G[i] * cur[r][i];
          gd = fmaf(Av[i], q, gd);
          gA[i] = fmaf(in.x, q, gA[i]);
          gbp[i] = g * in.w;
          gcp[i] = in.z * hcur[i];
          hcur[i] = cur[r][i];
        }
        S = group_sum<L>(S);
        gd = group_sum<L>(gd);
        if (j == 0) s_gxd[tt * CPW + ch] = make_float2(in.x * S, fmaf(in.y, S, gd));
#pragma unroll
        for (int i = 0; i < K; ++i) {
          gbp[i] = cross_row_sum(row_channel_sum<L>(gbp[i]));
          gcp[i] = cross_row_sum(row_channel_sum<L>(gcp[i]));
        }
        if (lane < L) {
#pragma unroll
          for (int i = 0; i < K; ++i) s_red[wave * BC + tt * DS + j * K + i] = make_float2(gbp[i], gcp[i]);
        }
      }
    }

    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + e * kThreads;
      const int t = ts + idx / CPW;
      const int dd = d0 + idx % CPW;
      if (t < T && dd < D) {
        const float2 v = s_gxd[idx];
        const int64_t o = (int64_t)bb * p.y_bs + (int64_t)t * D + dd;
        p.gx[o] = v.x;
        p.gdelta[o] = v.y;
      }
    }
    float2* __restrict__ part = p.part_bc + ((int64_t)blockIdx.x * p.B + bb) * T * DS;
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      const int idx = tid + e * kThreads;
      const int t = ts + idx / DS;
      if (idx < BC && t < T) {
        float2 acc = s_red[idx];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) {
          const float2 v = s_red[w * BC + idx];
          acc.x += v.x;
          acc.y += v.y;
        }
        part[(int64_t)t * DS + idx % DS] = acc;
      }
    }
  }

  if (!dvalid) return;
  float* pa = p.part_A + soff;
#pragma unroll
  for (int i = 0; i < K; ++i) pa[i] = gA[i];
  if (p.gh0 != nullptr) {
    float* g0 = p.gh0 + soff;
#pragma unroll
    for (int i = 0; i < K; ++i) g0[i] = G[i];
  }
}

// gb, gc: add the per-workgroup partials over channel tiles in ascending tile order.
// gA: add the per-batch-row partials in ascending batch order.
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(const ReduceParams p) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nbc = (int64_t)p.B * p.T * p.DS;
  const int64_t nA = (int64_t)p.D * p.DS;
  if (i < nbc) {
    const int64_t per_b = (int64_t)p.T * p.DS;
    const int64_t bb = i / per_b;
    const int64_t r = i - bb * per_b;
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < p.ntiles_d; ++k) {
      const float2 v = p.part_bc[((int64_t)k * p.B + bb) * per_b + r];
      sb += v.x;
      sc += v.y;
    }
    p.gb[i] = sb;
    p.gc[i] = sc;
  } else if (i < nbc + nA) {
    const int64_t e = i - nbc;
    float s = 0.f;
    for (int bb = 0; bb < p.B; ++bb) s += p.part_A[(int64_t)bb * nA + e];
    p.gA[e] = s;
  }
}

template <typename IO, int DS, int L>
hipError_t launch_bwd_t(const BwdParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((bwd_kernel<IO, DS, L>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int DS>
hipError_t launch_bwd_ds(int lanes, const BwdParams& p, dim3 grid, hipStream_t s) {
  switch (lanes) {
    case 1: return launch_bwd_t<IO, DS, 1>(p, grid, s);
    case 2: if constexpr (DS >= 2) return launch_bwd_t<IO, DS, 2>(p, grid, s); break;
    case 4: if constexpr (DS >= 4) return launch_bwd_t<IO, DS, 4>(p, grid, s); break;
    case 8: if constexpr (DS >= 8) return launch_bwd_t<IO, DS, 8>(p, grid, s); break;
    case 16: if constexpr (DS >= 16) return launch_bwd_t<IO, DS, 16>(p, grid, s); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_bwd_io(int DS, int lanes, const BwdParams& p, dim3 grid, hipStream_t s) {
  switch (DS) {
    case 1: return launch_bwd_ds<IO, 1>(lanes, p, grid, s);
    case 2: return launch_bwd_ds<IO, 2>(lanes, p, grid, s);
    case 4: return launch_bwd_ds<IO, 4>(lanes, p, grid, s);
    case 8: return launch_bwd_ds<IO, 8>(lanes, p, grid, s);
    case 16: return launch_bwd_ds<IO, 16>(lanes, p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_bwd(int io, int DS, int lanes, const BwdParams& p, dim3 grid, hipStream_t s) {
  if (io == 0) return launch_bwd_io<float>(DS, lanes, p, grid, s);
  return launch_bwd_io<bf16_t>(DS, lanes, p, grid, s);
}

hipError_t launch_bwd_reduce(const ReduceParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.T * p.DS + (int64_t)p.D * p.DS;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace sscan
