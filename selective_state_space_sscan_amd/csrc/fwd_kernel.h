// Forward selective scan kernel for gfx950 (included by fwd.hip and fwd_mamba.hip, which
// instantiate it without and with the Mamba-style wrapper).
//
// Recurrence ("pssa-100m/pssa_kernels.py" page, module docstring and scan_fwd):
//   h_t = exp(delta_t * A) * h_{t-1} + delta_t * b_t * x_t,   y_t = <h_t, c_t>.
//
// Work decomposition.  A workgroup of 256 threads owns one batch row and a tile of
// CPW = 256/L channels; the L consecutive lanes of a channel each hold K = DS/L of its
// fp32 states in VGPRs for the whole sequence.  Steps are processed in tiles of TB:
// the workgroup loads the x / delta tile and the b / c rows of the tile with coalesced
// loads (prefetched one tile ahead into registers), converts them to fp32 once and
// parks (delta, delta*x) and b, c in LDS, where every lane of a channel reads them as a
// broadcast.  Per (step, state) a lane does one v_exp_f32 and four fp32 ops; the
// readout <h, c> is reduced over the L lanes with DPP and y is written back through
// LDS so the store is coalesced.  Steps past the end of the sequence are padded with
// delta = 0 and delta*x = 0, which leave the state bit-for-bit unchanged (exp2(0) = 1).
//
// Two-level scan along T (used when B*D*L lanes cannot fill the GPU).  The local pass
// runs chunks 0..C-2 from a zero state and records, per (b, d, n), the chunk's decay
// product exp(A * sum(delta)) (the product of its per-step decays) and its end state.
// Each workgroup of the full pass composes the pairs of the chunks before its own, left
// to right from h0 (h <- P_k h + hloc_k), and reruns its chunk from that true start
// state.  The decomposition is the associativity of the affine maps h -> a*h + u.
#pragma once
#include "device_common.h"

namespace sscan {
namespace {

template <int K>
__device__ __forceinline__ void load_state(const float* __restrict__ p, float (&v)[K]) {
  lds_load_vec<K>(p, v);  // plain vector load; also valid for global memory
}

// Steps whose decays and injections are formed together before the serial update:
// at most 32 floats per array per lane, at most 16 steps.
template <int K, int TB>
__host__ __device__ constexpr int fwd_batch_steps() {
  return (32 / K) < 16 ? ((32 / K) < TB ? (32 / K) : TB) : (16 < TB ? 16 : TB);
}

// MODE: kLocal (local pass of the two-level scan: no outputs but the chunk pair),
// kFull (y and hT), kFullH (y, hT and H), kFullCk (y, hT and the H-free path's boundary
// states).  What is stored is a compile-time choice so that the stores are unconditional
// in the step code.
constexpr int kLocal = 0, kFull = 1, kFullH = 2, kFullCk = 3;

// MAMBA: the Mamba-style wrapper -- delta is read as delta_raw and passed through the
// thresholded softplus when it is staged, A is read as A_log (A = -exp(A_log)), and the
// skip term Dskip * x is added to y before it is rounded and stored.
template <typename IO, int DS, int L, int MODE, bool MAMBA>
__global__ __launch_bounds__(kThreads) void fwd_kernel(const FwdParams p) {
  constexpr bool LOCAL = MODE == kLocal;
  constexpr int K = DS / L;
  constexpr int CPW = kThreads / L;
  constexpr int TB = fwd_tile_steps(L);
  constexpr int TILE = TB * CPW;
  constexpr int PER = TILE / kThreads;
  constexpr int BC = TB * DS;
  constexpr int PER_BC = (BC + kThreads - 1) / kThreads;
  constexpr int S = fwd_batch_steps<K, TB>();
  constexpr uint32_t ES = sizeof(IO);
  static_assert(TILE % kThreads == 0 && TB % S == 0, "tile shape");

  __shared__ float2 s_dw[TILE];            // (delta, delta*x) at [step*CPW + channel]
  __shared__ float s_b[BC];                // b at [step*DS + n]
  __shared__ float s_c[BC];
  __shared__ float s_y[LOCAL ? 1 : TILE];  // y at [step*CPW + channel]
  __shared__ float s_skip[(MAMBA && !LOCAL) ? TILE : 1];  // Dskip * x of the tile

  const int lin = xcd_grouped(blockIdx.x, gridDim.x, p.xcd_group);
  const int dtile = lin % p.ntiles_d;
  const int rest = lin / p.ntiles_d;
  const int bb = rest % p.B;
  const int chunk = rest / p.B;

  const int tid = threadIdx.x;
  const int ch = tid / L;
  const int j = tid % L;
  const int D = p.D;
  const int d0 = dtile * CPW;
  const int t_begin = chunk * p.chunk_len;
  const int t_end = min(p.T, t_begin + p.chunk_len);
  const int d = d0 + ch;
  const bool dvalid = d < D;

  const IO* xrow = static_cast<const IO*>(p.x) + (int64_t)bb * p.x_bs;
  const IO* drow = static_cast<const IO*>(p.delta) + (int64_t)bb * p.x_bs;
  const IO* brow = static_cast<const IO*>(p.b) + (int64_t)bb * p.bc_bs;
  const IO* crow = static_cast<const IO*>(p.c) + (int64_t)bb * p.bc_bs;
  IO* yrow = static_cast<IO*>(p.y) + (int64_t)bb * p.y_bs;
  float* Hrow = p.H + (int64_t)bb * p.T * D * DS;

  const int64_t nstate = (int64_t)p.B * D * DS;
  const int64_t soff = ((int64_t)bb * D + d) * DS + j * K;  // this lane's states in (B,D,DS)
  // boundary states of this batch row; each tile addresses the (at most kCkBlocks) blocks it
  // touches through a resource based at its first block, so offsets stay 32-bit at any T
  const float* ckrow = MODE == kFullCk ? p.hck + (int64_t)bb * p.nck * D * DS : nullptr;
  constexpr int kCkBlocks = (TB + kCkptSteps - 1) / kCkptSteps;

  float A2[K], h[K];
  if (dvalid) {
    load_state<K>(p.A + (int64_t)d * DS + j * K, A2);
#pragma unroll
    for (int i = 0; i < K; ++i) A2[i] = (MAMBA ? -expf(A2[i]) : A2[i]) * kLog2e;
    if (LOCAL || (chunk == 0 && p.h0 == nullptr)) {
#pragma unroll
      for (int i = 0; i < K; ++i) h[i] = 0.f;
    } else {
      // h0, then left to right the (decay product, local end state) pair of every chunk
      // before this one: h <- P h + hloc
      if (p.h0 != nullptr) {
        load_state<K>(p.h0 + soff, h);
      } else {
#pragma unroll
        for (int i = 0; i < K; ++i) h[i] = 0.f;
      }
      for (int k = 0; k < chunk; ++k) {
        const float2* pr = p.pairs + (int64_t)k * nstate + soff;
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const float2 m = pr[i];
          h[i] = fmaf(m.x, h[i], m.y);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) { A2[i] = 0.f; h[i] = 0.f; }
  }
  double dsum = 0.0;  // local pass: sum of delta over the chunk

  // Per-thread element offsets inside an x/delta/y tile (rows beyond the tile end fall
  // outside the resource; columns beyond D are forced out of range).
  uint32_t xoff[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid + e * kThreads;
    const int dd = d0 + idx % CPW;
    xoff[e] = dd < D ? static_cast<uint32_t>((idx / CPW) * D + dd) * ES : kOutOfRange;
  }
  uint32_t bcoff[PER_BC];
#pragma unroll
  for (int e = 0; e < PER_BC; ++e) {
    const int idx = tid + e * kThreads;
    bcoff[e] = idx < BC ? static_cast<uint32_t>(idx) * ES : kOutOfRange;
  }
  const uint32_t hstep = static_cast<uint32_t>(D) * DS * 4u;  // bytes between steps of H
  const uint32_t hlane = dvalid ? static_cast<uint32_t>(d * DS + j * K) * 4u : kOutOfRange;

  // the next tile as loaded (raw bits, a bf16 zero-extended): widened only when parked in
  // LDS, since a widening next to the load makes the compiler wait for the load right there
  uint32_t rx[PER], rd[PER], rb[PER_BC], rc[PER_BC];
  int pend_rows = 0;  // rows of the tile whose loads are in flight
  // Past the end of the chunk the resource is empty and every load returns 0: the
  // prefetch is issued unconditionally, so that the wait for it never has to cover the
  // H and y stores issued after it (a conditional load makes the wait count path-dependent).
  auto load_tile = [&](int ts) {
    const int rows = tile_rows(t_end, ts, TB);
    pend_rows = rows;
    const rsrc_t rX = make_rsrc(xrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rD = make_rsrc(drow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rB = make_rsrc(brow + (int64_t)ts * DS, static_cast<uint32_t>(rows * DS) * ES);
    const rsrc_t rC = make_rsrc(crow + (int64_t)ts * DS, static_cast<uint32_t>(rows * DS) * ES);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      rx[e] = buf_load_bits<IO>(rX, xoff[e]);
      rd[e] = buf_load_bits<IO>(rD, xoff[e]);
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      rb[e] = buf_load_bits<IO>(rB, bcoff[e]);
      rc[e] = buf_load_bits<IO>(rC, bcoff[e]);
    }
  };
  // The channel a thread stages is the same in every row of a tile (256 is a multiple of CPW).
  const int sdd = d0 + tid % CPW;
  const float dskip = (MAMBA && p.Dskip != nullptr && sdd < D) ? p.Dskip[sdd] : 0.f;
  auto store_tile = [&]() {
    // keep the scheduler from hoisting the delta*x products (and with them the wait for
    // the loads) into the step code that runs while the loads are still in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      // padded steps and channels keep delta = 0 (the softplus of a zero would not be 0)
      // (a multiply by a 0/1 mask, not a select: a select lets the compiler branch around
      // the softplus, which costs registers across the step code)
      const float keep = ((tid + e * kThreads) / CPW < pend_rows && xoff[e] != kOutOfRange) ? 1.f : 0.f;
      const float xv = bits_to_f32<IO>(rx[e]), dv = bits_to_f32<IO>(rd[e]);
      const float dl = MAMBA ? softplus_th(dv) * keep : dv;
      s_dw[tid + e * kThreads] = make_float2(dl, dl * xv);
      if constexpr (MAMBA && !LOCAL) s_skip[tid + e * kThreads] = dskip * xv;
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      const int idx = tid + e * kThreads;
      if (BC % kThreads == 0 || idx < BC) {
        s_b[idx] = bits_to_f32<IO>(rb[e]);
        s_c[idx] = bits_to_f32<IO>(rc[e]);
      }
    }
  };

  const int nsteps_total = t_end - t_begin;
  const int ntiles = nsteps_total > 0 ? (nsteps_total + TB - 1) / TB : 0;
  if (ntiles > 0) {
    load_tile(t_begin);
    store_tile();
  }

  // Each tile issues the next tile's loads before its own steps and parks them in LDS
  // only after them, so no loaded register is live across the loop back-edge and the
  // wait for those loads never has to cover the H stores issued in between.
  for (int it = 0; it < ntiles; ++it) {
    const int ts = t_begin + it * TB;
    const int rows = min(TB, t_end - ts);
    __syncthreads();  // this tile's inputs are in LDS; the previous tile's y reads are done
    load_tile(ts + TB);

    const rsrc_t rH = make_rsrc(Hrow + (int64_t)ts * D * DS, static_cast<uint32_t>(rows) * hstep);
    const int kb0 = ts / kCkptSteps;  // first boundary block of the tile
    const rsrc_t rCk = make_rsrc(MODE == kFullCk ? ckrow + (int64_t)kb0 * D * DS : nullptr,
                                 MODE == kFullCk ? static_cast<uint32_t>(min(p.nck - kb0, kCkBlocks) * D * DS) * 4u : 0u);
#pragma unroll
    for (int s0 = 0; s0 < TB; s0 += S) {
      if constexpr (MODE == kFullCk) {
        // H-free path: the state entering every block of kCkptSteps steps.  S divides the
        // block length and tiles start on multiples of min(TB, kCkptSteps), so block starts
        // are batch starts; where the tile holds whole blocks they are fixed batches.  The
        // store is unconditional (out of range elsewhere, and past the end of the chunk, where
        // batches are padding), so the wait counts stay the same on every path.
        if (s0 % (TB < kCkptSteps ? TB : kCkptSteps) == 0) {  // a constant once the loop is unrolled
          const bool ok = dvalid && ts + s0 < t_end && (ts + s0) % kCkptSteps == 0;
          buf_store_vec<K>(rCk, ok ? static_cast<uint32_t>((((ts + s0) / kCkptSteps - kb0) * D + d) * DS + j * K) * 4u
                                   : kOutOfRange, h);
        }
      }
      // decays and injections of S steps: independent of the state, issued together
      float a[S][K], u[S][K];
      float dl[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const float2 dw = s_dw[(s0 + s) * CPW + ch];
        float bv[K];
        lds_load_vec<K>(&s_b[(s0 + s) * DS + j * K], bv);
#pragma unroll
        for (int i = 0; i < K; ++i) {
          a[s][i] = exp2_hw(dw.x * A2[i]);
          u[s][i] = dw.y * bv[i];
        }
        dl[s] = dw.x;
      }
      // the serial part: one fma per (step, state); a[s] then holds the state after step s
#pragma unroll
      for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int i = 0; i < K; ++i) {
          h[i] = fmaf(a[s][i], h[i], u[s][i]);
          a[s][i] = h[i];
        }
      }
      if constexpr (LOCAL) {
        dsum += static_cast<double>(tree_sum<S>(dl));  // the batch's delta sum as an fp32 tree
      } else {
        // readouts of S steps, independent of each other
#pragma unroll
        for (int s = 0; s < S; ++s) {
          float cv[K];
          lds_load_vec<K>(&s_c[(s0 + s) * DS + j * K], cv);
          float yp = 0.f;
#pragma unroll
          for (int i = 0; i < K; ++i) yp = fmaf(a[s][i], cv[i], yp);
          s_y[(s0 + s) * CPW + ch] = group_sum<L>(yp);  // every lane of the channel holds the sum
        }
        if constexpr (MODE == kFullH) {
#pragma unroll
          for (int s = 0; s < S; ++s)
            buf_store_vec<K, kNonTemporal>(rH, hlane + static_cast<uint32_t>(s0 + s) * hstep, a[s]);
        }
      }
    }

    __syncthreads();  // every lane is done with this tile's inputs and has written its y
    if constexpr (!LOCAL) {
      const rsrc_t rY = make_rsrc(yrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        float yv = s_y[tid + e * kThreads];
        if constexpr (MAMBA) yv += s_skip[tid + e * kThreads];
        buf_store_io<IO>(rY, xoff[e], yv);
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

template <typename IO, int DS, int L, bool MAMBA>
hipError_t launch_fwd_t(bool local_pass, const FwdParams& p, unsigned blocks, hipStream_t s) {
  if (local_pass)
    hipLaunchKernelGGL((fwd_kernel<IO, DS, L, kLocal, MAMBA>), dim3(blocks), dim3(kThreads), 0, s, p);
  else if (p.H != nullptr)
    hipLaunchKernelGGL((fwd_kernel<IO, DS, L, kFullH, MAMBA>), dim3(blocks), dim3(kThreads), 0, s, p);
  else if (p.hck != nullptr)
    hipLaunchKernelGGL((fwd_kernel<IO, DS, L, kFullCk, MAMBA>), dim3(blocks), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_kernel<IO, DS, L, kFull, MAMBA>), dim3(blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int DS, bool MAMBA>
hipError_t launch_fwd_ds(int lanes, bool local_pass, const FwdParams& p, unsigned grid, hipStream_t s) {
  switch (lanes) {
    case 1: return launch_fwd_t<IO, DS, 1, MAMBA>(local_pass, p, grid, s);
    case 2: if constexpr (DS >= 2) return launch_fwd_t<IO, DS, 2, MAMBA>(local_pass, p, grid, s); break;
    case 4: if constexpr (DS >= 4) return launch_fwd_t<IO, DS, 4, MAMBA>(local_pass, p, grid, s); break;
    case 8: if constexpr (DS >= 8) return launch_fwd_t<IO, DS, 8, MAMBA>(local_pass, p, grid, s); break;
    case 16: if constexpr (DS >= 16) return launch_fwd_t<IO, DS, 16, MAMBA>(local_pass, p, grid, s); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename IO, bool MAMBA>
hipError_t launch_fwd_io(int DS, int lanes, bool local_pass, const FwdParams& p, unsigned grid, hipStream_t s) {
  switch (DS) {
    case 1: return launch_fwd_ds<IO, 1, MAMBA>(lanes, local_pass, p, grid, s);
    case 2: return launch_fwd_ds<IO, 2, MAMBA>(lanes, local_pass, p, grid, s);
    case 4: return launch_fwd_ds<IO, 4, MAMBA>(lanes, local_pass, p, grid, s);
    case 8: return launch_fwd_ds<IO, 8, MAMBA>(lanes, local_pass, p, grid, s);
    case 16: return launch_fwd_ds<IO, 16, MAMBA>(lanes, local_pass, p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace sscan
