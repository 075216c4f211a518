// Backward selective scan kernels for gfx950 (included by bwd.hip and bwd_mamba.hip, which
// instantiate them without and with the Mamba-style wrapper).
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
// parked in LDS as fp32.  The states H_{t-1} of a wave's channels are fetched a
// sub-block ahead with 16-byte non-temporal loads per lane (a wave's channels cover
// consecutive addresses of each step row; H is read once, and kept out of the caches
// it would otherwise flush), parked in a per-wave LDS block when their sub-block starts
// (with four states per lane each lane's load is exactly its own states, which stay in
// registers; then only the first row of each block is read, and the rows after it are formed
// from it by the forward's own update -- bit for bit the stored rows when the forward ran
// as one pass, within fp32 rounding of them where a split forward started a chunk inside
// the block), and read back by each lane
// for its own states; H_t is kept from the step before.  Sums over a channel's states
// use DPP; sums over channels use DPP row rotations, the gfx950 row-swap permutes and
// one LDS slot per wave, and each workgroup writes one (gb, gc) partial per (step,
// state) and one gA partial per (batch row, channel, state).  A second kernel adds the
// partials in a fixed order: no float atomics, results are bitwise reproducible.
#pragma once
#include "device_common.h"

namespace sscan {
namespace {

template <int K>
__device__ __forceinline__ void load_k(const float* __restrict__ p, float (&v)[K]) {
  lds_load_vec<K>(p, v);  // plain vector load; also valid for global memory
}

// Steps per batch: the decays of a batch are formed together, then the adjoint carry
// runs through it, then the per-step gradient terms and their sums.  S*K <= 4 (so three
// waves fit on a SIMD) and at least two batches per tile.
template <int K, int TB>
__host__ __device__ constexpr int bwd_batch_steps() {
  return (4 / K) < 2 ? ((K == 1) ? 2 : 1) : ((4 / K) < (TB / 2) ? (4 / K) : (TB / 2));
}

// Reduce-scatter of per-lane values over the four 16-lane rows of a wave for a pair of
// items: afterwards row 0 holds the 4-row total of b0, row 1 of b1, row 2 of c0 and
// row 3 of c1.  The gfx950 row-swap permutes exchange halves between two registers.
__device__ __forceinline__ float rows_reduce_scatter(float b0, float c0, float b1, float c1) {
  auto p0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(b0), __float_as_uint(c0), false, false);
  auto p1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(b1), __float_as_uint(c1), false, false);
  // lanes 0-31: b summed over rows (r, r+2); lanes 32-63: c summed likewise
  const float v0 = __uint_as_float(p0[0]) + __uint_as_float(p0[1]);
  const float v1 = __uint_as_float(p1[0]) + __uint_as_float(p1[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Sums over the four DPP banks (4-lane groups) of each 16-lane row, reduce-scattered: on
// entry every lane holds b[0..3] and c[0..3]; on exit b[0] and c[0] of a lane in bank k
// hold the row totals of b[k] and c[k] over its four banks (lanes l, l^4, l^8, l^12).
// Stage 1 pairs banks k and k^2 (row_ror:8): banks 0, 1 keep items 0, 1 and banks 2, 3
// items 2, 3; stage 2 pairs banks k and k^1 (row_shl / row_shr by 4).  Each pair costs two
// bank-masked DPP adds that write disjoint banks, the first reading the partner's copy
// before the second overwrites it.  The leading s_nop gives the two wait states a DPP read
// of a register written by the previous vector instruction requires; within the block every
// DPP source was written at least two instructions earlier.
__device__ __forceinline__ void bank_reduce_scatter(float (&b)[4], float (&c)[4]) {
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %0, %0, %0 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %2, %2 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %3, %3 row_shr:4 row_mask:0xf bank_mask:0xa"
      : "+v"(b[0]), "+v"(b[1]), "+v"(c[0]), "+v"(c[1])
      : "v"(b[2]), "v"(b[3]), "v"(c[2]), "v"(c[3]));
}

// Sum over the four 16-lane rows of a wave for a pair (b, c) of per-lane values: rows 0
// and 1 receive the total of b, rows 2 and 3 the total of c (gfx950 row-swap permutes).
__device__ __forceinline__ float rows_pair_sum(float b, float c) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(b), __float_as_uint(c), false, false);
  const float v = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // rows 0-1: b over rows (r, r+2); 2-3: c
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// DPP pattern that pairs each lane with one whose lane-index bit M differs and whose
// higher bits agree (M = 1, 2, 4, 8).
template <int M>
__host__ __device__ constexpr int pair_ctrl() {
  return M == 8 ? kDppRowMirror : (M == 4 ? kDppRowHalfMirror : (M == 2 ? kDppQuadXor2 : kDppQuadXor1));
}

// Reduce-scatter over a group of 2M lanes (group index j): on entry every lane holds C
// live values v[0..C); each stage halves the live values, keeping the half selected by
// bit M of j and adding the partner's copy of it.  On exit lane j holds group totals of
// max(1, C/2M) consecutive items starting at idx0; once a single value is left the
// remaining stages are plain all-reduce steps.  Every stage's adds are independent.
template <int M, int C, int V>
__device__ __forceinline__ void reduce_scatter(float (&v)[V], int j, int& idx0) {
  if constexpr (M >= 1) {
    if constexpr (C >= 2) {
      constexpr int H = C / 2;
      const bool up = (j & M) != 0;
#pragma unroll
      for (int q = 0; q < H; ++q) {
        const float keep = up ? v[q + H] : v[q];
        const float send = up ? v[q] : v[q + H];
        v[q] = keep + dpp<pair_ctrl<M>()>(send);
      }
      if (up) idx0 += H;
      reduce_scatter<M / 2, H, V>(v, j, idx0);
    } else {
      v[0] += dpp<pair_ctrl<M>()>(v[0]);
      reduce_scatter<M / 2, 1, V>(v, j, idx0);
    }
  }
}

// MAMBA: the Mamba-style wrapper -- delta is read as delta_raw (delta = softplus, whose
// derivative scales gdelta), A as A_log (A = -exp(A_log)), the skip term adds dy * Dskip
// to gx, and each workgroup leaves a partial sum of dy * x per channel for gDskip.
// HF: the H-free sweep -- instead of reading H, each tile recomputes its states from the
// boundary state saved by the forward at the tile's first step (tiles and checkpoint
// blocks are both kCkptSteps long), with the forward's own arithmetic, so the states
// are the forward's bit for bit.  They go to a per-wave LDS block that the sweep reads.
template <typename IO, int DS, int L, bool MAMBA, bool HF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DS == 16 && (L == 16 || L == 4) ? 3 : (DS / L >= 8 ? 1 : 2)))) void bwd_kernel(const BwdParams p) {
  constexpr int K = DS / L;
  constexpr int CPW = kThreads / L;
  constexpr int TB = bwd_tile_steps(L);
  constexpr int TILE = TB * CPW;
  constexpr int PER = TILE / kThreads;
  constexpr int BC = TB * DS;
  constexpr int PER_BC = (BC + kThreads - 1) / kThreads;
  constexpr int NWAVE = kThreads / 64;
  constexpr int S = bwd_batch_steps<K, TB>();
  // steps of H per prefetch block (four with four states per lane, where only its first row
  // is read)
  constexpr int HB = (!HF && K == 4) ? 4 : (2 * S) < (TB / 2) ? (2 * S) : (TB / 2);
  constexpr int NSUB = TB / HB;
  constexpr int NBAT = HB / S;
  constexpr int NITEM = S * K;
  constexpr uint32_t ES = sizeof(IO);
  static_assert(TILE % kThreads == 0 && TB % HB == 0 && HB % S == 0, "tile shape");
  static_assert(NITEM % 2 == 0, "items per batch must pair up");
  static_assert(!HF || TB == kCkptSteps, "the H-free sweep takes one boundary block per tile");

  __shared__ float4 s_in[TILE];              // (delta, x, dy, delta*x) at [step*CPW + channel]
  __shared__ float s_b[BC];
  __shared__ float s_c[BC];
  __shared__ float2 s_gxd[TILE];             // (gx, gdelta)
  __shared__ float s_red[2 * NWAVE * BC];    // per-wave gb sums, then per-wave gc sums
  __shared__ float s_sig[MAMBA ? TILE : 1];  // d delta / d delta_raw of the tile
  __shared__ float s_acc[MAMBA ? kThreads : 1];

  const int lin = xcd_grouped(blockIdx.x, gridDim.x, p.xcd_group);
  const int dtile = lin % p.ntiles_d;
  const int rest = lin / p.ntiles_d;
  const int bb = rest % p.B;
  const int chunk = rest / p.B;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane >> 4;
  const int ch = tid / L;
  const int j = tid % L;
  const int d0 = dtile * CPW;
  const int D = p.D;
  const int T = p.T;
  const int t_lo = chunk * p.chunk_len;           // this workgroup's steps: [t_lo, t_hi)
  const int t_hi = min(T, t_lo + p.chunk_len);
  const int d = d0 + ch;
  const bool dvalid = d < D;
  const int64_t nstate = (int64_t)p.B * D * DS;

  const IO* xrow = static_cast<const IO*>(p.x) + (int64_t)bb * p.x_bs;
  const IO* drow = static_cast<const IO*>(p.delta) + (int64_t)bb * p.x_bs;
  const IO* yrow = static_cast<const IO*>(p.dy) + (int64_t)bb * p.x_bs;
  const IO* brow = static_cast<const IO*>(p.b) + (int64_t)bb * p.bc_bs;
  const IO* crow = static_cast<const IO*>(p.c) + (int64_t)bb * p.bc_bs;
  float* gxrow = p.gx + (int64_t)bb * p.y_bs;
  float* gdrow = p.gdelta + (int64_t)bb * p.y_bs;
  const float* Hrow = HF ? nullptr : p.H + (int64_t)bb * T * D * DS;
  const int64_t soff = ((int64_t)bb * D + d) * DS + j * K;
  const uint32_t hstep = static_cast<uint32_t>(D) * DS * 4u;

  float Av[K], A2[K], G[K], gA[K], hcur[K];
#pragma unroll
  for (int i = 0; i < K; ++i) { Av[i] = 0.f; G[i] = 0.f; gA[i] = 0.f; hcur[i] = 0.f; }
  if (dvalid) {
    load_k<K>(p.A + (int64_t)d * DS + j * K, Av);
    // the adjoint entering this chunk from the right: dhT composed, right to left, with
    // the carry maps G -> P G + Gloc of every sub-chunk after this chunk (the local pass
    // left one pair per sub-chunk of chunks 1 .. C-1)
    if (p.dhT != nullptr) load_k<K>(p.dhT + soff, G);
    for (int k = p.chunks * p.subs - 1; k >= (chunk + 1) * p.subs; --k) {
      const float2* pr = p.pairs + (int64_t)(k - p.subs) * nstate + soff;
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const float2 m = pr[i];
        G[i] = fmaf(m.x, G[i], m.y);
      }
    }
    if (!HF && t_hi > t_lo) load_k<K>(Hrow + (int64_t)(t_hi - 1) * D * DS + d * DS + j * K, hcur);
  }
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if constexpr (MAMBA) Av[i] = dvalid ? -expf(Av[i]) : 0.f;
    A2[i] = Av[i] * kLog2e;
  }

  const int ntiles = t_hi > t_lo ? (t_hi - t_lo + TB - 1) / TB : 0;

  // ---- staged step inputs (one tile ahead) ----
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
  float rx[PER], rd[PER], ry[PER], rb[PER_BC], rc[PER_BC];
  int pend_rows = 0;  // rows of the tile whose loads are in flight
  // Every prefetch below is issued unconditionally, with an empty resource (all loads
  // return 0) where there is nothing to fetch: a load issued on one path only makes the
  // compiler's wait for older loads path-dependent, and it then waits for everything.
  auto load_tile = [&](int ts) {
    const int rows = ts >= t_lo ? tile_rows(t_hi, ts, TB) : 0;
    pend_rows = rows;
    const rsrc_t rX = make_rsrc(xrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rD = make_rsrc(drow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rY = make_rsrc(yrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rB = make_rsrc(brow + (int64_t)ts * DS, static_cast<uint32_t>(rows * DS) * ES);
    const rsrc_t rC = make_rsrc(crow + (int64_t)ts * DS, static_cast<uint32_t>(rows * DS) * ES);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      rx[e] = buf_load_elem<IO>(rX, xoff[e]);
      rd[e] = buf_load_elem<IO>(rD, xoff[e]);
      ry[e] = buf_load_elem<IO>(rY, xoff[e]);
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      rb[e] = buf_load_elem<IO>(rB, bcoff[e]);
      rc[e] = buf_load_elem<IO>(rC, bcoff[e]);
    }
  };
  auto store_tile = [&]() {
    // keep the scheduler from hoisting the delta*x products (and with them the wait for
    // the loads) into the step code that runs while the loads are still in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float dl = rd[e];
      if constexpr (MAMBA) {
        // padded steps and channels keep delta = 0 (the softplus of a zero would not be 0)
        // (a multiply by a 0/1 mask, not a select, which the compiler would turn into a branch)
        const float keep = ((tid + e * kThreads) / CPW < pend_rows && xoff[e] != kOutOfRange) ? 1.f : 0.f;
        dl = softplus_th(rd[e]) * keep;
        s_sig[tid + e * kThreads] = softplus_th_grad(rd[e]) * keep;
      }
      s_in[tid + e * kThreads] = make_float4(dl, rx[e], ry[e], dl * rx[e]);
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      const int idx = tid + e * kThreads;
      if (BC % kThreads == 0 || idx < BC) {
        s_b[idx] = rb[e];
        s_c[idx] = rc[e];
      }
    }
  };
  // The channel a thread stages and stores is the same in every row of a tile.
  const int sdd = d0 + tid % CPW;
  const float dskip = (MAMBA && p.Dskip != nullptr && sdd < D) ? p.Dskip[sdd] : 0.f;
  float accD = 0.f;  // sum of dy * x over this thread's elements (one channel)

  // ---- H_{t-1} for a block of HB steps starting at step tf, prefetched a block ahead ----
  // Per step, the lanes of a wave need 64*K consecutive floats of H (its channels' rows).
  // A block is fetched with 16-byte loads per lane (a quarter of the vector-memory
  // instructions and address work of one dword per lane and step) into registers, and
  // parked in a per-wave LDS block at the start of the sub-block that reads it, where
  // each lane picks up its own states.  Row r of a block holds H_{tf+r-1}, and 0 for
  // steps outside [1, T], for channels past D, or when the block is not valid; step 0
  // takes h0 from registers.
  constexpr int WROW = 64 * K;                                  // floats per step and wave
  constexpr int HBLK = HB * WROW;                               // floats per block and wave
  constexpr int DB = (HBLK * 4) % (64 * 16) == 0 ? 16 : 4;      // bytes per lane and load
  constexpr int NQ = HBLK * 4 / (64 * DB);                      // loads per block
  static_assert(NQ * 64 * DB == HBLK * 4, "an H block is a whole number of loads");
  __shared__ float s_h[(HF || (K == 4 && DB == 16)) ? 1 : NWAVE * HBLK];
  // boundary state of the next tile to sweep, loaded one tile ahead
  float hck_next[K];
  const float* ckrow = HF ? p.hck + (int64_t)bb * p.nck * D * DS : nullptr;
  // (tiles are one boundary block long: the resource covers just the tile's block, so
  // offsets stay 32-bit at any T)
  auto load_ckpt = [&](int ts, bool valid) {
    const rsrc_t rK = make_rsrc(HF ? ckrow + (int64_t)(max(ts, 0) / kCkptSteps) * D * DS : nullptr,
                                valid ? static_cast<uint32_t>(D * DS) * 4u : 0u);
    const uint32_t off = dvalid ? static_cast<uint32_t>(d * DS + j * K) * 4u : kOutOfRange;
    buf_load_vec<K>(rK, off, hck_next);
  };
  const int wd0 = d0 + wave * (64 / L);                         // first channel of this wave
  const uint32_t wbytes = static_cast<uint32_t>(max(0, min(64 / L, D - wd0)) * DS * 4);
  const uint32_t whoff = static_cast<uint32_t>(wd0) * DS * 4u;
  float* const hblk = s_h + ((HF || (K == 4 && DB == 16)) ? 0 : wave * HBLK);
  // With four states per lane every 16-byte load of a block is one step row and each lane
  // fetches exactly its own states, so the block goes straight to registers (hb) instead of
  // through the per-wave LDS block.
  constexpr bool HDIRECT = !HF && K == 4 && DB == 16;
  static_assert(!HDIRECT || NQ == HB, "one load per step row");
  // With one step per batch, only the first row of each HB-row block is read; the rows
  // after it are formed from it with the forward's own operations on the same inputs: a
  // quarter of the H traffic at HB = 4.  They are bit for bit the rows a single-pass
  // forward stored; where the forward split the sequence (its two-level scan), the state
  // it started a chunk from was composed from the chunk pairs rather than read from the
  // row before, so rows formed across such a chunk start agree with the stored ones only
  // to fp32 rounding (well inside the tolerance; the gradients are still exact adjoints
  // of states within rounding of the forward's).
  constexpr bool HFIRST = HDIRECT && S == 1;
  float hq[NQ][DB / 4];
  float hb[HDIRECT ? NQ : 1][DB / 4];
  float hzero[K];
#pragma unroll
  for (int i = 0; i < K; ++i) hzero[i] = 0.f;
  if (chunk == 0 && p.h0 != nullptr && dvalid) load_k<K>(p.h0 + soff, hzero);
  auto load_hblock = [&](float (&dst)[NQ][DB / 4], int tf, bool valid) {
    const int h_lo = max(tf - 1, 0);
    const int h_hi = min(tf - 1 + HB, T);  // exclusive
    const uint32_t nrow = valid ? static_cast<uint32_t>(max(h_hi - h_lo, 0)) : 0u;
    const rsrc_t rH = make_rsrc(Hrow + (int64_t)h_lo * D * DS, nrow * hstep);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (HFIRST && q > 0) continue;  // the later rows are formed from the first
      const int pos = q * 64 * DB + lane * DB;  // byte within the wave's block
      const int r = pos / (WROW * 4);
      const uint32_t b = static_cast<uint32_t>(pos % (WROW * 4));
      const int tp = tf - 1 + r;
      const uint32_t off = (tp >= 0 && b < wbytes) ? static_cast<uint32_t>(tp - h_lo) * hstep + whoff + b : kOutOfRange;
      buf_load_vec<DB / 4, kNonTemporal>(rH, off, dst[q]);
    }
  };
  auto park_hblock = [&](const float (&src)[NQ][DB / 4]) {
    if constexpr (HDIRECT) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < DB / 4; ++e) hb[q][e] = src[q][e];
      return;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float* dst = hblk + q * 16 * DB + lane * (DB / 4);
      if constexpr (DB == 16)
        *reinterpret_cast<float4*>(dst) = make_float4(src[q][0], src[q][1], src[q][2], src[q][3]);
      else
        dst[0] = src[q][0];
    }
  };

  if (ntiles > 0) {
    const int ts_last = t_lo + (ntiles - 1) * TB;
    load_tile(ts_last);
    if constexpr (HF)
      load_ckpt(ts_last, true);
    else
      load_hblock(hq, ts_last + (NSUB - 1) * HB, true);
    store_tile();
  }

  // As in the forward, each tile issues the loads of the tile before it first and parks
  // them in LDS only after its own steps, so that no loaded tile register is live across
  // the loop back-edge (the wait for it would otherwise cover every later load).
  for (int it = ntiles - 1; it >= 0; --it) {
    const int ts = t_lo + it * TB;
    __syncthreads();  // this tile's inputs are in LDS; the previous tile's output reads are done
    load_tile(ts - TB);

    // H-free sweep: the tile's decays, formed once by the recomputation and reused by the
    // sweep (the same values the sweep would form again)
    float at[HF ? TB : 1][K];
    // and its states: hrec[r] = H_{ts+r-1}, r = 0..TB (each lane keeps its own)
    float hrec[HF ? TB + 1 : 1][K];
    if constexpr (HF) {
      // recompute the tile's states from its boundary state, as the forward formed them:
      // a = exp2(delta * A log2 e), h = fma(a, h, (delta x) b); padded steps leave h as is
      float hs[K];
#pragma unroll
      for (int i = 0; i < K; ++i) hs[i] = hck_next[i];
      load_ckpt(ts - TB, it > 0);
#pragma unroll
      for (int i = 0; i < K; ++i) hrec[0][i] = hs[i];
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const float4 in4 = s_in[t * CPW + ch];
        float bv[K];
        lds_load_vec<K>(&s_b[t * DS + j * K], bv);
#pragma unroll
        for (int i = 0; i < K; ++i) {
          at[t][i] = exp2_hw(in4.x * A2[i]);
          hs[i] = fmaf(at[t][i], hs[i], in4.w * bv[i]);
        }
#pragma unroll
        for (int i = 0; i < K; ++i) hrec[t + 1][i] = hs[i];
      }
#pragma unroll
      for (int i = 0; i < K; ++i) hcur[i] = hs[i];  // H_t of the tile's last step
    }

    // Each batch's (delta, x, dy, delta x) and c are read from LDS one batch ahead, and a
    // scheduling barrier keeps those reads at the top of the batch before: left to itself
    // the compiler issues them just before their use, and every batch then waits out the
    // LDS latency (8x2048x768x16 fp32: 172 -> 165 us per backward call).
    float4 in_next[S];
    float cv_next[S][K];
    auto load_batch_inputs = [&](int t0) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        in_next[s] = s_in[(t0 + s) * CPW + ch];
        lds_load_vec<K>(&s_c[(t0 + s) * DS + j * K], cv_next[s]);
      }
    };
    load_batch_inputs((NSUB - 1) * HB + (NBAT - 1) * S);
#pragma unroll
    for (int sb = NSUB - 1; sb >= 0; --sb) {
      if constexpr (!HF) {
        park_hblock(hq);  // this sub-block's H rows, loaded during the previous one
        if (sb > 0)
          load_hblock(hq, ts + (sb - 1) * HB, true);
        else
          load_hblock(hq, ts - TB + (NSUB - 1) * HB, it > 0);
      }
      float aq[HFIRST ? HB - 1 : 1][K];  // decays of the sub-block's steps but the last
      if constexpr (HFIRST) {
        // only the row entering the sub-block was loaded: the states after its steps are
        // formed from it exactly as the forward formed them (same operations, same inputs)
        const bool first = ts + sb * HB == 0;  // step 0 of the sequence: H_{-1} = h0
#pragma unroll
        for (int i = 0; i < K; ++i) hb[0][i] = first ? hzero[i] : hb[0][i];
#pragma unroll
        for (int r = 1; r < HB; ++r) {
          const int tq = sb * HB + r - 1;
          const float4 inq = s_in[tq * CPW + ch];
          float bq[K];
          lds_load_vec<K>(&s_b[tq * DS + j * K], bq);
#pragma unroll
          for (int i = 0; i < K; ++i) {
            aq[r - 1][i] = exp2_hw(inq.x * A2[i]);
            hb[r][i] = fmaf(aq[r - 1][i], hb[r - 1][i], inq.w * bq[i]);
          }
        }
      }

#pragma unroll
      for (int bt = NBAT - 1; bt >= 0; --bt) {
        const int tt0 = sb * HB + bt * S;  // first step of the batch within the tile
        // phase A: decays of the batch
        float a[S][K], g[S][K], cv[S][K];
        float4 in[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          in[s] = in_next[s];
#pragma unroll
          for (int i = 0; i < K; ++i) cv[s][i] = cv_next[s][i];
        }
        if (sb > 0 || bt > 0) {  // the batch after this one in the sweep (the step before it)
          load_batch_inputs(bt > 0 ? tt0 - S : (sb - 1) * HB + (NBAT - 1) * S);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
#pragma unroll
          for (int i = 0; i < K; ++i)
            a[s][i] = HF ? at[tt0 + s][i] : ((HFIRST && bt < HB - 1) ? aq[HFIRST ? bt : 0][i] : exp2_hw(in[s].x * A2[i]));
        }
        // phase B: the adjoint carry, last step first; a[s] becomes the carry a_t g_t
#pragma unroll
        for (int s = S - 1; s >= 0; --s) {
#pragma unroll
          for (int i = 0; i < K; ++i) {
            g[s][i] = fmaf(in[s].z, cv[s][i], G[i]);
            G[i] = a[s][i] * g[s][i];
            a[s][i] = G[i];
          }
        }
        // phase C: gradient terms of each step
        float Sl[S], gdl[S], gbv[S][K], gcv[S][K];
        float hrow[S][K];  // H_{t-1} of the batch's steps
#pragma unroll
        for (int s = 0; s < S; ++s) {
          if constexpr (HF) {
#pragma unroll
            for (int i = 0; i < K; ++i) hrow[s][i] = hrec[tt0 + s][i];
          } else if constexpr (HDIRECT) {
#pragma unroll
            for (int i = 0; i < K; ++i) hrow[s][i] = hb[bt * S + s][i];
          } else {
            lds_load_vec<K>(&hblk[(bt * S + s) * WROW + lane * K], hrow[s]);
          }
        }
        if (!HF && bt == 0) {
          const bool first = ts + sb * HB == 0;  // step 0 of the sequence: H_{-1} = h0
#pragma unroll
          for (int i = 0; i < K; ++i) hrow[0][i] = first ? hzero[i] : hrow[0][i];
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
          float bv[K];
          lds_load_vec<K>(&s_b[(tt0 + s) * DS + j * K], bv);
          const float(&hp)[K] = hrow[s];                                     // H_{t-1}
          const float(&ht)[K] = (s == S - 1) ? hcur : hrow[s + 1];           // H_t
          float sl = 0.f, gd = 0.f;
#pragma unroll
          for (int i = 0; i < K; ++i) {
            sl = fmaf(g[s][i], bv[i], sl);
            const float q = a[s][i] * hp[i];
            gd = fmaf(Av[i], q, gd);
            gA[i] = fmaf(in[s].x, q, gA[i]);
            gbv[s][i] = g[s][i] * in[s].w;
            gcv[s][i] = in[s].z * ht[i];
          }
          Sl[s] = sl;
          gdl[s] = gd;
        }
#pragma unroll
        for (int i = 0; i < K; ++i) hcur[i] = hrow[0][i];
        // phase D: sums over each channel's states -> gx, gdelta.  The (Sl, gdl) pairs of
        // the whole batch are reduce-scattered over the channel's lanes, so that the
        // stages carry independent adds instead of one dependent chain per step.
        {
          constexpr int V = 2 * S;
          constexpr int CF = V / L > 1 ? V / L : 1;  // items each lane finishes
          float red[V];
#pragma unroll
          for (int s = 0; s < S; ++s) { red[2 * s] = Sl[s]; red[2 * s + 1] = gdl[s]; }
          int idx0 = 0;
          if constexpr (L > 1) reduce_scatter<L / 2, V, V>(red, j, idx0);
          if constexpr (CF == 1) {
            // lanes that differ only in the bits below MP hold the same item; the lane
            // across bit MP holds the other half of the step's pair
            constexpr int MP = L / V;
            const float other = dpp<pair_ctrl<MP>()>(red[0]);
            const bool second = (idx0 & 1) != 0;
            if (!second && (j & (MP - 1)) == 0) {
              const int tr = (tt0 + (idx0 >> 1)) * CPW + ch;
              // with one step per batch the item is the batch's own step, already in registers
              const float4 v = S == 1 ? in[0] : s_in[tr];
              s_gxd[tr] = make_float2(v.x * red[0], fmaf(v.y, red[0], other));
            }
          } else {
#pragma unroll
            for (int r = 0; r < CF / 2; ++r) {
              const int tr = (tt0 + (idx0 >> 1) + r) * CPW + ch;
              const float4 v = s_in[tr];
              s_gxd[tr] = make_float2(v.x * red[2 * r], fmaf(v.y, red[2 * r], red[2 * r + 1]));
            }
          }
        }
        // phase E: sums over the channels of the wave -> one (gb, gc) slot per wave
        if constexpr (L == 4 && K == 4 && S == 1) {
          // Four lanes per channel: the four channels of a 16-lane row sit in its four DPP
          // banks.  Reduce-scatter the 8 values of each lane over the banks with bank-masked
          // DPP adds (each bank keeps one state; no selects), then over the wave's rows.
          bank_reduce_scatter(gbv[0], gcv[0]);
          const float v = rows_pair_sum(gbv[0][0], gcv[0][0]);
          const int n = j * K + ((lane >> 2) & 3);
          s_red[(row >> 1) * (NWAVE * BC) + wave * BC + tt0 * DS + n] = v;
        } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
#pragma unroll
          for (int i = 0; i < K; ++i) {
            gbv[s][i] = row_channel_sum<L>(gbv[s][i]);
            gcv[s][i] = row_channel_sum<L>(gcv[s][i]);
          }
        }
#pragma unroll
        for (int it2 = 0; it2 < NITEM; it2 += 2) {
          const int s_a = it2 / K, i_a = it2 % K;
          const int s_b2 = (it2 + 1) / K, i_b = (it2 + 1) % K;
          const float v = rows_reduce_scatter(gbv[s_a][i_a], gcv[s_a][i_a], gbv[s_b2][i_b], gcv[s_b2][i_b]);
          const int sel = row & 1;
          const int ss = sel ? s_b2 : s_a;
          const int ii = sel ? i_b : i_a;
          s_red[(row >> 1) * (NWAVE * BC) + wave * BC + (tt0 + ss) * DS + j * K + ii] = v;
        }
        }
      }
    }

    __syncthreads();
    {
      const int rows = min(TB, t_hi - ts);
      const rsrc_t rGX = make_rsrc(gxrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * 4u);
      const rsrc_t rGD = make_rsrc(gdrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * 4u);
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float2 v = s_gxd[tid + e * kThreads];
        float gxo = v.x, gdo = v.y;
        if constexpr (MAMBA) {
          const float4 in4 = s_in[tid + e * kThreads];  // (delta, x, dy, delta x); 0 when padded
          gxo = fmaf(in4.z, dskip, gxo);
          gdo *= s_sig[tid + e * kThreads];
          accD = fmaf(in4.z, in4.y, accD);
        }
        const uint32_t off = xoff[e] == kOutOfRange ? kOutOfRange : xoff[e] / ES * 4u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gxo), rGX, off, 0, kNonTemporal);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gdo), rGD, off, 0, kNonTemporal);
      }
      const rsrc_t rP = make_rsrc(p.part_bc + ((int64_t)dtile * p.B + bb) * T * DS + (int64_t)ts * DS,
                                  static_cast<uint32_t>(rows * DS) * 8u);
#pragma unroll
      for (int e = 0; e < PER_BC; ++e) {
        const int idx = tid + e * kThreads;
        const int ridx = (BC % kThreads == 0 || idx < BC) ? idx : 0;
        float sb = s_red[ridx], sc = s_red[NWAVE * BC + ridx];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) {
          sb += s_red[w * BC + ridx];
          sc += s_red[NWAVE * BC + w * BC + ridx];
        }
        const uint32_t off = (BC % kThreads == 0 || idx < BC) ? static_cast<uint32_t>(idx) * 8u : kOutOfRange;
        float v2[2] = {sb, sc};
        buf_store_vec<2>(rP, off, v2);
      }
    }
    store_tile();  // the inputs of the tile before this one (zeros before the chunk start)
  }

  if constexpr (MAMBA) {
    if (p.part_D != nullptr) {
      // channel sums of dy * x for gDskip: the 256/CPW threads of a channel, in a fixed order
      s_acc[tid] = accD;
      __syncthreads();
      if (tid < CPW && d0 + tid < D) {
        float sacc = 0.f;
#pragma unroll
        for (int k = 0; k < kThreads / CPW; ++k) sacc += s_acc[tid + k * CPW];
        p.part_D[((int64_t)chunk * p.B + bb) * D + d0 + tid] = sacc;
      }
    }
  }

  if (!dvalid) return;
  float* pa = p.part_A + (int64_t)chunk * nstate + soff;
#pragma unroll
  for (int i = 0; i < K; ++i) pa[i] = gA[i];
  if (p.gh0 != nullptr && chunk == 0) {
    float* g0 = p.gh0 + soff;
#pragma unroll
    for (int i = 0; i < K; ++i) g0[i] = G[i];
  }
}

// Local pass of the two-level reverse sweep.  The chunks 1..C-1 of the sweep are split
// into `subs` sub-chunks each, so that this pass has several times the sweep's parallelism;
// every sub-chunk runs its steps from a zero adjoint and records, per (b, d, n), its decay
// product exp(A * sum(delta)) and the carry it hands to the sub-chunk before it.  The carry
// map of a sub-chunk is G -> P G + Gloc; each workgroup of the sweep composes the maps of
// the sub-chunks after its chunk, right to left from dhT.
template <typename IO, int DS, int L, bool MAMBA>
__global__ __launch_bounds__(kThreads) void bwd_local_kernel(const BwdParams p) {
  constexpr int K = DS / L;
  constexpr int CPW = kThreads / L;
  constexpr int TB = (2048 / CPW) < 64 ? (2048 / CPW) : 64;  // 16 KiB of staged (delta, dy) at most
  constexpr int TILE = TB * CPW;
  constexpr int PER = TILE / kThreads;
  constexpr int BC = TB * DS;
  constexpr int PER_BC = (BC + kThreads - 1) / kThreads;
  constexpr int S = (32 / K) < 1 ? 1 : ((32 / K) < TB ? (32 / K) : TB);  // steps per batch
  constexpr uint32_t ES = sizeof(IO);
  static_assert(TILE % kThreads == 0 && TB % S == 0, "tile shape");

  __shared__ float2 s_dd[TILE];  // (delta, dy) at [step*CPW + channel]
  __shared__ float s_c[BC];

  const int lin = xcd_grouped(blockIdx.x, gridDim.x, p.xcd_group);
  const int dtile = lin % p.ntiles_d;
  const int rest = lin / p.ntiles_d;
  const int bb = rest % p.B;
  const int sub = p.subs + rest / p.B;  // sub-chunk index; those of chunk 0 are not needed

  const int tid = threadIdx.x;
  const int ch = tid / L;
  const int j = tid % L;
  const int d0 = dtile * CPW;
  const int D = p.D;
  const int t_lo = min(p.T, sub * p.sub_len);
  const int t_hi = min(p.T, t_lo + p.sub_len);
  const int d = d0 + ch;
  const bool dvalid = d < D;
  const int64_t nstate = (int64_t)p.B * D * DS;
  const int64_t soff = ((int64_t)bb * D + d) * DS + j * K;

  const IO* drow = static_cast<const IO*>(p.delta) + (int64_t)bb * p.x_bs;
  const IO* yrow = static_cast<const IO*>(p.dy) + (int64_t)bb * p.x_bs;
  const IO* crow = static_cast<const IO*>(p.c) + (int64_t)bb * p.bc_bs;

  float A2[K], G[K];
  if (dvalid) {
    load_k<K>(p.A + (int64_t)d * DS + j * K, A2);
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) A2[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if constexpr (MAMBA) A2[i] = dvalid ? -expf(A2[i]) : 0.f;
    A2[i] *= kLog2e;
    G[i] = 0.f;
  }
  double dsum = 0.0;

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
  float rd[PER], ry[PER], rc[PER_BC];
  int pend_rows = 0;
  auto load_tile = [&](int ts) {
    const int rows = min(TB, t_hi - ts);
    pend_rows = rows;
    const rsrc_t rD = make_rsrc(drow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rY = make_rsrc(yrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
    const rsrc_t rC = make_rsrc(crow + (int64_t)ts * DS, static_cast<uint32_t>(rows * DS) * ES);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      rd[e] = buf_load_elem<IO>(rD, xoff[e]);
      ry[e] = buf_load_elem<IO>(rY, xoff[e]);
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) rc[e] = buf_load_elem<IO>(rC, bcoff[e]);
  };

  const int ntiles = t_hi > t_lo ? (t_hi - t_lo + TB - 1) / TB : 0;
  if (ntiles > 0) load_tile(t_lo + (ntiles - 1) * TB);
  for (int it = ntiles - 1; it >= 0; --it) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float dl = rd[e];
      if constexpr (MAMBA) {
        const float keep = ((tid + e * kThreads) / CPW < pend_rows && xoff[e] != kOutOfRange) ? 1.f : 0.f;
        dl = softplus_th(rd[e]) * keep;
      }
      s_dd[tid + e * kThreads] = make_float2(dl, ry[e]);
    }
#pragma unroll
    for (int e = 0; e < PER_BC; ++e) {
      const int idx = tid + e * kThreads;
      if (BC % kThreads == 0 || idx < BC) s_c[idx] = rc[e];
    }
    __syncthreads();
    if (it > 0) load_tile(t_lo + (it - 1) * TB);
    // batches of S steps, all of a tile unrolled: each batch reads its inputs and forms
    // its decays up front, then runs the carry through them
#pragma unroll
    for (int s0 = TB - S; s0 >= 0; s0 -= S) {
      float a[S][K], cv[S][K];
      float2 dd[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        dd[s] = s_dd[(s0 + s) * CPW + ch];
        lds_load_vec<K>(&s_c[(s0 + s) * DS + j * K], cv[s]);
#pragma unroll
        for (int i = 0; i < K; ++i) a[s][i] = exp2_hw(dd[s].x * A2[i]);
      }
#pragma unroll
      for (int s = S - 1; s >= 0; --s) {
#pragma unroll
        for (int i = 0; i < K; ++i) G[i] = a[s][i] * fmaf(dd[s].y, cv[s][i], G[i]);
      }
      // the batch's delta sum as a tree in fp32 (a few ulp), then one fp64 add per batch
      float dls[S];
#pragma unroll
      for (int s = 0; s < S; ++s) dls[s] = dd[s].x;
      dsum += static_cast<double>(tree_sum<S>(dls));
    }
  }
  if (!dvalid) return;
  float2* pr = p.pairs + (int64_t)(sub - p.subs) * nstate + soff;
#pragma unroll
  for (int i = 0; i < K; ++i)
    pr[i] = make_float2(exp2_hw(static_cast<float>(static_cast<double>(A2[i]) * dsum)), G[i]);
}

// HF picks the H-free sweep; it exists only where the tile is one boundary block long.
// The local pass of the two-level sweep reads no states and is the same for both.
template <typename IO, int DS, int L, bool MAMBA, bool HF>
hipError_t launch_bwd_t(bool local_pass, const BwdParams& p, unsigned blocks, hipStream_t s) {
  if (local_pass) {
    hipLaunchKernelGGL((bwd_local_kernel<IO, DS, L, MAMBA>), dim3(blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  if constexpr (HF && bwd_tile_steps(L) != kCkptSteps) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((bwd_kernel<IO, DS, L, MAMBA, HF>), dim3(blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
}

template <typename IO, int DS, bool MAMBA, bool HF>
hipError_t launch_bwd_ds(int lanes, bool local_pass, const BwdParams& p, unsigned grid, hipStream_t s) {
  switch (lanes) {
    case 1: return launch_bwd_t<IO, DS, 1, MAMBA, HF>(local_pass, p, grid, s);
    case 2: if constexpr (DS >= 2) return launch_bwd_t<IO, DS, 2, MAMBA, HF>(local_pass, p, grid, s); break;
    case 4: if constexpr (DS >= 4) return launch_bwd_t<IO, DS, 4, MAMBA, HF>(local_pass, p, grid, s); break;
    case 8: if constexpr (DS >= 8) return launch_bwd_t<IO, DS, 8, MAMBA, HF>(local_pass, p, grid, s); break;
    case 16: if constexpr (DS >= 16) return launch_bwd_t<IO, DS, 16, MAMBA, HF>(local_pass, p, grid, s); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename IO, bool MAMBA, bool HF>
hipError_t launch_bwd_io(int DS, int lanes, bool local_pass, const BwdParams& p, unsigned grid, hipStream_t s) {
  switch (DS) {
    case 1: return launch_bwd_ds<IO, 1, MAMBA, HF>(lanes, local_pass, p, grid, s);
    case 2: return launch_bwd_ds<IO, 2, MAMBA, HF>(lanes, local_pass, p, grid, s);
    case 4: return launch_bwd_ds<IO, 4, MAMBA, HF>(lanes, local_pass, p, grid, s);
    case 8: return launch_bwd_ds<IO, 8, MAMBA, HF>(lanes, local_pass, p, grid, s);
    case 16: return launch_bwd_ds<IO, 16, MAMBA, HF>(lanes, local_pass, p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace sscan
