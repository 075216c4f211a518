// Forward selective scan, state-group layout, for gfx950 (the forward without the
// materialised states H: y, hT, the two-level scan's local pass, and the H-free path's
// boundary states).
//
// Recurrence ("pssa-100m/pssa_kernels.py" page, module docstring and scan_fwd):
//   h_t = exp(delta_t * A) * h_{t-1} + delta_t * b_t * x_t,   y_t = <h_t, c_t>.
//
// Work decomposition.  A workgroup owns one batch row and CW consecutive channels (CW =
// 64 or 32): lane l of a wave is channel d0 + l % CW, and the wave's 64/CW groups of CW
// lanes hold state groups of K states each, NG = DS/K groups over the workgroup's waves.
// Within a 16-lane row, b_t and c_t of its group's K states are the same for every lane.
// A small packing kernel lays them out per (batch row, state group) as fp32, contiguous
// over steps; each row loads its group's block of them (lane q holds floats 4q .. 4q+3 of
// a 64-float block), and every use reads the value it needs from the lane that holds it
// with a DPP row broadcast folded into the multiply (row_newbcast), so b and c cost
// neither LDS traffic nor extra instructions.  Separate reducer waves of the workgroup stage
// (delta, delta*x) of a tile once in LDS (each element converted by one thread, the softplus
// of the wrapper applied there), and every lane reads its channel's from it.  Each group
// leaves its partial sum over its K states of h * c per (step, channel) in LDS, and the
// reducer waves add the NG partials and store y coalesced while the next tile computes.
// Per (step, state) a compute lane does one v_exp_f32 and four fp32 operations, with no
// other cross-lane traffic: about 5.7 instructions per state against 7 for the lane-split
// forward, which spends 1.5 on DPP sums over a channel's lanes.
//
// Steps past the end of the chunk load delta = 0 and b = c = 0 (buffer range checks),
// which leaves the state bit-for-bit unchanged.
#pragma once
#include "device_common.h"

namespace sscan {
namespace {

// Packed b/c: element (bb, g, t, e) at ((bb * NG + g) * tpad + t) * 2K + e holds
// b[bb, t, gK + e] for e < K and c[bb, t, gK + e - K] otherwise (state group g of NG =
// DS/K); zero for t >= T.  One thread per (bb, t, g) writes its 2K floats together.
// Neighbouring threads take neighbouring state groups of a step, so a wave reads whole
// rows of b and c, each element once, and writes 64 / NG consecutive steps of each
// group's row (with steps fastest, every row of b and c is read once per group, by
// workgroups on different XCDs: 6.3 against 5.7 us at 16x4096x16 bf16; at the smaller
// sizes the kernel takes ~4.9 us either way, the latency of one cold read and write).
template <typename IO, int DS, int K>
__global__ __launch_bounds__(kThreads) void bc_pack_kernel(const FwdParams p) {
  constexpr int NG = DS / K;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)p.B * NG * p.tpad;
  if (i >= total) return;
  const int g = static_cast<int>(i % NG);
  const int64_t r = i / NG;
  const int t = static_cast<int>(r % p.tpad);
  const int64_t bb = r / p.tpad;
  float v[2 * K];
#pragma unroll
  for (int e = 0; e < 2 * K; ++e) v[e] = 0.f;
  if (t < p.T) {
    const IO* b = static_cast<const IO*>(p.b) + bb * p.bc_bs + (int64_t)t * DS + g * K;
    const IO* c = static_cast<const IO*>(p.c) + bb * p.bc_bs + (int64_t)t * DS + g * K;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      v[e] = to_f32(b[e]);
      v[K + e] = to_f32(c[e]);
    }
  }
  store_state<2 * K>(p.bcp + ((bb * NG + g) * p.tpad + t) * 2 * K, v);
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
// compiler does not fold a broadcast into an fma).  A DPP read of a register needs two wait
// states after a vector instruction writes it; c is always one of the b/c block registers,
// which only buffer loads write (the tile loop alternates two register sets instead of
// copying one into the other), so no such write can precede it.  A host test scans every
// DPP instruction of the built library for that distance.
template <int LANE>
__device__ __forceinline__ void fmac_bcast(float& acc, float c, float h) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc) : "v"(c), "v"(h), "i"(LANE));
}

// fmac_bcast with the lane given at run time; every call site passes a value that is
// constant once the step loops are unrolled, so the switch folds away.
__device__ __forceinline__ void fmac_bcast_rt(float& acc, float c, float h, int lane) {
#define SSCAN_FMAC_CASE(L) \
  case L:                  \
    fmac_bcast<L>(acc, c, h); \
    break;
  switch (lane) {
    SSCAN_FMAC_CASE(0) SSCAN_FMAC_CASE(1) SSCAN_FMAC_CASE(2) SSCAN_FMAC_CASE(3)
    SSCAN_FMAC_CASE(4) SSCAN_FMAC_CASE(5) SSCAN_FMAC_CASE(6) SSCAN_FMAC_CASE(7)
    SSCAN_FMAC_CASE(8) SSCAN_FMAC_CASE(9) SSCAN_FMAC_CASE(10) SSCAN_FMAC_CASE(11)
    SSCAN_FMAC_CASE(12) SSCAN_FMAC_CASE(13) SSCAN_FMAC_CASE(14) default: SSCAN_FMAC_CASE(15)
  }
#undef SSCAN_FMAC_CASE
}

// Reducer waves per workgroup of the state-group forward, and (step, channel) elements of
// one tile: 32 steps of 64 channels or 64 of 32.
constexpr int kSgReducerWaves = 4;
constexpr int kSgTileElems = 2048;
// store waves of the forward writing H (MODE 3)
constexpr int kSgStoreWaves = 4;

template <int DS, int K, int CW, int MODE>
__host__ __device__ constexpr int sg_threads() {
  return 64 * ((DS / K) / (64 / CW) + kSgReducerWaves + (MODE == 3 ? kSgStoreWaves : 0));
}

// MODE: 0 the two-level scan's local pass (only the chunk pair leaves the kernel), 1 y and
// hT, 2 y, hT and the H-free path's boundary states, 3 y, hT and every state H (DS = 16,
// CW = 32, two states per lane only; see below).  CW: channels per wave (64 or 32); a
// wave holds 64/CW state groups, one per CW/16 rows, so every 16-lane row belongs to a
// single group and its DPP row broadcasts stay within it.
//
// Two kinds of wave.  The compute waves (one per state group pair: NW of them) run only the
// step code: per batch of S = 4 steps, the decays and injections, the serial update, and
// the partial readouts of their K states, left as one 16-byte LDS store per lane.  The
// kSgReducerWaves reducer waves stage the inputs of the next tile (global loads of x and
// delta as raw bits, widened -- and passed through the softplus of the wrapper -- when they
// are parked in LDS) and sum the previous tile's partial readouts over the state groups into
// y.  Staged inputs and partial sums are double-buffered, so the two kinds meet at one
// barrier per tile: at tile it the compute waves read inputs buffer it % 2 and write partial
// buffer it % 2 while the reducers sum partial buffer (it-1) % 2 and fill inputs buffer
// (it+1) % 2.  The compute waves load the next tile's b/c blocks into the other of two
// register sets, so every DPP source is written by a buffer load only.  Measured against the
// same kernel with the staging and the sum over groups done by the compute waves between
// two barriers per tile: 16x4096x1024x16 bf16 292 -> 270 us, 4x2048x2048x16 bf16 90 -> 73 us
// per call, bitwise the same y and hT.
//
// MODE 3 writes H through LDS: a lane's two states of a step land 64 bytes from the next
// lane's in H, and stores of that shape run at a fraction of the HBM write rate, so each
// compute lane parks its states in a per-step row laid out as H's (the workgroup's 32
// channels x 16 states, 2 KB), and after the tile's barrier kSgStoreWaves store waves copy
// the rows to H with 16-byte stores, each wave's covering 1 KB of one row: the same
// protocol as the partial readouts, on a double buffer of 16-step tiles (with the 128-step
// x/delta staging, 160 KB of LDS in all).  The store waves issue no loads, so nothing they
// store is waited for before a load is used (a wave's memory counter retires loads and
// stores in issue order): the reducers' prefetches stay independent of the H stream.
// Within a row a channel's four 16-byte blocks of states are rotated by the channel's bits
// 2-3, so that a wave's 8-byte parking stores, which all fall in the same block of 32
// channels, spread over all 64 banks.
template <typename IO, int DS, int K, int CW, int MODE, bool MAMBA>
__global__ __launch_bounds__((sg_threads<DS, K, CW, MODE>())) void fwd_sg_kernel(const FwdParams p) {
  constexpr bool LOCAL = MODE == 0;
  constexpr bool WH = MODE == 3;        // every state to H, through LDS
  constexpr int NG = DS / K;            // state groups
  constexpr int GPW = 64 / CW;          // state groups per wave
  constexpr int NW = NG / GPW;          // compute waves
  constexpr int NTC = 64 * NW;          // compute threads
  constexpr int NTR = 64 * kSgReducerWaves;  // reducer threads
  constexpr int TB = (WH ? kSgTileElems / 4 : kSgTileElems) / CW;  // steps per tile
  constexpr int S = 4;  // steps per batch: one 16-byte store of partial readouts
  constexpr int E2 = 2 * K;
  constexpr uint32_t ES = sizeof(IO);
  constexpr int TILE = TB * CW;         // (step, channel) elements of a tile
  // x and delta are staged in tiles of GS tiles (64 or 32 steps in modes 0-2, 128 in
  // MODE 3, the 160 KB of LDS in all): fetched in MODE 3's 16-step pieces, those reads,
  // interleaved with the H stream, cut its HBM write rate by about 40%
  constexpr int GS = WH ? 8 : 1;
  constexpr int TILE_S = GS * TILE;     // (step, channel) elements of a staging tile
  constexpr int PER = TILE_S / NTR;     // elements each reducer thread stages
  constexpr int NB = TB * E2 / 64;      // 64-float blocks of packed b/c per tile
  constexpr int ITEMS = CW * (TB / 4);  // (channel, 4-step) items of a tile's readout
  // partial readouts: [group][channel][step], the 4-step blocks of a channel's row permuted
  // by its low channel bits so that a wave's 16-byte stores and loads spread over all banks
  constexpr int QM = (TB / 4 < 16 ? TB / 4 : 16) - 1;
  constexpr int PSZ = NG * CW * TB / 4;  // float4 of one partial buffer
  static_assert(CW % 16 == 0 && NG % GPW == 0 && NW >= 1, "rows of one state group");
  static_assert(TILE % NTR == 0 && TB % S == 0 && (MODE != 2 || (TB % kCkptSteps == 0 && kCkptSteps % S == 0)) &&
                    (TB * E2) % 64 == 0 && kSgTile % TB == 0,
                "tile shape");
  static_assert(!WH || (DS == 16 && K == 2 && CW == 32), "H is written for DS = 16, two states per lane, 32 channels");
  constexpr int HROW4 = CW * DS / 4;    // 16-byte blocks of one step's row of H (per workgroup)
  constexpr int NTS = 64 * kSgStoreWaves;  // store threads (MODE 3)
  // Prefetch depth of the compute waves' b/c blocks: RB - 1 tiles, 32-64 steps in every
  // mode (a load issued one 16-step tile ahead arrives after the tile that needs it started)
  constexpr int RB = WH ? 4 : 2;
  static_assert(!WH || (TB * HROW4) % NTS == 0, "a tile's rows of H are whole rounds of the store threads");
  static_assert(!WH || (GS % RB == 0 && RB * TB == kSgTile), "whole rings per staging tile");

  // (delta, delta*x) at [buffer][step*CW + channel]; with the wrapper (delta, x), so that
  // the first state group can add the skip term Dskip * x to its partial sums
  __shared__ float2 s_dw[2 * TILE_S];
  __shared__ float4 s_y[LOCAL ? 1 : 2 * PSZ];
  // MODE 3: the tile's states, [buffer][step][16-byte block], blocks rotated per channel
  __shared__ float4 s_h[WH ? 2 * TB * HROW4 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lin = blockIdx.x;
  const int dtile = lin % p.ntiles_d;
  const int rest = lin / p.ntiles_d;
  const int bb = rest % p.B;
  const int chunk = rest / p.B;
  const int D = p.D;
  const int d0 = dtile * CW;
  const int t_begin = chunk * p.chunk_len;
  const int t_end = min(p.T, t_begin + p.chunk_len);
  const int nsteps_total = t_end - t_begin;
  // MODE 3 runs a whole number of staging tiles: its unrolled tile loops then have no
  // per-tile condition, which would make the compiler wait for every load in flight where
  // the paths merge, the prefetched ones included.  The tiles added past the end (at most
  // 112 steps) read delta = 0 (their x/delta rows fall outside the resource) and b = c = 0
  // (the packing's zero padding, or zeros past the padded row), which leaves the state
  // bit-for-bit unchanged; they store nothing (no rows of y or H in range).
  const int ntiles_used = nsteps_total > 0 ? (nsteps_total + TB - 1) / TB : 0;
  const int ntiles = WH ? (ntiles_used + GS - 1) / GS * GS : ntiles_used;

  if constexpr (WH) {
    if (w >= NW + kSgReducerWaves) {
      // ---- store waves: copy each tile's parked states to H after the tile's barrier
      const int rt = tid - NTC - NTR;
      // copy tile `it`'s parked states to H.  Block q of the tile is step q / HROW4 and
      // position q % HROW4 of its row: channel cc = pos / 4 and, undoing the rotation, state
      // block (pos - cc / 4) % 4.  Rows past the chunk fall outside the resource, channels
      // past D are forced out of range.
      auto store_h = [&](int it) {
        const int ts = t_begin + it * TB;
        const int rows = tile_rows(t_end, ts, TB);  // 0 for a tile past the end
        float* Hrow = p.H + ((int64_t)bb * p.T + ts) * D * DS;
        const rsrc_t rH = make_rsrc(Hrow, static_cast<uint32_t>(rows * D * DS) * 4u);
        const float4* src = s_h + (it & 1) * (TB * HROW4);
#pragma unroll
        for (int e = 0; e < TB * HROW4 / NTS; ++e) {
          const int q = rt + e * NTS;
          const int r = q / HROW4, pos = q % HROW4;
          const int cc = pos >> 2, blk = (pos - (cc >> 2)) & 3;
          const float4 v4 = src[q];
          const float v[4] = {v4.x, v4.y, v4.z, v4.w};
          const uint32_t off =
              d0 + cc < D ? (static_cast<uint32_t>(r * D + d0 + cc) * DS + blk * 4) * 4u : kOutOfRange;
          buf_store_vec<4, kNonTemporal>(rH, off, v);
        }
      };
      for (int it = 0; it < ntiles; ++it) {
        __syncthreads();  // tile `it` computed into its buffer; tile it-1's is complete
        if (it > 0) store_h(it - 1);
      }
      if (ntiles > 0) {
        __syncthreads();
        store_h(ntiles - 1);
      }
      return;
    }
  }
  if (w >= NW) {
    // ---- reducer waves: stage the next tile, sum the previous one's partials into y
    const int rt = tid - NTC;
    const IO* xrow = static_cast<const IO*>(p.x) + (int64_t)bb * p.x_bs;
    const IO* drow = static_cast<const IO*>(p.delta) + (int64_t)bb * p.x_bs;
    IO* yrow = static_cast<IO*>(p.y) + (int64_t)bb * p.y_bs;
    // staged elements: idx = rt + e*NTR is (step idx / CW, channel idx % CW); columns past D
    // are forced out of range, rows past the chunk fall outside the resource
    uint32_t xoff[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = rt + e * NTR;
      const int dd = d0 + (idx % CW);
      xoff[e] = dd < D ? static_cast<uint32_t>((idx / CW) * D + dd) * ES : kOutOfRange;
    }
    uint32_t rx[PER], rd[PER];  // raw bits of the staging tile loaded last
    int pend_rows = 0;
    auto load_tile = [&](int ts, uint32_t (&lx)[PER], uint32_t (&ld)[PER], int& prow) {
      const int rows = tile_rows(t_end, ts, GS * TB);
      prow = rows;
      const rsrc_t rX = make_rsrc(xrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
      const rsrc_t rD = make_rsrc(drow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        lx[e] = buf_load_bits<IO>(rX, xoff[e]);
        ld[e] = buf_load_bits<IO>(rD, xoff[e]);
      }
    };
    auto store_tile = [&](int buf, const uint32_t (&lx)[PER], const uint32_t (&ld)[PER], int prow) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float xv = bits_to_f32<IO>(lx[e]);
        const float dv = bits_to_f32<IO>(ld[e]);
        // padded steps and channels keep delta = 0 (a multiply by a 0/1 mask: a select
        // lets the compiler branch around the softplus)
        const float keep = (((rt + e * NTR) / CW) < prow && xoff[e] != kOutOfRange) ? 1.f : 0.f;
        const float dl = MAMBA ? softplus_th(dv) * keep : dv;
        s_dw[buf * TILE_S + rt + e * NTR] = make_float2(dl, MAMBA ? xv : dl * xv);
      }
    };
    auto reduce_tile = [&](int it) {
      const int ts = t_begin + it * TB;
      const int rows = tile_rows(t_end, ts, TB);  // 0 for a tile past the end
      const rsrc_t rY = make_rsrc(yrow + (int64_t)ts * D, static_cast<uint32_t>(rows * D) * ES);
      const float* P = reinterpret_cast<const float*>(s_y + (it & 1) * PSZ);
#pragma unroll
      for (int i0 = 0; i0 < ITEMS; i0 += NTR) {
        // every thread stores (out of range when it has no item), so the number of
        // stores in flight does not depend on the thread
        const int item = i0 + rt;
        const bool act = ITEMS % NTR == 0 || item < ITEMS;
        const int cc = item % CW;            // channel
        const int q4 = act ? item / CW : 0;  // 4-step block
        const float* src = P + cc * TB + 4 * (q4 ^ (cc & QM));
        float4 acc = *reinterpret_cast<const float4*>(src);
#pragma unroll
        for (int gg = 1; gg < NG; ++gg) {
          const float4 v = *reinterpret_cast<const float4*>(src + gg * CW * TB);
          acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        // one value per step row; lanes hold consecutive channels, so each store is
        // coalesced; rows past the tile fall outside the resource
        const int dd = d0 + cc;
        const uint32_t off = (act && dd < D) ? static_cast<uint32_t>(4 * q4 * D + dd) * ES : kOutOfRange;
        const uint32_t row = static_cast<uint32_t>(D) * ES;
        buf_store_io<IO>(rY, off, acc.x);
        buf_store_io<IO>(rY, off == kOutOfRange ? off : off + row, acc.y);
        buf_store_io<IO>(rY, off == kOutOfRange ? off : off + 2 * row, acc.z);
        buf_store_io<IO>(rY, off == kOutOfRange ? off : off + 3 * row, acc.w);
      }
    };
    if (ntiles > 0) {
      load_tile(t_begin, rx, rd, pend_rows);
      store_tile(0, rx, rd, pend_rows);
      load_tile(t_begin + GS * TB, rx, rd, pend_rows);  // zeros past the end of the chunk
    }
    // unrolled by GS: the staging tile j + 1 is parked during the last tile of staging tile j
    // (a condition known at compile time, so the loads' waits stay exact)
    for (int it0 = 0; it0 < ntiles; it0 += GS) {
#pragma unroll
      for (int u = 0; u < GS; ++u) {
        const int it = it0 + u;
        if (WH || it < ntiles) {  // WH: ntiles is a multiple of GS
          __syncthreads();  // tile `it` staged; its partial buffer's previous contents summed
          if constexpr (!LOCAL) {
            if (it > 0) reduce_tile(it - 1);
          }
          if (u == GS - 1) {
            const int j = it0 / GS + 1;  // the staging tile after the current one
            store_tile(j & 1, rx, rd, pend_rows);
            load_tile(t_begin + (j + 1) * GS * TB, rx, rd, pend_rows);
          }
        }
      }
    }
    if (ntiles > 0) {
      __syncthreads();  // the last tile's partials
      if constexpr (!LOCAL) reduce_tile(ntiles - 1);
    }
    return;
  }

  // ---- compute waves
  const int c = lane % CW;              // this lane's channel within the workgroup
  const int grp = w * GPW + lane / CW;  // this lane's state group
  const int d = d0 + c;
  const bool dvalid = d < D;
  // the packed b/c rows of this batch row; lane q of each 16-lane row loads floats
  // 4q .. 4q+3 of every 64-float block of its group's row
  const rsrc_t rBC = make_rsrc(p.bcp + (int64_t)bb * NG * p.tpad * E2, static_cast<uint32_t>(NG * p.tpad * E2) * 4u);
  const uint32_t bcrow = static_cast<uint32_t>(grp * p.tpad * E2) * 4u + static_cast<uint32_t>(lane & 15) * 16u;

  const int64_t nstate = (int64_t)p.B * D * DS;
  const int64_t soff = ((int64_t)bb * D + d) * DS + grp * K;  // this lane's states in (B,D,DS)
  // boundary states of this batch row, addressed per tile from the tile's first block
  const float* ckrow = MODE == 2 ? p.hck + (int64_t)bb * p.nck * D * DS : nullptr;
  constexpr int kCkBlocks = TB / kCkptSteps;

  float A2[K], h[K];
  if (dvalid) {
    lds_load_vec<K>(p.A + (int64_t)d * DS + grp * K, A2);
#pragma unroll
    for (int i = 0; i < K; ++i) A2[i] = (MAMBA ? -expf(A2[i]) : A2[i]) * kLog2e;
    if (LOCAL || (chunk == 0 && p.h0 == nullptr)) {
#pragma unroll
      for (int i = 0; i < K; ++i) h[i] = 0.f;
    } else {
      // h0, then left to right the (decay product, local end state) pair of every chunk
      // before this one: h <- P h + hloc
      if (p.h0 != nullptr) {
        lds_load_vec<K>(p.h0 + soff, h);
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
  // the skip weight of this lane's channel (used by the first state group)
  const float dskip = (MAMBA && !LOCAL && grp == 0 && p.Dskip != nullptr && dvalid) ? p.Dskip[d] : 0.f;

  auto load_bc = [&](int ts, float (&dst)[NB][4]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      // blocks at or past the padded row length load zeros (not the next group's values,
      // which MODE 3's added tiles would otherwise multiply by delta = 0: a non-finite b
      // there would make the state NaN)
      const bool in_row = ts + k * (64 / E2) < p.tpad;
      const uint32_t off = in_row ? bcrow + static_cast<uint32_t>(ts) * E2 * 4u + k * 256u : kOutOfRange;
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rBC, off, 0, 0);
      dst[k][0] = __uint_as_float(t[0]); dst[k][1] = __uint_as_float(t[1]);
      dst[k][2] = __uint_as_float(t[2]); dst[k][3] = __uint_as_float(t[3]);
    }
  };
  // b/c blocks: a ring of RB register sets, tile j in set j % RB; each tile loads tile
  // it + RB - 1 into the set tile it - 1 used (only buffer loads write these registers)
  float bcr[RB][NB][4];
#pragma unroll
  for (int k = 0; k + 1 < RB; ++k)
    if (ntiles > 0) load_bc(t_begin + k * TB, bcr[k]);

  auto do_tile = [&](int it, const float (&bcv)[NB][4], float (&bcw)[NB][4]) {
    const int ts = t_begin + it * TB;
    const int buf = it & 1;
    const int kb0 = ts / kCkptSteps;  // first boundary block of the tile
    const rsrc_t rCk = make_rsrc(MODE == 2 ? ckrow + (int64_t)kb0 * D * DS : nullptr,
                                 MODE == 2 ? static_cast<uint32_t>(min(p.nck - kb0, kCkBlocks) * D * DS) * 4u : 0u);
    __syncthreads();  // this tile's inputs are staged; the partial buffer it writes is free
    load_bc(ts + (RB - 1) * TB, bcw);
    const float2* DW = s_dw + ((it / GS) & 1) * TILE_S + (it % GS) * TILE;
    float* const sy = reinterpret_cast<float*>(s_y + (LOCAL ? 0 : buf * PSZ)) + (grp * CW + c) * TB;
    float* const shw = reinterpret_cast<float*>(s_h + (WH ? buf * (TB * HROW4) : 0)) +
                       (WH ? c * DS + ((((grp >> 1) + (c >> 2)) & 3) << 2) + ((grp & 1) << 1) : 0);

    float2 dwc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) dwc[s] = DW[s * CW + c];
#pragma unroll
    for (int s0 = 0; s0 < TB; s0 += S) {
      float2 dwn[S];  // the next batch's inputs, read while this one computes
      if (s0 + S < TB) {
#pragma unroll
        for (int s = 0; s < S; ++s) dwn[s] = DW[(s0 + S + s) * CW + c];
        // With 32-channel workgroups (chosen below 256 workgroups of 64, so at most about
        // one compute wave per SIMD) keep these reads at the top of the batch: left to
        // itself the compiler issues them at its end, just before their use, and the LDS
        // latency then stalls a SIMD that has no other compute wave (4x2048x2048 bf16 per
        // call -4.5%, the forward keeping boundary states -3%).  With two waves per SIMD,
        // and in MODE 3, the fence costs more than it gains (+3-4%).
        if constexpr (CW == 32 && !WH) __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (MODE == 2) {
        // the state entering every kCkptSteps-step block: tiles start on multiples of the
        // block length, so block starts are fixed batches of the tile; the store is
        // unconditional (out of range past the chunk), so the wait counts stay the same on
        // every path
        if (s0 % kCkptSteps == 0) {  // a constant once the batch loop is unrolled
          const bool ok = dvalid && ts + s0 < t_end;
          buf_store_vec<K>(rCk, ok ? static_cast<uint32_t>((((ts + s0) / kCkptSteps - kb0) * D + d) * DS + grp * K) * 4u
                                   : kOutOfRange, h);
        }
      }
      float xs[S];  // with the wrapper: x of the step (dwc[s].y becomes delta * x)
#pragma unroll
      for (int s = 0; s < S; ++s) {
        xs[s] = dwc[s].y;
        if constexpr (MAMBA) dwc[s].y *= dwc[s].x;
      }
      (void)xs;
      float a[S][K], u[S][K];
#pragma unroll
      for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const int q = (s0 + s) * E2 + i;  // b_i of this step in the tile's packed floats
          a[s][i] = exp2_hw(dwc[s].x * A2[i]);
          u[s][i] = dwc[s].y * row_bcast(bcv[q / 64][q % 4], (q % 64) / 4);
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
      if constexpr (WH) {
        // the batch's states into the tile's rows of H (block grp / 2 of the channel,
        // rotated by its bits 2-3; the half grp % 2 of the block)
#pragma unroll
        for (int s = 0; s < S; ++s)
          *reinterpret_cast<float2*>(shw + (s0 + s) * (HROW4 * 4)) = make_float2(a[s][0], a[s][1]);
      }
      if constexpr (LOCAL) {
        float dls[S];
#pragma unroll
        for (int s = 0; s < S; ++s) dls[s] = dwc[s].x;
        dsum += static_cast<double>(tree_sum<S>(dls));
      } else {
        float yp[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int q0 = (s0 + s) * E2 + K;  // c_0 of this step
          yp[s] = row_bcast(bcv[q0 / 64][q0 % 4], (q0 % 64) / 4) * a[s][0];
#pragma unroll
          for (int i = 1; i < K; ++i) {
            const int q = q0 + i;  // c_i
            fmac_bcast_rt(yp[s], bcv[q / 64][q % 4], a[s][i], (q % 64) / 4);
          }
          if constexpr (MAMBA) yp[s] = fmaf(dskip, xs[s], yp[s]);  // the skip term (dskip = 0 past the first group)
        }
        *reinterpret_cast<float4*>(sy + 4 * ((s0 / 4) ^ (c & QM))) = make_float4(yp[0], yp[1], yp[2], yp[3]);
      }
      if (s0 + S < TB) {
#pragma unroll
        for (int s = 0; s < S; ++s) dwc[s] = dwn[s];
      }
    }
  };

  for (int it = 0; it < ntiles; it += RB) {
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (WH || it + u < ntiles) do_tile(it + u, bcr[u], bcr[(u + RB - 1) % RB]);  // WH: ntiles % RB == 0
  }
  if (ntiles > 0) __syncthreads();  // the reducers' last barrier: this tile's partials are complete

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
  constexpr int NG = DS / K;
  const int64_t npack = (int64_t)p.B * NG * p.tpad;
  if (npack > 0)
    hipLaunchKernelGGL((bc_pack_kernel<IO, DS, K>), dim3((unsigned)((npack + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int DS, int K, int CW, bool MAMBA>
hipError_t launch_fwd_sg_t(bool local_pass, const FwdParams& p, unsigned blocks, hipStream_t s) {
  constexpr int NT = sg_threads<DS, K, CW, 0>();
  if (local_pass)
    hipLaunchKernelGGL((fwd_sg_kernel<IO, DS, K, CW, 0, MAMBA>), dim3(blocks), dim3(NT), 0, s, p);
  else if (p.H != nullptr) {
    if constexpr (DS == 16 && K == 2 && CW == 32)
      hipLaunchKernelGGL((fwd_sg_kernel<IO, DS, K, CW, 3, MAMBA>), dim3(blocks), dim3(sg_threads<DS, K, CW, 3>()), 0,
                         s, p);
    else
      return hipErrorInvalidValue;
  } else if (p.hck != nullptr)
    hipLaunchKernelGGL((fwd_sg_kernel<IO, DS, K, CW, 2, MAMBA>), dim3(blocks), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_sg_kernel<IO, DS, K, CW, 1, MAMBA>), dim3(blocks), dim3(NT), 0, s, p);
  return hipGetLastError();
}

// Dispatch on DS and the channels per wave (io: 0 fp32, 1 bf16).
template <bool MAMBA, int CW>
hipError_t launch_fwd_sg_cw(int io, int DS, bool local_pass, const FwdParams& p, unsigned blocks, hipStream_t s) {
  switch (DS) {
    case 4:
      return io == 0 ? launch_fwd_sg_t<float, 4, kSgK, CW, MAMBA>(local_pass, p, blocks, s)
                     : launch_fwd_sg_t<bf16_t, 4, kSgK, CW, MAMBA>(local_pass, p, blocks, s);
    case 8:
      return io == 0 ? launch_fwd_sg_t<float, 8, kSgK, CW, MAMBA>(local_pass, p, blocks, s)
                     : launch_fwd_sg_t<bf16_t, 8, kSgK, CW, MAMBA>(local_pass, p, blocks, s);
    case 16:
      return io == 0 ? launch_fwd_sg_t<float, 16, kSgK, CW, MAMBA>(local_pass, p, blocks, s)
                     : launch_fwd_sg_t<bf16_t, 16, kSgK, CW, MAMBA>(local_pass, p, blocks, s);
    default:
      return hipErrorInvalidValue;
  }
}

template <bool MAMBA>
hipError_t launch_fwd_sg_io(int io, int DS, int cw, bool local_pass, const FwdParams& p, unsigned blocks,
                            hipStream_t s) {
  switch (cw) {
    case 64: return launch_fwd_sg_cw<MAMBA, 64>(io, DS, local_pass, p, blocks, s);
    case 32: return launch_fwd_sg_cw<MAMBA, 32>(io, DS, local_pass, p, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace sscan
