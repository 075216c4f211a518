// Internal definitions shared by the host side and the gfx950 kernels of libsscan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sscan {

constexpr int kThreads = 256;  // every kernel runs 256-thread workgroups (4 wave64)
constexpr int kCkptSteps = 32;  // steps between the boundary states of the H-free path
// State-group forward: steps per tile (its two-level scan's chunks are whole tiles) and
// states per lane (a workgroup has DS/kSgK waves of 64 channels).
constexpr int kSgTile = 64;
constexpr int kSgK = 2;

// Storage type for bf16 I/O: the raw 16 bits.
struct bf16_t {
  uint16_t bits;
};

// Steps staged per tile.  The forward stages (delta, delta*x) per (step, channel),
// 4096 of them per tile, at most 64 steps; the backward stages (delta, x, dy, delta*x),
// 1024 per tile, at most 32 steps.  Both keep a workgroup's LDS under 64 KiB.
__host__ __device__ constexpr int fwd_tile_steps(int lanes) {
  return (4096 / (kThreads / lanes)) < 64 ? (4096 / (kThreads / lanes)) : 64;
}
// Steps per tile of the backward sweep: 4 KiB of staged (delta, x, dy, delta x) rows per
// workgroup, at most 32; with four lanes per channel 8 steps, which keeps the unrolled tile
// (four states per lane, four-row H blocks) within the registers of three waves per SIMD.
__host__ __device__ constexpr int bwd_tile_steps(int lanes) {
  return lanes == 4 ? 8 : (1024 / (kThreads / lanes)) < 32 ? (1024 / (kThreads / lanes)) : 32;
}

struct FwdParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* b;
  const void* c;
  const float* h0;     // may be null
  void* y;             // may be null only in the local pass
  float* hT;           // may be null
  float* H;            // may be null
  float2* pairs;       // two-level scan: (decay product, local end state) per chunk, (C-1,B,D,DS)
  const float* Dskip;  // Mamba wrapper: per-channel skip weight (D,), may be null (no skip)
  float* hck;          // H-free path: state entering every kCkptSteps-step block, (B,nck,D,DS), or null
  int32_t nck;         // ceil(T / kCkptSteps)
  float* bcp;          // state-group forward: packed fp32 b/c, (B, DS/K, tpad, 2K)
  int32_t tpad;        // state-group forward: steps of bcp per row (T rounded up to whole tiles)
  int64_t x_bs;        // batch stride of x, delta (elements)
  int64_t bc_bs;       // batch stride of b, c (elements)
  int64_t y_bs;        // batch stride of y (elements)
  int32_t B, T, D;
  int32_t chunk_len;   // steps per chunk (T when there is a single chunk)
  int32_t chunks;      // number of chunks C
  int32_t ntiles_d;    // channel tiles per batch row
  int32_t xcd_group;   // consecutive channel tiles kept on one XCD
};

struct BwdParams {
  const void* dy;
  const float* dhT;    // may be null
  const void* x;
  const void* delta;
  const float* A;
  const void* b;
  const void* c;
  const float* h0;     // may be null
  const float* H;
  float* gx;
  float* gdelta;
  float* gh0;          // may be null
  float2* part_bc;     // (ntiles_d, B, T, DS): per-workgroup (gb, gc) partial sums
  float* part_A;       // (chunks, B, D, DS): per-(chunk, batch row) gA partial sums
  float2* pairs;       // two-level sweep: (decay product, local carry) of the sub-chunks of chunks
                       // 1..C-1, ((C-1)*subs,B,D,DS)
  const float* Dskip;  // Mamba wrapper: per-channel skip weight (D,), may be null (zero)
  float* part_D;       // Mamba wrapper: per-(chunk, batch row) partial sums of dy*x, (chunks,B,D), or null
  const float* hck;    // H-free sweep: state entering every kCkptSteps-step block, (B,nck,D,DS)
  int32_t nck;         // ceil(T / kCkptSteps)
  int64_t x_bs;        // x, delta, dy
  int64_t bc_bs;       // b, c
  int64_t y_bs;        // gx, gdelta
  int32_t B, T, D;
  int32_t ntiles_d;
  int32_t xcd_group;
  int32_t chunk_len;   // steps per chunk, a multiple of the tile
  int32_t chunks;
  int32_t subs;        // two-level sweep: sub-chunks per chunk in the local pass (divides chunk_len)
  int32_t sub_len;     // chunk_len / subs
};

struct ReduceParams {
  const float2* part_bc;
  const float* part_A;
  float* gb;
  float* gc;
  float* gA;
  const float* A_log;   // Mamba wrapper: gA is scaled by A = -exp(A_log) (gradient for A_log); null otherwise
  const float* part_D;  // Mamba wrapper: (chunks, B, D) partials of dy*x, or null
  float* gD;            // Mamba wrapper: gradient for Dskip (D,), or null
  int32_t B, T, D, DS;
  int32_t ntiles_d;
  int32_t chunks;
};

struct DecodeParams {
  const void* x;          // (B, D) rows at b*x_bs
  const void* delta;
  const float* A;         // (D, DS)
  const void* b;          // (B, DS) rows at b*bc_bs
  const void* c;
  const float* state_in;  // (B, D, DS)
  float* state_out;       // (B, D, DS); may be state_in itself
  void* y;                // (B, D) rows at b*y_bs
  int64_t x_bs, bc_bs, y_bs;
  int32_t B, D;
};

// Launchers (defined in the .hip translation units).  Each returns a hipError_t.
// mamba: delta holds delta_raw (delta = softplus), A holds A_log (A = -exp(A_log)), and
// the skip term Dskip * x is added to y (forward) or its gradients formed (backward).
hipError_t launch_fwd(int io, int DS, int lanes, bool local_pass, bool mamba, const FwdParams& p, unsigned blocks,
                      hipStream_t s);
hipError_t launch_fwd_plain(int io, int DS, int lanes, bool local_pass, const FwdParams& p, unsigned blocks,
                            hipStream_t s);
hipError_t launch_fwd_mamba(int io, int DS, int lanes, bool local_pass, const FwdParams& p, unsigned blocks,
                            hipStream_t s);
// State-group forward (no H; DS in {4, 8, 16}, D a multiple of 4): the packing of b and c
// into p.bcp, which must precede the passes, and a pass (local or full) over workgroups of
// cw channels (64 or 32) and DS/kSgK state groups.
hipError_t launch_bc_pack(int io, int DS, const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_sg(int io, int DS, int cw, bool local_pass, bool mamba, const FwdParams& p, unsigned blocks,
                         hipStream_t s);
hipError_t launch_fwd_sg_plain(int io, int DS, int cw, bool local_pass, const FwdParams& p, unsigned blocks,
                               hipStream_t s);
hipError_t launch_fwd_sg_mamba(int io, int DS, int cw, bool local_pass, const FwdParams& p, unsigned blocks,
                               hipStream_t s);
hipError_t launch_bwd(int io, int DS, int lanes, bool local_pass, bool mamba, const BwdParams& p, unsigned blocks,
                      hipStream_t s);
hipError_t launch_bwd_plain(int io, int DS, int lanes, bool local_pass, const BwdParams& p, unsigned blocks,
                            hipStream_t s);
hipError_t launch_bwd_mamba(int io, int DS, int lanes, bool local_pass, const BwdParams& p, unsigned blocks,
                            hipStream_t s);
// The H-free sweep (boundary states in p.hck, every kCkptSteps steps); lanes must give
// kCkptSteps-step tiles.  Its local pass is launch_bwd's.
hipError_t launch_bwd_hf(int io, int DS, int lanes, bool mamba, const BwdParams& p, unsigned blocks, hipStream_t s);
hipError_t launch_bwd_reduce(const ReduceParams& p, hipStream_t s);
hipError_t launch_decode(int io, int DS, const DecodeParams& p, hipStream_t s);
hipError_t launch_fill(float* dst, int64_t n, hipStream_t s);                         // dst[i] = 0
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t s);  // src ? copy : zero

}  // namespace sscan
