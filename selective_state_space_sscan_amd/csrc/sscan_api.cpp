// libsscan host side: argument validation, plan selection, workspace layout and
// kernel launches.  Nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <limits>
#include <mutex>

#include "sscan.h"
#include "sscan_internal.h"

namespace {

using sscan::kThreads;

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return SSCAN_OK;
}

// MI355X: 256 CUs x 4 SIMDs; one wave64 per SIMD is 1024 waves, 65536 lanes.
constexpr int64_t kWavesOnePerSimd = 1024;
constexpr int64_t kLanesOneWavePerSimd = 64 * kWavesOnePerSimd;

bool valid_ds(int64_t ds) { return ds == 1 || ds == 2 || ds == 4 || ds == 8 || ds == 16; }
bool pow2_upto16(int64_t v) { return v == 1 || v == 2 || v == 4 || v == 8 || v == 16; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Resolved {
  int64_t B, T, D, DS;
  int io;
  int64_t x_bs, bc_bs, y_bs;
  size_t io_size;
};

int resolve_desc(const sscan_desc* desc, Resolved* r) {
  if (desc == nullptr) return fail(SSCAN_ERR_NULL, "desc is NULL");
  if (desc->B < 0 || desc->T < 0 || desc->D < 0)
    return fail(SSCAN_ERR_SHAPE, "negative size (B=%lld T=%lld D=%lld)", (long long)desc->B, (long long)desc->T,
                (long long)desc->D);
  if (!valid_ds(desc->DS)) return fail(SSCAN_ERR_UNSUPPORTED, "DS=%lld is not one of 1,2,4,8,16", (long long)desc->DS);
  if (desc->io != SSCAN_F32 && desc->io != SSCAN_BF16) return fail(SSCAN_ERR_DTYPE, "io dtype %d is unknown", desc->io);
  if (desc->reserved != 0) return fail(SSCAN_ERR_UNSUPPORTED, "desc.reserved must be 0");
  const int64_t i32max = std::numeric_limits<int32_t>::max();
  // Kernels address one tile of a batch row with 32-bit byte offsets: D*DS <= 2^22 keeps
  // every such offset (at most 64 steps of states) below 2^30.
  if (desc->T > i32max || desc->D * desc->DS > (int64_t(1) << 22) || desc->B > 65535)
    return fail(SSCAN_ERR_UNSUPPORTED, "sizes beyond addressing limits (B <= 65535, T < 2^31, D*DS <= 2^22)");
  r->B = desc->B;
  r->T = desc->T;
  r->D = desc->D;
  r->DS = desc->DS;
  r->io = desc->io;
  r->io_size = desc->io == SSCAN_F32 ? 4 : 2;
  const int64_t row = desc->T * desc->D;
  const int64_t bcrow = desc->T * desc->DS;
  r->x_bs = desc->x_bstride == 0 ? row : desc->x_bstride;
  r->bc_bs = desc->bc_bstride == 0 ? bcrow : desc->bc_bstride;
  r->y_bs = desc->y_bstride == 0 ? row : desc->y_bstride;
  if (r->x_bs < row) return fail(SSCAN_ERR_SHAPE, "x_bstride %lld < T*D = %lld", (long long)r->x_bs, (long long)row);
  if (r->y_bs < row) return fail(SSCAN_ERR_SHAPE, "y_bstride %lld < T*D = %lld", (long long)r->y_bs, (long long)row);
  if (r->bc_bs < bcrow)
    return fail(SSCAN_ERR_SHAPE, "bc_bstride %lld < T*DS = %lld", (long long)r->bc_bs, (long long)bcrow);
  return SSCAN_OK;
}

// Smallest lane count L (power of two, <= min(DS,16)) with B*D*L >= target lanes.
// Plan kinds: the forward, the backward, and the backward of the Mamba-style wrapper.
enum PlanKind { kPlanFwd = 0, kPlanBwd = 1, kPlanMambaBwd = 2 };

int resolve_plan(const Resolved& r, const sscan_plan* plan, PlanKind kind, int* lanes, int* chunks) {
  const bool backward = kind != kPlanFwd;
  if (plan != nullptr) {
    for (int i = 0; i < 5; ++i)
      if (plan->reserved[i] != 0) return fail(SSCAN_ERR_UNSUPPORTED, "plan.reserved must be 0");
    if (plan->layout < SSCAN_LAYOUT_AUTO || plan->layout > SSCAN_LAYOUT_STATE_GROUPS)
      return fail(SSCAN_ERR_UNSUPPORTED, "plan.layout=%d is not an sscan_layout", plan->layout);
    if (backward && plan->layout == SSCAN_LAYOUT_STATE_GROUPS)
      return fail(SSCAN_ERR_UNSUPPORTED, "the backward runs the lanes layout only");
    if (plan->lanes != 0 && (!pow2_upto16(plan->lanes) || plan->lanes > r.DS))
      return fail(SSCAN_ERR_UNSUPPORTED, "plan.lanes=%d must be a power of two <= min(DS,16)", plan->lanes);
    if (plan->chunks < 0 || plan->chunks > 65535)
      return fail(SSCAN_ERR_UNSUPPORTED, "plan.chunks=%d out of range", plan->chunks);
  }
  // Measured on MI355X: the forward runs best with 8 lanes per channel (two states per
  // lane) on every size tried; the backward, plain or wrapped, with 4 lanes (four states per
  // lane: a quarter of the per-workgroup gb/gc partials of one state per lane, and fewer
  // cross-lane sums), split along T for occupancy (8x2048x768x16: 4 lanes and 8 chunks
  // 0.268 ms, 16 lanes and 2 chunks 0.304 ms; the wrapper's 0.273 and 0.302 ms).
  // Below DS = 16 the backward also keeps four states per lane (DS/4 lanes per channel)
  // unless that leaves fewer than three waves per SIMD at 16 T-chunks, in which case it
  // takes more lanes per channel, up to DS (16x2048x2048x4 fp32: one lane and 8 chunks
  // 416 us against 519 us for four lanes and 2; 2x8192x512x8: eight lanes 125 us against
  // 166 us for four; 32x1024x1024x8 bf16: two lanes 302 against 334 us).
  int l;
  if (plan != nullptr && plan->lanes != 0) {
    l = plan->lanes;
  } else if (kind == kPlanFwd) {
    l = (int)(r.DS < 8 ? r.DS : 8);
  } else if (r.DS >= 16) {
    l = 4;
  } else if (r.DS >= 4) {
    l = (int)(r.DS / 4);
    while (l < r.DS && r.B * r.D * l * 16 < 3 * kLanesOneWavePerSimd) l *= 2;
  } else {
    l = (int)r.DS;
  }
  int c = 1;
  if (backward) {
    if (plan != nullptr && plan->chunks != 0) {
      c = plan->chunks;
    } else {
      // Split the reverse sweep until there are three waves per SIMD (at 8x2048x768x16 a
      // single pass would leave 0.375); every chunk keeps at least four tiles.
      const int64_t lanes_total = r.B * r.D * l;
      const int64_t tb = sscan::bwd_tile_steps(l);
      if (lanes_total > 0 && lanes_total < 3 * kLanesOneWavePerSimd) {
        int64_t want = ceil_div(3 * kLanesOneWavePerSimd, lanes_total);
        int64_t cap = r.T / (4 * tb);
        if (want > cap) want = cap;
        if (want > 16) want = 16;
        if (want > 1) c = (int)want;
      }
    }
    if (r.T > 0 && c > r.T) c = (int)r.T;
    if (c < 1) c = 1;
  } else {
    if (plan != nullptr && plan->chunks != 0) {
      c = plan->chunks;
    } else {
      // Split the sequence when the single pass would leave at least half of the
      // SIMDs idle, aiming at two waves per SIMD; every chunk keeps at least 128 steps.
      // The forwards writing H or keeping boundary states in the lanes layout start from
      // this count; the plain forward there takes lanes_fwd_chunks instead.
      const int64_t lanes_total = r.B * r.D * l;
      if (lanes_total > 0 && 2 * lanes_total <= kLanesOneWavePerSimd) {
        int64_t want = ceil_div(2 * kLanesOneWavePerSimd, lanes_total);
        int64_t cap = r.T / 128;
        if (want > cap) want = cap;
        if (want > 16) want = 16;
        if (want > 1) c = (int)want;
      }
    }
    if (r.T > 0 && c > r.T) c = (int)r.T;
    if (c < 1) c = 1;
  }
  *lanes = l;
  *chunks = c;
  return SSCAN_OK;
}

// T-chunks of a forward without H in the state-group layout, or 0 to leave the plan to the
// lanes layout: one pass from 512 compute waves (B * D * DS/2 lanes / 64) up; below that,
// enough chunks for about 2048 waves (two per SIMD), a power of two up to 16, as long as
// the chunks keep at least 256 steps (shorter ones, where the lanes layout's two launches
// without a packing pass are as fast or faster, go to that layout).  Measured against
// every chunk count of both layouts: 1x8192x2048x16 bf16 (256 waves per pass) 8 chunks 128
// us against 199 us for the lanes layout's choice; 4x4096x1536x8 bf16 (384) 8 chunks 118 us
// against 270; 2x8192x512x8 bf16 (64) 16 chunks 54 us against 92; 8x2048x1024x8 fp32
// (512) one pass 72 us against 114; within 8% of the fastest plan on every shape tried.
// 8x1024x256x16 fp32 (it would take 128-step chunks) stays in the lanes layout, as fast
// there (8 chunks 30 us, 8 state-group chunks 30 us) without the packing pass.
int sg_plain_chunks(const Resolved& r) {
  const int64_t waves = ceil_div(r.B * r.D * (r.DS / sscan::kSgK), 64);
  if (waves >= 512) return 1;
  int64_t c = 1;
  while (c < 16 && waves * c < 2048) c *= 2;
  const int64_t cap = r.T / 128;
  if (c > cap) c = cap;
  if (c < 2 || r.T / c < 256) return 0;
  return (int)c;
}

// T-chunks of a forward without H (or boundary states) in the lanes layout: split when one
// pass would have under one wave per SIMD.  With at most four waves per SIMD (whole
// 256-thread workgroups of 256/L channels) and at most 16 chunks, the longest chunk needs
// at least ceil(tiles / cmax) of the kernel's tiles; take the fewest chunks that reach that
// (a chunk with a partial last tile costs a whole tile, so more chunks would only add work).
// Measured (16 input copies in turn, 600 calls) against the earlier rule of two waves per
// SIMD from below half a wave: 8x1024x256x16 fp32 16 chunks 25.9 us against 8 chunks 27.2;
// 16x1024x257x8 6 chunks 44.2 against one pass 58.5; 4x4096x510x16 16 chunks 77.9 against 9
// chunks 93.2; 2x1000x64x16 16 chunks 14.7 against 7 chunks 25.8; 32x512x130x16 4 chunks
// 31.6 against one pass 37.5; equal on the other shapes tried (8x1024x258x16: 8 chunks of
// two tiles, where 14 chunks of 74 steps, also two tiles each, took 41.5 us).
int lanes_fwd_chunks(const Resolved& r, int l) {
  const int64_t cpw = kThreads / l;
  const int64_t waves = r.B * ceil_div(r.D, cpw) * (kThreads / 64);
  if (waves <= 0 || waves >= kWavesOnePerSimd || r.T <= 0) return 1;
  int64_t cmax = 4 * kWavesOnePerSimd / waves;
  if (cmax > 16) cmax = 16;
  const int64_t tb = sscan::fwd_tile_steps(l);
  const int64_t chunk = ceil_div(ceil_div(r.T, tb), cmax) * tb;  // the longest chunk, in whole tiles
  const int64_t c = ceil_div(r.T, chunk);
  return c > 1 ? (int)c : 1;
}

// The forward's plan: lanes, T-chunks, whether the state-group layout runs and its
// channels per workgroup (cw).  That layout needs DS in {4, 8, 16}, D a multiple of 4 and
// T < 2^24, and DS = 16 when it writes H (with_H; then cw = 32).  Chosen by itself for a
// single pass with at least 256 64-channel or 128 32-channel workgroups, with or without
// boundary states or H (16x4096x1024x16 bf16: 0.278 ms against 0.32 ms for lanes;
// 8x2048x768x16 fp32: 73 us against 137 us).  The forwards without H (with boundary states
// or not) run it wherever it applies unless a split into short T-chunks would be needed
// (sg_plain_chunks; keeping boundary states: 4x4096x1536x8 bf16 8 chunks 116 us against 210
// us for the lanes layout's choice, 8x2048x1024x8 fp32 one pass 77 against 120 us).
int resolve_fwd_plan(const Resolved& r, const sscan_plan* plan, bool with_H, bool with_ck, int* lanes, int* chunks,
                     bool* sg, int* cw) {
  const bool sg_ok = (r.DS == 4 || r.DS == 8 || r.DS == 16) && (!with_H || r.DS == 16) && r.D % 4 == 0 &&
                     r.T < (1 << 24);
  const int sg_lanes = (int)(r.DS / sscan::kSgK);
  const int want = plan != nullptr ? plan->layout : SSCAN_LAYOUT_AUTO;
  if (want == SSCAN_LAYOUT_STATE_GROUPS) {
    if (!sg_ok)
      return fail(SSCAN_ERR_UNSUPPORTED, "the state-group layout needs DS in {4, 8, 16} (16 when it writes H), "
                                         "D a multiple of 4 and T < 2^24");
    if (plan->lanes != 0 && plan->lanes != sg_lanes)
      return fail(SSCAN_ERR_UNSUPPORTED, "the state-group layout runs DS/2 = %d threads per channel, not %d", sg_lanes,
                  plan->lanes);
  }
  int st = resolve_plan(r, plan, kPlanFwd, lanes, chunks);
  if (st != SSCAN_OK) return st;
  const int plain_chunks = (!with_H && sg_ok && want == SSCAN_LAYOUT_AUTO &&
                            (plan == nullptr || plan->lanes == 0 || plan->lanes == sg_lanes))
                               ? (plan != nullptr && plan->chunks != 0 ? *chunks : sg_plain_chunks(r))
                               : 0;
  if (plain_chunks > 0) {
    *lanes = sg_lanes;
    *chunks = plain_chunks;
    *cw = r.B * ceil_div(r.D, 64) * *chunks >= 256 ? 64 : 32;
    *sg = true;
    return SSCAN_OK;
  }
  // a single pass of the state-group layout with enough workgroups beats every split of the
  // forward keeping boundary states (8x2048x768x16 fp32: 78 us against 110 us for the lanes
  // layout in 4 chunks; 16x4096x1024x16 bf16: 264 against 321-355 us), so that forward
  // splits only when the state-group layout cannot fill the GPU in one pass
  const bool sg_single = sg_ok && *lanes == sg_lanes && want != SSCAN_LAYOUT_LANES && (plan == nullptr || plan->chunks <= 1) &&
                         (plan == nullptr || plan->lanes == 0 || plan->lanes == sg_lanes) &&
                         (r.B * ceil_div(r.D, 64) >= 256 || r.B * ceil_div(r.D, 32) >= 128);
  if (with_ck && !sg_single && (plan == nullptr || plan->chunks == 0)) {
    // The forward keeping boundary states is bound by its per-step latency below one wave
    // per SIMD: split the sequence to three waves per SIMD, every chunk keeping at least 128
    // steps (8x2048x768x16 fp32: 4 chunks 0.119 ms, 1 chunk 0.139 ms; the forward without
    // boundary states gains under 4% there and keeps the rule above)
    const int64_t lanes_total = r.B * r.D * *lanes;
    if (lanes_total > 0 && lanes_total < kLanesOneWavePerSimd) {
      int64_t want = ceil_div(3 * kLanesOneWavePerSimd, lanes_total);
      const int64_t cap = r.T / 128;
      if (want > cap) want = cap;
      if (want > 16) want = 16;
      if (want > *chunks) *chunks = (int)want;
    }
  }
  // channels per workgroup: 64 when that gives at least 256 workgroups per pass, else 32
  // (whose four-wave workgroups measured better from 128 workgroups up: 4x2048x2048x16
  // bf16 0.115 ms against 0.125 ms for lanes and 0.150 ms with 64 channels; 8x2048x768x16
  // fp32 0.113 against 0.120 and 0.149 ms); the forward writing H runs 32 channels
  const int64_t wgs64 = r.B * ceil_div(r.D, 64) * *chunks, wgs32 = r.B * ceil_div(r.D, 32) * *chunks;
  *cw = (wgs64 >= 256 && !with_H) ? 64 : 32;
  *sg = false;
  if (want == SSCAN_LAYOUT_STATE_GROUPS) {
    *sg = true;
  } else if (want == SSCAN_LAYOUT_AUTO && sg_ok && *lanes == sg_lanes) {
    *sg = *chunks == 1 && (with_H ? wgs32 >= 128 : (wgs64 >= 256 || wgs32 >= 128));
  }
  if (*sg) *lanes = sg_lanes;
  if (!*sg && !with_H && !with_ck && (plan == nullptr || plan->chunks == 0)) *chunks = lanes_fwd_chunks(r, *lanes);
  return SSCAN_OK;
}

struct FwdLayout {
  size_t pairs_off, bc_off, total;
  int64_t tpad;  // state-group layout: steps of packed b/c per row
};

FwdLayout fwd_layout(const Resolved& r, int chunks, bool sg) {
  FwdLayout L{0, 0, 0, 0};
  const size_t nstate = (size_t)(r.B * r.D * r.DS);
  if (chunks > 1) {
    L.pairs_off = 0;
    L.total = align_up(L.pairs_off + (size_t)(chunks - 1) * nstate * sizeof(float2), 256);
  }
  if (sg) {
    L.tpad = ceil_div(r.T, sscan::kSgTile) * sscan::kSgTile;
    L.bc_off = L.total;
    L.total = align_up(L.bc_off + (size_t)(r.B * L.tpad * 2 * r.DS) * sizeof(float), 256);
  }
  return L;
}

struct BwdLayout {
  size_t bc_off, a_off, pairs_off, d_off, total;
  int64_t ntiles_d, chunk_len, chunks, subs, sub_len;
};

// Chunks of the reverse sweep are whole tiles long; the last one takes the remainder.
// The local pass splits chunks 1..C-1 into `subs` sub-chunks each (a power of two that
// divides the chunk length, sub-chunks at least 64 steps long), doubling it while the pass
// stays within about six waves per SIMD: it reads only delta, dy and c, and more
// parallelism is what it lacks.
// with_D: room for the Mamba wrapper's per-(chunk, batch row) partial sums of dy * x.
BwdLayout bwd_layout(const Resolved& r, int lanes, int chunks, bool with_D) {
  BwdLayout L{};
  const int64_t cpw = kThreads / lanes;
  const int64_t tb = sscan::bwd_tile_steps(lanes);
  L.ntiles_d = ceil_div(r.D, cpw);
  L.chunk_len = r.T > 0 ? ceil_div(ceil_div(r.T, chunks), tb) * tb : tb;
  L.chunks = r.T > 0 ? ceil_div(r.T, L.chunk_len) : 1;
  L.subs = 1;
  if (L.chunks > 1) {
    const int64_t waves = L.ntiles_d * r.B * (L.chunks - 1) * (kThreads / 64);
    while (L.subs < 8 && waves * L.subs * 2 <= 6 * 1024 && L.chunk_len % (L.subs * 2) == 0 &&
           L.chunk_len / (L.subs * 2) >= 64)
      L.subs *= 2;
  }
  L.sub_len = L.chunk_len / L.subs;
  const size_t nstate = (size_t)(r.B * r.D * r.DS);
  L.bc_off = 0;
  L.a_off = align_up((size_t)(L.ntiles_d * r.B * r.T * r.DS) * sizeof(float2), 256);
  L.pairs_off = align_up(L.a_off + (size_t)L.chunks * nstate * sizeof(float), 256);
  L.d_off = align_up(L.pairs_off + (size_t)((L.chunks - 1) * L.subs) * nstate * sizeof(float2), 256);
  L.total = with_D ? align_up(L.d_off + (size_t)(L.chunks * r.B * r.D) * sizeof(float), 256) : L.d_off;
  return L;
}

// Channel tiles whose x / delta / y rows share one 128-byte line are kept on one XCD.
int xcd_group(int lanes, size_t io_size) {
  const int64_t seg = (int64_t)(kThreads / lanes) * (int64_t)io_size;  // bytes of a tile row
  int64_t g = seg >= 128 ? 1 : 128 / seg;
  return (int)(g > 8 ? 8 : g);
}

bool misaligned(const void* p, size_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(SSCAN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Scratch of the allocation-free forward (sscan_fwd_noalloc): one array per GPU, held
// from the library's load until the process ends.  On the host, `scratch` names a
// host-side stand-in, not device memory: kernels are given the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[SSCAN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch` for work enqueued on `stream`.
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(SSCAN_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "current device");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "selecting the stream's device");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "address of the scratch array");
    if (e2 != hipSuccess) return hip_fail(e2, "restoring the current device");
    if (ptr == nullptr) return fail(SSCAN_ERR_HIP, "the scratch array has no device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SSCAN_OK;
}

// The forward, plain (mamba = false) or wrapped: delta holds delta_raw, A holds A_log and
// Dskip (may be null) adds the skip term.
// The H-free sweep takes one boundary block per tile: lanes with kCkptSteps-step tiles
// (8 or 16 lanes per channel, so DS >= 8).  Each lane keeps its tile of recomputed states
// in registers, which allows three waves per SIMD; the default T-chunk count fills them
// once (8x2048x768x16: 223 us with 2 chunks, 236 us with 4, 237 us with 8).
int resolve_hf_plan(const Resolved& r, const sscan_plan* plan, int* lanes, int* chunks) {
  if (r.DS < 8) return fail(SSCAN_ERR_UNSUPPORTED, "the H-free backward needs DS >= 8, got DS=%lld", (long long)r.DS);
  if (plan != nullptr && plan->lanes != 0 && plan->lanes < 8)
    return fail(SSCAN_ERR_UNSUPPORTED, "the H-free backward runs 8 or 16 lanes per channel, plan.lanes=%d",
                plan->lanes);
  if (*lanes < 8) *lanes = (int)(r.DS < 16 ? r.DS : 16);
  if (plan == nullptr || plan->chunks == 0) {
    const int64_t lanes_total = r.B * r.D * *lanes;
    int64_t c = lanes_total > 0 ? ceil_div(3 * kLanesOneWavePerSimd, lanes_total) : 1;
    const int64_t cap = r.T / (4 * sscan::kCkptSteps);
    if (c > cap) c = cap;
    if (c > 16) c = 16;
    *chunks = c > 1 ? (int)c : 1;
  }
  return SSCAN_OK;
}

// hck (not null): instead of H, keep the state entering every kCkptSteps-step block.
// use_scratch: ws/ws_bytes are ignored and the workspace is this device's `scratch` array
// (sscan_fwd_noalloc); a call needing more than it holds fails before any GPU call.
int fwd_impl(bool mamba, const sscan_desc* desc, const sscan_plan* plan, const void* x, const void* delta,
             const float* A, const void* b, const void* c, const float* Dskip, const float* h0, void* y, float* hT,
             float* H, float* hck, void* ws, size_t ws_bytes, hipStream_t stream, bool use_scratch = false) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  int lanes, chunks;
  bool sg;
  int cw;
  st = resolve_fwd_plan(r, plan, H != nullptr, hck != nullptr, &lanes, &chunks, &sg, &cw);
  if (st != SSCAN_OK) return st;
  if (r.B == 0 || r.D == 0) return ok();
  const bool steps = r.T > 0;
  if (steps && (x == nullptr || delta == nullptr || A == nullptr || b == nullptr || c == nullptr || y == nullptr))
    return fail(SSCAN_ERR_NULL, "x, delta, A, b, c and y are required when T > 0");
  const size_t es = r.io_size;
  if (misaligned(x, es) || misaligned(delta, es) || misaligned(b, es) || misaligned(c, es) || misaligned(y, es))
    return fail(SSCAN_ERR_ALIGN, "io tensors must be aligned to their element size");
  if (misaligned(A, 16) || misaligned(h0, 16) || misaligned(hT, 16) || misaligned(H, 16))
    return fail(SSCAN_ERR_ALIGN, "A, h0, hT and H must be 16-byte aligned");
  if (misaligned(Dskip, 4)) return fail(SSCAN_ERR_ALIGN, "Dskip must be 4-byte aligned");
  if (misaligned(hck, 16)) return fail(SSCAN_ERR_ALIGN, "hck must be 16-byte aligned");
  if (hck != nullptr && H != nullptr) return fail(SSCAN_ERR_UNSUPPORTED, "H and boundary states are alternatives");
  if (!steps) {
    if (hT == nullptr) return ok();
    const hipError_t e = sscan::launch_copy_or_zero(hT, h0, r.B * r.D * r.DS, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hT <- h0");
  }
  FwdLayout lay = fwd_layout(r, chunks, sg);
  if (use_scratch && lay.total > SSCAN_NOALLOC_SCRATCH_BYTES && sg &&
      (plan == nullptr || plan->layout == SSCAN_LAYOUT_AUTO)) {
    // the state-group layout's packed b/c does not fit the static scratch: the lanes
    // layout, which packs nothing, keeps such a call within it
    sscan_plan lp = plan != nullptr ? *plan : sscan_plan{};
    lp.layout = SSCAN_LAYOUT_LANES;
    st = resolve_fwd_plan(r, &lp, H != nullptr, hck != nullptr, &lanes, &chunks, &sg, &cw);
    if (st != SSCAN_OK) return st;
    lay = fwd_layout(r, chunks, sg);
  }
  if (use_scratch) {
    if (lay.total > SSCAN_NOALLOC_SCRATCH_BYTES)
      return fail(SSCAN_ERR_WORKSPACE, "this forward needs %zu bytes of scratch; the allocation-free entry point has %zu",
                  lay.total, (size_t)SSCAN_NOALLOC_SCRATCH_BYTES);
    ws = nullptr;
    ws_bytes = 0;
    if (lay.total > 0) {
      st = scratch_address(stream, &ws);
      if (st != SSCAN_OK) return st;
      ws_bytes = SSCAN_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (lay.total > 0) {
    if (ws == nullptr || ws_bytes < lay.total)
      return fail(SSCAN_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", lay.total, ws_bytes);
    if (misaligned(ws, 16)) return fail(SSCAN_ERR_ALIGN, "workspace must be 16-byte aligned");
  }

  sscan::FwdParams p{};
  p.x = x; p.delta = delta; p.A = A; p.b = b; p.c = c; p.h0 = h0; p.y = y; p.hT = hT; p.H = H;
  p.Dskip = mamba ? Dskip : nullptr;
  p.hck = hck;
  p.nck = (int32_t)ceil_div(r.T, sscan::kCkptSteps);
  p.x_bs = r.x_bs; p.bc_bs = r.bc_bs; p.y_bs = r.y_bs;
  p.B = (int32_t)r.B; p.T = (int32_t)r.T; p.D = (int32_t)r.D;
  p.chunks = chunks;
  p.chunk_len = (int32_t)ceil_div(r.T, chunks);
  if ((hck != nullptr || sg) && chunks > 1) {
    // boundary blocks must not straddle chunks, and the state-group layout's chunks are
    // whole tiles: chunks start on multiples of 64 steps (a multiple of every forward
    // tile and of the block length)
    static_assert(64 % sscan::kSgTile == 0 && 64 % sscan::kCkptSteps == 0, "chunk alignment");
    p.chunk_len = (int32_t)(ceil_div(p.chunk_len, 64) * 64);
    p.chunks = (int32_t)ceil_div(r.T, p.chunk_len);
    chunks = p.chunks;
  }
  const int64_t cpw = sg ? cw : kThreads / lanes;
  const int64_t ntiles_d = ceil_div(r.D, cpw);
  p.ntiles_d = (int32_t)ntiles_d;
  p.xcd_group = sg ? 1 : xcd_group(lanes, r.io_size);
  if (ntiles_d * r.B * chunks > std::numeric_limits<int32_t>::max())
    return fail(SSCAN_ERR_UNSUPPORTED, "too many workgroups");
  hipError_t e;
  char* wsb = static_cast<char*>(ws);
  if (sg) {
    p.bcp = reinterpret_cast<float*>(wsb + lay.bc_off);
    p.tpad = (int32_t)lay.tpad;
    e = sscan::launch_bc_pack(r.io, (int)r.DS, p, stream);
    if (e != hipSuccess) return hip_fail(e, "b/c packing");
  }
  auto pass = [&](bool local, unsigned blocks) {
    return sg ? sscan::launch_fwd_sg(r.io, (int)r.DS, cw, local, mamba, p, blocks, stream)
              : sscan::launch_fwd(r.io, (int)r.DS, lanes, local, mamba, p, blocks, stream);
  };
  if (chunks > 1) {
    p.pairs = reinterpret_cast<float2*>(wsb + lay.pairs_off);
    e = pass(true, (unsigned)(ntiles_d * r.B * (chunks - 1)));
    if (e != hipSuccess) return hip_fail(e, "forward local pass");
  }
  e = pass(false, (unsigned)(ntiles_d * r.B * chunks));
  if (e != hipSuccess) return hip_fail(e, "forward pass");
  return ok();
}

// The backward, plain or wrapped (then gdelta is for delta_raw, gA for A_log, gx includes
// dy * Dskip, and gD, if not null, receives the gradient for Dskip).
// hck (not null, H null): the H-free sweep, recomputing each tile's states from the
// boundary states the forward kept.
int bwd_impl(bool mamba, const sscan_desc* desc, const sscan_plan* plan, const void* dy, const float* dhT,
             const void* x, const void* delta, const float* A, const void* b, const void* c, const float* Dskip,
             const float* h0, const float* H, const float* hck, float* gx, float* gdelta, float* gb, float* gc,
             float* gA, float* gD, float* gh0, void* ws, size_t ws_bytes, hipStream_t stream) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  int lanes, chunks;
  st = resolve_plan(r, plan, mamba ? kPlanMambaBwd : kPlanBwd, &lanes, &chunks);
  if (st != SSCAN_OK) return st;
  const bool hf = hck != nullptr;
  if (hf) {
    if (H != nullptr) return fail(SSCAN_ERR_UNSUPPORTED, "H and boundary states are alternatives");
    st = resolve_hf_plan(r, plan, &lanes, &chunks);
    if (st != SSCAN_OK) return st;
  }
  const bool steps = r.T > 0 && r.B > 0;
  if (r.D > 0 && gA == nullptr) return fail(SSCAN_ERR_NULL, "gA is required");
  if (steps && r.D > 0 &&
      (dy == nullptr || x == nullptr || delta == nullptr || A == nullptr || b == nullptr || c == nullptr ||
       (H == nullptr && !hf) || gx == nullptr || gdelta == nullptr || gb == nullptr || gc == nullptr))
    return fail(SSCAN_ERR_NULL, "dy, x, delta, A, b, c, H (or the boundary states), gx, gdelta, gb and gc are "
                                "required when T > 0");
  if (steps && r.D == 0 && (gb == nullptr || gc == nullptr))
    return fail(SSCAN_ERR_NULL, "gb and gc are required when T > 0");
  const size_t es = r.io_size;
  if (misaligned(dy, es) || misaligned(x, es) || misaligned(delta, es) || misaligned(b, es) || misaligned(c, es))
    return fail(SSCAN_ERR_ALIGN, "io tensors must be aligned to their element size");
  if (misaligned(gx, 4) || misaligned(gdelta, 4) || misaligned(gb, 4) || misaligned(gc, 4) || misaligned(gD, 4) ||
      misaligned(Dskip, 4))
    return fail(SSCAN_ERR_ALIGN, "gradient tensors and Dskip must be 4-byte aligned");
  if (!mamba) gD = nullptr;
  if (misaligned(A, 16) || misaligned(h0, 16) || misaligned(H, 16) || misaligned(dhT, 16) || misaligned(gA, 16) ||
      misaligned(gh0, 16))
    return fail(SSCAN_ERR_ALIGN, "A, h0, H, dhT, gA and gh0 must be 16-byte aligned");
  if (misaligned(hck, 16)) return fail(SSCAN_ERR_ALIGN, "hck must be 16-byte aligned");

  if (!steps || r.D == 0) {
    // No step to sweep: gA = 0, gh0 = dhT (zeros if absent); gb, gc over D = 0 channels are 0.
    hipError_t e = sscan::launch_fill(gA, r.D * r.DS, stream);
    if (e == hipSuccess && gD != nullptr) e = sscan::launch_fill(gD, r.D, stream);  // no step: sum of nothing
    if (e == hipSuccess && gh0 != nullptr) e = sscan::launch_copy_or_zero(gh0, dhT, r.B * r.D * r.DS, stream);
    if (e == hipSuccess && steps && r.D == 0) {
      e = sscan::launch_fill(gb, r.B * r.T * r.DS, stream);
      if (e == hipSuccess) e = sscan::launch_fill(gc, r.B * r.T * r.DS, stream);
    }
    return e == hipSuccess ? ok() : hip_fail(e, "backward without steps");
  }

  const BwdLayout lay = bwd_layout(r, lanes, chunks, mamba);
  if (ws == nullptr || ws_bytes < lay.total)
    return fail(SSCAN_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", lay.total, ws_bytes);
  if (misaligned(ws, 16)) return fail(SSCAN_ERR_ALIGN, "workspace must be 16-byte aligned");

  char* wsb = static_cast<char*>(ws);
  sscan::BwdParams p{};
  p.dy = dy; p.dhT = dhT; p.x = x; p.delta = delta; p.A = A; p.b = b; p.c = c; p.h0 = h0; p.H = H;
  p.gx = gx; p.gdelta = gdelta; p.gh0 = gh0;
  p.part_bc = reinterpret_cast<float2*>(wsb + lay.bc_off);
  p.part_A = reinterpret_cast<float*>(wsb + lay.a_off);
  p.pairs = reinterpret_cast<float2*>(wsb + lay.pairs_off);
  p.Dskip = mamba ? Dskip : nullptr;
  p.part_D = gD != nullptr ? reinterpret_cast<float*>(wsb + lay.d_off) : nullptr;
  p.hck = hck;
  p.nck = (int32_t)ceil_div(r.T, sscan::kCkptSteps);
  p.chunk_len = (int32_t)lay.chunk_len;
  p.chunks = (int32_t)lay.chunks;
  p.subs = (int32_t)lay.subs;
  p.sub_len = (int32_t)lay.sub_len;
  p.x_bs = r.x_bs; p.bc_bs = r.bc_bs; p.y_bs = r.y_bs;
  p.B = (int32_t)r.B; p.T = (int32_t)r.T; p.D = (int32_t)r.D;
  p.ntiles_d = (int32_t)lay.ntiles_d;
  p.xcd_group = xcd_group(lanes, r.io_size);
  if (lay.ntiles_d * r.B * lay.chunks * lay.subs > std::numeric_limits<int32_t>::max())
    return fail(SSCAN_ERR_UNSUPPORTED, "too many workgroups");
  hipError_t e;
  if (lay.chunks > 1) {
    e = sscan::launch_bwd(r.io, (int)r.DS, lanes, true, mamba, p,
                          (unsigned)(lay.ntiles_d * r.B * (lay.chunks - 1) * lay.subs), stream);
    if (e != hipSuccess) return hip_fail(e, "backward local pass");
  }
  const unsigned sweep_grid = (unsigned)(lay.ntiles_d * r.B * lay.chunks);
  e = hf ? sscan::launch_bwd_hf(r.io, (int)r.DS, lanes, mamba, p, sweep_grid, stream)
         : sscan::launch_bwd(r.io, (int)r.DS, lanes, false, mamba, p, sweep_grid, stream);
  if (e != hipSuccess) return hip_fail(e, "backward sweep");
  sscan::ReduceParams q{};
  q.part_bc = p.part_bc; q.part_A = p.part_A; q.gb = gb; q.gc = gc; q.gA = gA;
  q.A_log = mamba ? A : nullptr;
  q.part_D = p.part_D;
  q.gD = gD;
  q.B = p.B; q.T = p.T; q.D = p.D; q.DS = (int32_t)r.DS; q.ntiles_d = p.ntiles_d; q.chunks = p.chunks;
  e = sscan::launch_bwd_reduce(q, stream);
  if (e != hipSuccess) return hip_fail(e, "backward reduce");
  return ok();
}

}  // namespace

extern "C" {

int sscan_version(void) { return SSCAN_VERSION; }

const char* sscan_last_error(void) { return g_last_error; }

const char* sscan_status_str(int status) {
  switch (status) {
    case SSCAN_OK: return "ok";
    case SSCAN_ERR_NULL: return "required pointer is NULL";
    case SSCAN_ERR_SHAPE: return "invalid shape or stride";
    case SSCAN_ERR_DTYPE: return "invalid dtype";
    case SSCAN_ERR_UNSUPPORTED: return "unsupported size or plan";
    case SSCAN_ERR_ALIGN: return "misaligned pointer";
    case SSCAN_ERR_WORKSPACE: return "workspace missing or too small";
    case SSCAN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int sscan_plan_select(const sscan_desc* desc, int backward, sscan_plan* plan) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  if (plan == nullptr) return fail(SSCAN_ERR_NULL, "plan is NULL");
  int lanes, chunks;
  bool sg = false;
  int cw;
  if (backward == SSCAN_PLAN_FWD || backward == SSCAN_PLAN_FWD_H || backward == SSCAN_PLAN_FWD_CKPT)
    st = resolve_fwd_plan(r, nullptr, backward == SSCAN_PLAN_FWD_H, backward == SSCAN_PLAN_FWD_CKPT, &lanes, &chunks,
                          &sg, &cw);
  else
    st = resolve_plan(r, nullptr, backward == SSCAN_PLAN_MAMBA_BWD ? kPlanMambaBwd : kPlanBwd, &lanes, &chunks);
  if (st != SSCAN_OK) return st;
  memset(plan, 0, sizeof(*plan));
  plan->lanes = lanes;
  plan->chunks = chunks;
  plan->layout = sg ? SSCAN_LAYOUT_STATE_GROUPS : SSCAN_LAYOUT_LANES;
  return ok();
}

int sscan_fwd_workspace(const sscan_desc* desc, const sscan_plan* plan, size_t* bytes) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  if (bytes == nullptr) return fail(SSCAN_ERR_NULL, "bytes is NULL");
  int lanes, chunks;
  bool sg;
  int cw;
  // the most that any forward needs: without H, with boundary states (more T-chunks) or
  // without, or writing H (the state-group layout's packed b/c)
  size_t need = 0;
  for (int kind = 0; kind < 3; ++kind) {
    // a plan forcing the state-group layout below DS = 16 has no call writing H to size
    if (kind == 2 && plan != nullptr && plan->layout == SSCAN_LAYOUT_STATE_GROUPS && r.DS != 16) continue;
    st = resolve_fwd_plan(r, plan, kind == 2, kind == 1, &lanes, &chunks, &sg, &cw);
    if (st != SSCAN_OK) return st;
    const size_t t = (r.B == 0 || r.D == 0 || r.T == 0) ? 0 : fwd_layout(r, chunks, sg).total;
    if (t > need) need = t;
  }
  *bytes = need;
  return ok();
}

int sscan_bwd_workspace(const sscan_desc* desc, const sscan_plan* plan, size_t* bytes) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  if (bytes == nullptr) return fail(SSCAN_ERR_NULL, "bytes is NULL");
  int lanes, chunks;
  st = resolve_plan(r, plan, kPlanBwd, &lanes, &chunks);
  if (st != SSCAN_OK) return st;
  *bytes = (r.B == 0 || r.D == 0 || r.T == 0) ? 0 : bwd_layout(r, lanes, chunks, false).total;
  return ok();
}

int sscan_mamba_bwd_workspace(const sscan_desc* desc, const sscan_plan* plan, size_t* bytes) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  if (bytes == nullptr) return fail(SSCAN_ERR_NULL, "bytes is NULL");
  int lanes, chunks;
  st = resolve_plan(r, plan, kPlanMambaBwd, &lanes, &chunks);
  if (st != SSCAN_OK) return st;
  *bytes = (r.B == 0 || r.D == 0 || r.T == 0) ? 0 : bwd_layout(r, lanes, chunks, true).total;
  return ok();
}

int sscan_fwd(const sscan_desc* desc, const sscan_plan* plan, const void* x, const void* delta, const float* A,
              const void* b, const void* c, const float* h0, void* y, float* hT, float* H, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  return fwd_impl(false, desc, plan, x, delta, A, b, c, nullptr, h0, y, hT, H, nullptr, ws, ws_bytes, stream);
}

int sscan_fwd_noalloc(const sscan_desc* desc, const sscan_plan* plan, const void* x, const void* delta,
                      const float* A, const void* b, const void* c, const float* h0, void* y, float* hT, float* H,
                      hipStream_t stream) {
  return fwd_impl(false, desc, plan, x, delta, A, b, c, nullptr, h0, y, hT, H, nullptr, nullptr, 0, stream, true);
}

int sscan_mamba_fwd(const sscan_desc* desc, const sscan_plan* plan, const void* x, const void* delta_raw,
                    const float* A_log, const void* b, const void* c, const float* Dskip, const float* h0, void* y,
                    float* hT, float* H, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(true, desc, plan, x, delta_raw, A_log, b, c, Dskip, h0, y, hT, H, nullptr, ws, ws_bytes, stream);
}

int sscan_bwd(const sscan_desc* desc, const sscan_plan* plan, const void* dy, const float* dhT, const void* x,
              const void* delta, const float* A, const void* b, const void* c, const float* h0, const float* H,
              float* gx, float* gdelta, float* gb, float* gc, float* gA, float* gh0, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  return bwd_impl(false, desc, plan, dy, dhT, x, delta, A, b, c, nullptr, h0, H, nullptr, gx, gdelta, gb, gc, gA,
                  nullptr, gh0, ws, ws_bytes, stream);
}

int sscan_mamba_bwd(const sscan_desc* desc, const sscan_plan* plan, const void* dy, const float* dhT, const void* x,
                    const void* delta_raw, const float* A_log, const void* b, const void* c, const float* Dskip,
                    const float* h0, const float* H, float* gx, float* gdelta_raw, float* gA_log, float* gb,
                    float* gc, float* gDskip, float* gh0, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(true, desc, plan, dy, dhT, x, delta_raw, A_log, b, c, Dskip, h0, H, nullptr, gx, gdelta_raw, gb, gc,
                  gA_log, gDskip, gh0, ws, ws_bytes, stream);
}

int sscan_fwd_ckpt(const sscan_desc* desc, const sscan_plan* plan, int wrapper, const void* x, const void* delta,
                   const float* A, const void* b, const void* c, const float* Dskip, const float* h0, void* y,
                   float* hT, float* hck, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (wrapper != SSCAN_WRAP_NONE && wrapper != SSCAN_WRAP_MAMBA)
    return fail(SSCAN_ERR_UNSUPPORTED, "wrapper %d is unknown", wrapper);
  if (hck == nullptr && desc != nullptr && desc->T > 0 && desc->B > 0 && desc->D > 0)
    return fail(SSCAN_ERR_NULL, "hck is required");
  return fwd_impl(wrapper == SSCAN_WRAP_MAMBA, desc, plan, x, delta, A, b, c, Dskip, h0, y, hT, nullptr, hck, ws,
                  ws_bytes, stream);
}

int sscan_bwd_ckpt(const sscan_desc* desc, const sscan_plan* plan, int wrapper, const void* dy, const float* dhT,
                   const void* x, const void* delta, const float* A, const void* b, const void* c, const float* Dskip,
                   const float* hck, float* gx, float* gdelta, float* gb, float* gc, float* gA, float* gDskip,
                   float* gh0, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (wrapper != SSCAN_WRAP_NONE && wrapper != SSCAN_WRAP_MAMBA)
    return fail(SSCAN_ERR_UNSUPPORTED, "wrapper %d is unknown", wrapper);
  if (hck == nullptr && desc != nullptr && desc->T > 0 && desc->B > 0 && desc->D > 0)
    return fail(SSCAN_ERR_NULL, "hck is required");
  return bwd_impl(wrapper == SSCAN_WRAP_MAMBA, desc, plan, dy, dhT, x, delta, A, b, c, Dskip, nullptr, nullptr, hck,
                  gx, gdelta, gb, gc, gA, gDskip, gh0, ws, ws_bytes, stream);
}

int sscan_bwd_ckpt_workspace(const sscan_desc* desc, const sscan_plan* plan, int wrapper, size_t* bytes) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  if (bytes == nullptr) return fail(SSCAN_ERR_NULL, "bytes is NULL");
  if (wrapper != SSCAN_WRAP_NONE && wrapper != SSCAN_WRAP_MAMBA)
    return fail(SSCAN_ERR_UNSUPPORTED, "wrapper %d is unknown", wrapper);
  int lanes, chunks;
  st = resolve_plan(r, plan, wrapper == SSCAN_WRAP_MAMBA ? kPlanMambaBwd : kPlanBwd, &lanes, &chunks);
  if (st != SSCAN_OK) return st;
  st = resolve_hf_plan(r, plan, &lanes, &chunks);
  if (st != SSCAN_OK) return st;
  *bytes = (r.B == 0 || r.D == 0 || r.T == 0) ? 0 : bwd_layout(r, lanes, chunks, wrapper == SSCAN_WRAP_MAMBA).total;
  return ok();
}

int sscan_decode(const sscan_desc* desc, const void* x, const void* delta, const float* A, const void* b,
                 const void* c, const float* state_in, float* state_out, void* y, hipStream_t stream) {
  Resolved r;
  int st = resolve_desc(desc, &r);
  if (st != SSCAN_OK) return st;
  if (r.T != 1) return fail(SSCAN_ERR_SHAPE, "decode takes one step: desc.T must be 1, got %lld", (long long)r.T);
  if (r.B == 0 || r.D == 0) return ok();
  if (x == nullptr || delta == nullptr || A == nullptr || b == nullptr || c == nullptr || state_in == nullptr ||
      state_out == nullptr || y == nullptr)
    return fail(SSCAN_ERR_NULL, "x, delta, A, b, c, state_in, state_out and y are required");
  const size_t es = r.io_size;
  if (misaligned(x, es) || misaligned(delta, es) || misaligned(b, es) || misaligned(c, es) || misaligned(y, es))
    return fail(SSCAN_ERR_ALIGN, "io tensors must be aligned to their element size");
  if (misaligned(A, 16) || misaligned(state_in, 16) || misaligned(state_out, 16))
    return fail(SSCAN_ERR_ALIGN, "A, state_in and state_out must be 16-byte aligned");
  const int64_t nstate = r.B * r.D * r.DS;
  const char* si = reinterpret_cast<const char*>(state_in);
  const char* so = reinterpret_cast<const char*>(state_out);
  const int64_t sbytes = nstate * 4;
  if (si != so && si < so + sbytes && so < si + sbytes)
    return fail(SSCAN_ERR_SHAPE, "state_out must be state_in itself or not overlap it");
  if ((nstate + kThreads - 1) / kThreads > std::numeric_limits<int32_t>::max())
    return fail(SSCAN_ERR_UNSUPPORTED, "too many workgroups");
  sscan::DecodeParams p{};
  p.x = x; p.delta = delta; p.A = A; p.b = b; p.c = c; p.state_in = state_in; p.state_out = state_out; p.y = y;
  p.x_bs = r.x_bs; p.bc_bs = r.bc_bs; p.y_bs = r.y_bs;
  p.B = (int32_t)r.B; p.D = (int32_t)r.D;
  const hipError_t e = sscan::launch_decode(r.io, (int)r.DS, p, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "decode step");
}

}  // extern "C"
