/*
 * sscan.h -- C ABI of libsscan, the selective diagonal state-space scan for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "pssa-100m/pssa_kernels.py", module docstring), for each
 * batch row b, channel d, state n and step t = 0..T-1:
 *
 *     h[b,t,d,n] = exp(delta[b,t,d] * A[d,n]) * h[b,t-1,d,n] + delta[b,t,d] * b[b,t,n] * x[b,t,d]
 *     y[b,t,d]   = sum_n h[b,t,d,n] * c[b,t,n]
 *
 * with h[b,-1,d,n] = h0[b,d,n] and hT[b,d,n] = h[b,T-1,d,n].  The per-token
 * states H = h (B,T,D,DS) may be materialised so that the backward is a single
 * reverse sweep (same page, the ScanFn forward); hT of one call is the h0 of
 * the next when a sequence is split into consecutive calls (same page, module
 * docstring: h0 carried across chunks).  The backward (same page, scan_bwd)
 * returns the gradients of L = sum(dy*y) + sum(dhT*hT) with respect to x,
 * delta, b, c, A and h0.  The page's backward has no dhT term; passing
 * dhT = NULL reproduces it.
 *
 * Conventions shared by every entry point:
 *  - Layouts are row-major with the last dimension contiguous:
 *      x, delta, dy   : (B,T,D)    element (b,t,d) at b*x_bstride + t*D + d
 *      y, gx, gdelta  : (B,T,D)    element (b,t,d) at b*y_bstride + t*D + d
 *      b, c           : (B,T,DS)   element (b,t,n) at b*bc_bstride + t*DS + n
 *      gb, gc         : (B,T,DS)   contiguous
 *      A, gA          : (D,DS)     contiguous
 *      h0, hT, dhT, gh0 : (B,D,DS) contiguous
 *      H              : (B,T,D,DS) contiguous
 *    Only the batch strides are free, so a T-slice of a longer sequence is a
 *    valid argument (input or output) without a copy.
 *  - Sizes: B <= 65535, T < 2^31 and D*DS <= 2^22 (the kernels address a tile
 *    with 32-bit offsets); larger ones give SSCAN_ERR_UNSUPPORTED.
 *  - dtypes: x, delta, b, c, y and dy have the descriptor's io dtype (fp32 or
 *    bf16).  A, h0, hT, H, dhT and every gradient are fp32.  Arithmetic and
 *    the state are fp32; y is rounded to bf16 with round-to-nearest-even.
 *  - Memory: every pointer is device memory owned by the caller.  The library
 *    allocates nothing; scratch space is the caller's workspace, sized by the
 *    *_workspace query (sscan_fwd_noalloc instead uses a static array of the
 *    library).  Inputs are never written.  Outputs are overwritten,
 *    never accumulated into, and must not alias any input or each other.
 *  - A, h0, hT, H, dhT, gA and gh0 must be 16-byte aligned; every other tensor
 *    must be aligned to its element size (4 bytes for fp32, 2 for bf16); the
 *    workspace to 16 bytes.
 *  - Asynchrony: work is enqueued on `stream` (NULL = the default stream) and
 *    the call returns without waiting.  Calls are thread-safe as long as
 *    concurrent calls use distinct workspaces and outputs.
 *  - Errors: every argument is validated before anything is enqueued.  A
 *    non-zero status other than SSCAN_ERR_HIP means nothing was enqueued and
 *    nothing was written.  SSCAN_ERR_HIP means the HIP runtime refused a
 *    launch; outputs are then undefined.  sscan_last_error() gives a message
 *    for the last failure on the calling thread.
 */
#ifndef SSCAN_H_
#define SSCAN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSCAN_VERSION 1

/* Bytes of device scratch that sscan_fwd_noalloc has on each GPU (32 MiB). */
#define SSCAN_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Steps between the boundary states kept by the H-free path (sscan_fwd_ckpt). */
#define SSCAN_CKPT_STEPS 32

/* Which inputs the checkpointed entry points take: the plain scan's (delta, A), or the
 * Mamba-style wrapper's (delta_raw, A_log, Dskip) as in sscan_mamba_fwd. */
typedef enum sscan_wrapper { SSCAN_WRAP_NONE = 0, SSCAN_WRAP_MAMBA = 1 } sscan_wrapper;

/* Element type of x, delta, b, c, y, dy. */
typedef enum sscan_dtype { SSCAN_F32 = 0, SSCAN_BF16 = 1 } sscan_dtype;

typedef enum sscan_status {
  SSCAN_OK = 0,
  SSCAN_ERR_NULL = 1,        /* a required pointer is NULL */
  SSCAN_ERR_SHAPE = 2,       /* a negative size, or a batch stride shorter than one batch row */
  SSCAN_ERR_DTYPE = 3,       /* io is not an sscan_dtype */
  SSCAN_ERR_UNSUPPORTED = 4, /* DS not in {1,2,4,8,16}, a bad plan, or a size beyond 32-bit grid limits */
  SSCAN_ERR_ALIGN = 5,       /* a pointer is not aligned to its element size */
  SSCAN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the size the query returned */
  SSCAN_ERR_HIP = 7          /* the HIP runtime reported an error */
} sscan_status;

/* Problem sizes and layout. */
typedef struct sscan_desc {
  int64_t B;          /* batch rows, >= 0 */
  int64_t T;          /* steps in this call, >= 0 */
  int64_t D;          /* channels, >= 0 */
  int64_t DS;         /* states per channel: 1, 2, 4, 8 or 16 */
  int32_t io;         /* sscan_dtype of x, delta, b, c, y, dy */
  int32_t reserved;   /* must be 0 */
  int64_t x_bstride;  /* elements between batch rows of x, delta, dy; 0 means T*D */
  int64_t bc_bstride; /* elements between batch rows of b, c; 0 means T*DS */
  int64_t y_bstride;  /* elements between batch rows of y, gx, gdelta; 0 means T*D */
} sscan_desc;

/* Forward layouts.  LANES: a 64-lane wave holds 64/lanes channels, the states of a channel
 * split over `lanes` consecutive lanes (the only layout of the backward).  STATE_GROUPS: a
 * workgroup holds 64 (or 32) channels, one per lane, and the states of a channel in pairs
 * across its waves (DS in {4, 8, 16}, D a multiple of 4, T < 2^24; writing H, DS = 16 and
 * 32 channels; its plan.lanes, the threads per channel, is DS/2).  Both layouts form every
 * state with the same operations, so hT, H and the boundary states agree bit for bit.
 * AUTO: the forwards without H (keeping boundary states or not) take state groups wherever
 * they apply, split into T-chunks (of at least 256 steps) when one pass has under 512
 * compute waves; the forward writing H takes them at DS = 16 for a single pass with enough
 * workgroups; the lanes layout otherwise, where the forward without H or boundary states
 * splits below one wave per SIMD into T-chunks of whole tiles for up to four waves per SIMD
 * (sscan_plan_select reports the choice). */
typedef enum sscan_layout { SSCAN_LAYOUT_AUTO = 0, SSCAN_LAYOUT_LANES = 1, SSCAN_LAYOUT_STATE_GROUPS = 2 } sscan_layout;

/* Launch plan.  Pass NULL wherever a plan is accepted to let the library choose. */
typedef struct sscan_plan {
  int32_t lanes;       /* lanes sharing one channel's DS states: 1,2,4,8,16 and <= DS; 0 = choose */
  int32_t chunks;      /* T-chunks of the in-kernel two-level scan (forward) or sweep (backward); 1 = single pass, 0 = choose */
  int32_t layout;      /* sscan_layout of the forward; AUTO = choose.  Entry points of the backward take AUTO or LANES */
  int32_t reserved[5]; /* must be 0 */
} sscan_plan;

/* Forward.
 *   x, delta (B,T,D) io; A (D,DS) fp32; b, c (B,T,DS) io; h0 (B,D,DS) fp32 or NULL (zeros).
 *   y (B,T,D) io, required.  hT (B,D,DS) fp32 or NULL (not written).
 *   H (B,T,D,DS) fp32 or NULL (not written); H[b,t] is the state after step t.
 *   T == 0: y is empty and hT = h0 (zeros if h0 is NULL).  B == 0 or D == 0: nothing to do.
 *   ws/ws_bytes: workspace of at least the size sscan_fwd_workspace reports (may be NULL if that is 0). */
int sscan_fwd(const sscan_desc* desc, const sscan_plan* plan, const void* x, const void* delta,
              const float* A, const void* b, const void* c, const float* h0, void* y, float* hT, float* H,
              void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace sscan_fwd needs for (desc, plan) -> *bytes. */
int sscan_fwd_workspace(const sscan_desc* desc, const sscan_plan* plan, size_t* bytes);

/* sscan_fwd for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments, results and
 * errors as sscan_fwd, without the workspace: the scratch the forward needs (the two-level
 * scan's carry pairs, the packed b/c of the state-group layout) lives in a static device
 * array of SSCAN_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from its load
 * until the process ends.  This call allocates nothing (no hipMalloc, no torch).
 *   Where the state-group layout's packed b/c would not fit (B*T > 262144 at DS = 16) and
 *   the plan leaves the layout to the library, the call runs the lanes layout instead.  A
 *   call whose forward still needs more scratch than the array holds (at most what
 *   sscan_fwd_workspace reports for the same desc and plan) returns SSCAN_ERR_WORKSPACE
 *   before any GPU call.
 *   Every call on one GPU shares its array: calls that overlap in time on one GPU (two
 *   streams, or two threads) race and give undefined results; calls in one stream order are
 *   safe.  Nothing in the array needs to start at zero: every call writes the scratch it
 *   reads.  The GPU is the device of `stream` (the current device for NULL). */
int sscan_fwd_noalloc(const sscan_desc* desc, const sscan_plan* plan, const void* x, const void* delta,
                      const float* A, const void* b, const void* c, const float* h0, void* y, float* hT, float* H,
                      hipStream_t stream);

/* Backward: gradients of L = sum(dy*y) + sum(dhT*hT) for the forward with the same inputs.
 *   dy (B,T,D) io; dhT (B,D,DS) fp32 or NULL (zeros); x, delta, A, b, c, h0 as in sscan_fwd;
 *   H (B,T,D,DS) fp32, the states the forward materialised, required when T > 0.  With four
 *   states per lane (the default plan for DS >= 4) the backward reads only rows 3, 7, 11, ...
 *   and the last of H, and forms the three rows after each of them with the forward's own
 *   update on the same inputs: bit for bit the stored rows when the forward ran as one pass,
 *   within fp32 rounding of them where the forward split T into chunks (sscan_plan_select
 *   with SSCAN_PLAN_FWD_H reports its chunks).  Other plans read every row.
 *   gx, gdelta (B,T,D) fp32; gb, gc (B,T,DS) fp32, summed over channels;
 *   gA (D,DS) fp32, summed over batch rows and steps; gh0 (B,D,DS) fp32 or NULL (not written).
 *   T == 0: gA = 0 and gh0 = dhT (zeros if NULL).  B == 0: gA = 0.
 *   Gradient sums are formed in a fixed order, so results are bitwise reproducible run to run. */
int sscan_bwd(const sscan_desc* desc, const sscan_plan* plan, const void* dy, const float* dhT, const void* x,
              const void* delta, const float* A, const void* b, const void* c, const float* h0, const float* H,
              float* gx, float* gdelta, float* gb, float* gc, float* gA, float* gh0, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* Bytes of workspace sscan_bwd needs for (desc, plan) -> *bytes. */
int sscan_bwd_workspace(const sscan_desc* desc, const sscan_plan* plan, size_t* bytes);

/* Mamba-style wrapper around the scan (POPCORNBENCH page: the module's forward, steps
 * 1, 4 and 9, and its numerically stable softplus that returns its argument above 20):
 *     delta = softplus(delta_raw)    softplus(r) = r if r > 20 else log(1 + e^r)
 *     A     = -exp(A_log)
 *     y     = scan(x, delta, A, b, c, h0) + Dskip * x
 * The prologue is applied as the inputs are staged and the skip term before y is
 * rounded, inside the scan kernels: nothing extra is read or written.
 *   Arguments, layouts, workspace (sscan_fwd_workspace) and errors as in sscan_fwd, with
 *   delta_raw (B,T,D) io in place of delta, A_log (D,DS) fp32 in place of A, and
 *   Dskip (D,) fp32, 4-byte aligned, or NULL (no skip term).  H holds the states of the
 *   scan (what sscan_mamba_bwd takes). */
int sscan_mamba_fwd(const sscan_desc* desc, const sscan_plan* plan, const void* x, const void* delta_raw,
                    const float* A_log, const void* b, const void* c, const float* Dskip, const float* h0, void* y,
                    float* hT, float* H, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of sscan_mamba_fwd: gradients of L = sum(dy*y) + sum(dhT*hT) by the chain rule
 * through the three maps (d delta/d delta_raw = 1 above 20, else e^r/(1+e^r); dA/dA_log = A;
 * the skip term adds dy * Dskip to gx).
 *   Arguments as in sscan_bwd, with delta_raw, A_log and Dskip as in sscan_mamba_fwd, and
 *   gdelta_raw (B,T,D), gA_log (D,DS) fp32 in place of gdelta, gA.  gDskip (D,) fp32 or
 *   NULL (not written) receives sum over b, t of dy * x -- the gradient for Dskip, also
 *   when Dskip is NULL (that is, at Dskip = 0).  T == 0: gA_log = 0, gDskip = 0, gh0 = dhT.
 *   ws/ws_bytes: at least what sscan_mamba_bwd_workspace reports. */
int sscan_mamba_bwd(const sscan_desc* desc, const sscan_plan* plan, const void* dy, const float* dhT, const void* x,
                    const void* delta_raw, const float* A_log, const void* b, const void* c, const float* Dskip,
                    const float* h0, const float* H, float* gx, float* gdelta_raw, float* gA_log, float* gb,
                    float* gc, float* gDskip, float* gh0, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace sscan_mamba_bwd needs for (desc, plan) -> *bytes. */
int sscan_mamba_bwd_workspace(const sscan_desc* desc, const sscan_plan* plan, size_t* bytes);

/* H-free path, forward: the forward of sscan_fwd (wrapper SSCAN_WRAP_NONE) or of
 * sscan_mamba_fwd (SSCAN_WRAP_MAMBA; then delta is delta_raw, A is A_log and Dskip is used)
 * that keeps, instead of every state H, only the state entering each block of
 * SSCAN_CKPT_STEPS steps, as the "ruDNN KDA chunk.rs" page keeps chunk boundary states
 * (retain_boundaries) rather than a state history:
 *     hck[b, k, d, n] = h[b, k*SSCAN_CKPT_STEPS - 1, d, n]   (h0, or zeros, for k = 0)
 *   hck (B, ceil(T/SSCAN_CKPT_STEPS), D, DS) fp32, 16-byte aligned, required when there are
 *   steps; 1/SSCAN_CKPT_STEPS of the memory and HBM writes of H.  Everything else as in
 *   sscan_fwd / sscan_mamba_fwd, including the workspace query (sscan_fwd_workspace).
 *   SSCAN_ERR_UNSUPPORTED for an unknown wrapper. */
int sscan_fwd_ckpt(const sscan_desc* desc, const sscan_plan* plan, int wrapper, const void* x, const void* delta,
                   const float* A, const void* b, const void* c, const float* Dskip, const float* h0, void* y,
                   float* hT, float* hck, void* ws, size_t ws_bytes, hipStream_t stream);

/* H-free path, backward: the gradients of sscan_bwd / sscan_mamba_bwd from the boundary
 * states of sscan_fwd_ckpt instead of H.  Each SSCAN_CKPT_STEPS-step tile of the reverse
 * sweep first recomputes its states from the boundary state at its start with the
 * forward's own arithmetic (so they equal the forward's states bit for bit), then sweeps.
 *   No h0 argument: hck[:, 0] is h0.  gDskip is used with SSCAN_WRAP_MAMBA only (NULL or
 *   the gradient for Dskip, as in sscan_mamba_bwd).  Runs 8 or 16 lanes per channel, so it
 *   needs DS >= 8 (SSCAN_ERR_UNSUPPORTED otherwise, or for plan.lanes < 8).
 *   ws/ws_bytes: at least what sscan_bwd_ckpt_workspace reports for the same wrapper. */
int sscan_bwd_ckpt(const sscan_desc* desc, const sscan_plan* plan, int wrapper, const void* dy, const float* dhT,
                   const void* x, const void* delta, const float* A, const void* b, const void* c, const float* Dskip,
                   const float* hck, float* gx, float* gdelta, float* gb, float* gc, float* gA, float* gDskip,
                   float* gh0, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace sscan_bwd_ckpt needs for (desc, plan, wrapper) -> *bytes. */
int sscan_bwd_ckpt_workspace(const sscan_desc* desc, const sscan_plan* plan, int wrapper, size_t* bytes);

/* One decode step (T = 1) on a state kept in device memory between calls: the recurrence
 * of the forward applied to a single token ("ruDNN KDA chunk.rs" page, chunk_kda: one
 * token goes through a fused recurrent kernel on the resident state, and inputs are
 * never mutated).  For each b, d, n:
 *     state_out[b,d,n] = exp(delta[b,d] A[d,n]) state_in[b,d,n] + delta[b,d] b[b,n] x[b,d]
 *     y[b,d]           = sum_n state_out[b,d,n] c[b,n]
 *   desc->T must be 1 (SSCAN_ERR_SHAPE otherwise); layouts, strides and dtypes are the
 *   forward's with T = 1: x, delta, y (B,1,D) io; b, c (B,1,DS) io; A (D,DS) fp32.
 *   state_in, state_out (B,D,DS) fp32, 16-byte aligned.  state_out may be state_in itself
 *   (the update is then in place); any other overlap is SSCAN_ERR_SHAPE.
 *   Same result as sscan_fwd with T = 1, h0 = state_in, hT = state_out, up to the order of
 *   the sum over states.  B == 0 or D == 0: nothing to do.  Needs no workspace. */
int sscan_decode(const sscan_desc* desc, const void* x, const void* delta, const float* A, const void* b,
                 const void* c, const float* state_in, float* state_out, void* y, hipStream_t stream);

/* Entry points whose plan sscan_plan_select reports (its `backward` argument). */
typedef enum sscan_plan_kind {
  SSCAN_PLAN_FWD = 0,       /* sscan_fwd / sscan_mamba_fwd without H */
  SSCAN_PLAN_BWD = 1,       /* sscan_bwd */
  SSCAN_PLAN_MAMBA_BWD = 2, /* sscan_mamba_bwd */
  SSCAN_PLAN_FWD_H = 3,     /* sscan_fwd / sscan_mamba_fwd writing H */
  SSCAN_PLAN_FWD_CKPT = 4   /* sscan_fwd_ckpt (the forward keeping boundary states) */
} sscan_plan_kind;

/* The plan the library picks for desc -> *plan when the caller passes none, for the entry
 * point named by `backward` (an sscan_plan_kind; any other value means sscan_bwd).  The
 * forward's plan depends on what it stores: only the forward without H or boundary states
 * runs the state-group layout, and the forward keeping boundary states splits T from below
 * one wave per SIMD.  Uses no GPU. */
int sscan_plan_select(const sscan_desc* desc, int backward, sscan_plan* plan);

/* Static text for a status code. */
const char* sscan_status_str(int status);

/* Message describing the last failure on the calling thread ("" if none). */
const char* sscan_last_error(void);

/* SSCAN_VERSION of the built library. */
int sscan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSCAN_H_ */
