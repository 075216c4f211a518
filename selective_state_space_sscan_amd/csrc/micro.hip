// Microbenchmarks for the ceilings the scan kernels are measured against: the v_exp_f32
// and fp32 FMA issue rates, the rate of a register-only loop with the forward's per-state
// mix (one exp2, two multiplies, two FMAs), and the HBM read and write stream rates.
// Built into its own library (libsscan_micro.so); nothing in libsscan uses it.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 16;  // independent dependency chains per thread

__global__ __launch_bounds__(kThreads) void exp_rate_kernel(float* out, int iters) {
  float v[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) v[i] = 0.5f + 0.01f * i + threadIdx.x * 1e-7f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) v[i] = __builtin_amdgcn_exp2f(-v[i]);  // the negation is a source modifier
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += v[i];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void fma_rate_kernel(float* out, int iters, float k) {
  float v[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) v[i] = 0.5f + 0.01f * i + threadIdx.x * 1e-7f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) v[i] = fmaf(v[i], k, 0.25f);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += v[i];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// The forward's per-(step, state) work with every operand in registers: a = exp2(delta *
// A log2 e), h = a h + (delta x) b, y += h c; K states per thread.
template <int K>
__global__ __launch_bounds__(kThreads) void mix_kernel(float* out, int steps, float s) {
  float A2[K], b[K], c[K], h[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    A2[i] = -0.1f * (i + 1) - threadIdx.x * 1e-6f;
    b[i] = 0.3f + i * 0.01f;
    c[i] = 0.2f - i * 0.01f;
    h[i] = 0.f;
  }
  float d = s, w = s * 0.5f, y = 0.f;
  for (int t = 0; t < steps; ++t) {
    float yp = 0.f;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const float a = __builtin_amdgcn_exp2f(d * A2[i]);
      h[i] = fmaf(a, h[i], w * b[i]);
      yp = fmaf(h[i], c[i], yp);
    }
    y += yp;
    d += 1e-6f;
    w -= 1e-6f;
  }
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = y;
}

__global__ __launch_bounds__(kThreads) void write_stream_kernel(float4* dst, int64_t n, float v) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    dst[i] = make_float4(v, v + 1.f, v + 2.f, v + 3.f);
}

// The same with non-temporal stores (the policy the forward writes H with).
typedef float f4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kThreads) void write_stream_nt_kernel(f4_t* dst, int64_t n, float v) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const f4_t q = {v, v + 1.f, v + 2.f, v + 3.f};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(q, dst + i);
}

// The store pattern of the forward writing H at B x T x D x DS = 8 x 2048 x 768 x 16 with
// nothing else: a workgroup per (batch row, 32 channels), 8 lanes per channel holding two
// states, each lane storing its 8 bytes of every step with the non-temporal policy.
constexpr int kHB = 8, kHT = 2048, kHD = 768, kHDS = 16;
typedef float f2_t __attribute__((ext_vector_type(2)));
__global__ __launch_bounds__(kThreads) void h_pattern_kernel(float* H, float v) {
  const int b = blockIdx.x / (kHD / 32);
  const int d = (blockIdx.x % (kHD / 32)) * 32 + threadIdx.x / 8;
  const int j = threadIdx.x % 8;
  const f2_t q = {v, v + 1.f};
  for (int t = 0; t < kHT; ++t) {
    const int64_t off = ((int64_t)(b * kHT + t) * kHD + d) * kHDS + j * 2;
    __builtin_nontemporal_store(q, reinterpret_cast<f2_t*>(H + off));
  }
}

// The whole memory traffic of the forward writing H at 8x2048x768x16 fp32, without its
// arithmetic: the same workgroups (a batch row and 32 channels each), x and delta loaded
// cooperatively one 64-step tile ahead, y written for the tile's elements, and H stored by 8
// lanes per channel, 8 bytes per lane and step, non-temporal.  The stored values depend on
// the tile's loads, so the loads complete before the tile's stores, as in the forward.
__global__ __launch_bounds__(kThreads) void fwd_pattern_kernel(const float* x, const float* dl, float* y, float* H) {
  constexpr int TB = 64, PER = TB * 32 / kThreads;
  const int b = blockIdx.x / (kHD / 32);
  const int d0 = (blockIdx.x % (kHD / 32)) * 32;
  const int d = d0 + threadIdx.x / 8;
  const int j = threadIdx.x % 8;
  float rx[PER], rd[PER];
  auto load = [&](int ts) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = threadIdx.x + k * kThreads;
      const int64_t off = ((int64_t)b * kHT + ts + e / 32) * kHD + d0 + e % 32;
      rx[k] = x[off];
      rd[k] = dl[off];
    }
  };
  load(0);
  for (int ts = 0; ts < kHT; ts += TB) {
    float cx[PER], cd[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) { cx[k] = rx[k]; cd[k] = rd[k]; }
    if (ts + TB < kHT) load(ts + TB);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) sum = fmaf(cx[k], cd[k], sum);
    for (int t = ts; t < ts + TB; ++t) {
      const f2_t q = {sum, sum + (float)t};
      const int64_t off = ((int64_t)(b * kHT + t) * kHD + d) * kHDS + j * 2;
      __builtin_nontemporal_store(q, reinterpret_cast<f2_t*>(H + off));
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = threadIdx.x + k * kThreads;
      y[((int64_t)b * kHT + ts + e / 32) * kHD + d0 + e % 32] = cx[k] + cd[k];
    }
  }
}

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const float4* src, int64_t n, float* out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float s = 0.f;
  for (int64_t i = gid; i < n; i += stride) {
    const float4 q = src[i];
    s += (q.x + q.y) + (q.z + q.w);
  }
  out[gid] = s;
}

struct Timer {
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool ok = false;
  Timer() {
    ok = hipStreamCreate(&s) == hipSuccess && hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess;
  }
  ~Timer() {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (s) (void)hipStreamDestroy(s);
  }
};

// Runs `launch` once untimed, then `reps` times between two events; mean ms per launch.
template <typename F>
int time_launches(Timer& t, int reps, F launch, double* ms) {
  launch(t.s);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(t.s) != hipSuccess) return 1;
  if (hipEventRecord(t.e0, t.s) != hipSuccess) return 1;
  for (int r = 0; r < reps; ++r) launch(t.s);
  if (hipGetLastError() != hipSuccess || hipEventRecord(t.e1, t.s) != hipSuccess) return 1;
  if (hipEventSynchronize(t.e1) != hipSuccess) return 1;
  float f = 0.f;
  if (hipEventElapsedTime(&f, t.e0, t.e1) != hipSuccess) return 1;
  *ms = (double)f / reps;
  return 0;
}

}  // namespace

extern "C" {

// which: 0 = v_exp_f32 results/s, 1 = fp32 FMA results/s, 2/3/4 = forward-mix states/s with
// 1/2/4 states per thread, 5 = write stream bytes/s, 6 = read stream bytes/s, 7 = write
// stream with non-temporal stores, bytes/s, 8 = the forward's H store pattern at
// 8x2048x768x16 alone, bytes/s, 9 = the whole memory traffic of the forward writing H at
// that size (x, delta read; y, H written) without its arithmetic, bytes/s, 10 = the same
// with x, delta and y taken from three copies in turn, so that no launch finds its inputs
// in the last-level cache (for 8-10 bytes and waves_per_simd are ignored).
// waves_per_simd: 1..8, the grid size of the compute kernels (256 CUs x 4 SIMDs each);
// bytes: buffer size of the stream kernels (a multiple of 16, at most 16 GiB).
// Allocates its own device buffers and stream.  Returns 0 and the rate in *rate, else 1.
int sscan_micro_rate(int which, int waves_per_simd, int64_t bytes, double* rate) {
  if (rate == nullptr || which < 0 || which > 10 || waves_per_simd < 1 || waves_per_simd > 8) return 1;
  if (which >= 5 && which <= 7 && (bytes <= 0 || bytes % 16 != 0 || bytes > (int64_t(16) << 30))) return 1;
  Timer t;
  if (!t.ok) return 1;
  const int blocks = 256 * 4 * waves_per_simd * 64 / kThreads;  // waves_per_simd waves on each SIMD
  const int64_t nthreads = (int64_t)blocks * kThreads;
  int rc = 1;
  double ms = 0.0;
  if (which <= 4) {
    float* out = nullptr;
    if (hipMalloc(&out, nthreads * sizeof(float)) != hipSuccess) return 1;
    if (which == 0) {
      const int iters = 4096;
      rc = time_launches(t, 5, [&](hipStream_t s) {
        hipLaunchKernelGGL(exp_rate_kernel, dim3(blocks), dim3(kThreads), 0, s, out, iters);
      }, &ms);
      if (rc == 0) *rate = (double)nthreads * iters * kChains / (ms * 1e-3);
    } else if (which == 1) {
      const int iters = 16384;
      rc = time_launches(t, 5, [&](hipStream_t s) {
        hipLaunchKernelGGL(fma_rate_kernel, dim3(blocks), dim3(kThreads), 0, s, out, iters, 0.999f);
      }, &ms);
      if (rc == 0) *rate = (double)nthreads * iters * kChains / (ms * 1e-3);
    } else {
      const int steps = 4096;
      const int K = which == 2 ? 1 : which == 3 ? 2 : 4;
      rc = time_launches(t, 5, [&](hipStream_t s) {
        if (K == 1) hipLaunchKernelGGL(mix_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, out, steps, 0.5f);
        else if (K == 2) hipLaunchKernelGGL(mix_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, out, steps, 0.5f);
        else hipLaunchKernelGGL(mix_kernel<4>, dim3(blocks), dim3(kThreads), 0, s, out, steps, 0.5f);
      }, &ms);
      if (rc == 0) *rate = (double)nthreads * steps * K / (ms * 1e-3);
    }
    (void)hipFree(out);
    return rc;
  }
  if (which == 8) {
    const int64_t hbytes = (int64_t)kHB * kHT * kHD * kHDS * 4;
    float* H = nullptr;
    if (hipMalloc(&H, hbytes) != hipSuccess) return 1;
    rc = time_launches(t, 5, [&](hipStream_t s) {
      hipLaunchKernelGGL(h_pattern_kernel, dim3(kHB * (kHD / 32)), dim3(kThreads), 0, s, H, 1.f);
    }, &ms);
    if (rc == 0) *rate = (double)hbytes / (ms * 1e-3);
    (void)hipFree(H);
    return rc;
  }
  if (which == 9 || which == 10) {
    const int64_t n = (int64_t)kHB * kHT * kHD;
    const int64_t hbytes = n * kHDS * 4;
    const int copies = which == 10 ? 3 : 1;
    float *H = nullptr, *io = nullptr;
    if (hipMalloc(&H, hbytes) != hipSuccess) return 1;
    if (hipMalloc(&io, copies * 3 * n * sizeof(float)) != hipSuccess) {
      (void)hipFree(H);
      return 1;
    }
    (void)hipMemsetAsync(io, 0, copies * 3 * n * sizeof(float), t.s);
    int k = 0;
    rc = time_launches(t, 6, [&](hipStream_t s) {
      float* c = io + (int64_t)(k++ % copies) * 3 * n;
      hipLaunchKernelGGL(fwd_pattern_kernel, dim3(kHB * (kHD / 32)), dim3(kThreads), 0, s, c, c + n, c + 2 * n, H);
    }, &ms);
    if (rc == 0) *rate = (double)(hbytes + 3 * n * sizeof(float)) / (ms * 1e-3);
    (void)hipFree(io);
    (void)hipFree(H);
    return rc;
  }
  const int64_t n = bytes / 16;
  const int sblocks = 256 * 16;  // 16 workgroups of 256 threads per CU, grid-stride
  float4* buf = nullptr;
  float* out = nullptr;
  if (hipMalloc(&buf, bytes) != hipSuccess) return 1;
  if (hipMalloc(&out, (size_t)sblocks * kThreads * sizeof(float)) != hipSuccess) {
    (void)hipFree(buf);
    return 1;
  }
  if (which == 5) {
    rc = time_launches(t, 10, [&](hipStream_t s) {
      hipLaunchKernelGGL(write_stream_kernel, dim3(sblocks), dim3(kThreads), 0, s, buf, n, 1.f);
    }, &ms);
  } else if (which == 7) {
    f4_t* vbuf = reinterpret_cast<f4_t*>(buf);
    rc = time_launches(t, 10, [&](hipStream_t s) {
      hipLaunchKernelGGL(write_stream_nt_kernel, dim3(sblocks), dim3(kThreads), 0, s, vbuf, n, 1.f);
    }, &ms);
  } else {
    hipLaunchKernelGGL(write_stream_kernel, dim3(sblocks), dim3(kThreads), 0, t.s, buf, n, 1.f);
    rc = time_launches(t, 10, [&](hipStream_t s) {
      hipLaunchKernelGGL(read_stream_kernel, dim3(sblocks), dim3(kThreads), 0, s, buf, n, out);
    }, &ms);
  }
  if (rc == 0) *rate = (double)bytes / (ms * 1e-3);
  (void)hipFree(out);
  (void)hipFree(buf);
  return rc;
}

}  // extern "C"
