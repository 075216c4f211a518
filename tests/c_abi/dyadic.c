/*
 * A plain C consumer of libsscan (no Python, no torch): the caller owns every buffer,
 * allocated with hipMalloc, and calls the C ABI of include/sscan.h directly.
 *
 *   dyadic validate   validation only (no GPU call): bad descriptors, a NULL output,
 *                     and the workspace query; runs without a GPU.
 *   dyadic run        forward (y, hT, H) and backward (six gradients) of the worked
 *                     example with A = [-ln 2, -2 ln 2] (every decay a power of 1/2, so
 *                     every value is exact in binary), against its hand-derived values.
 *
 * Exit status 0 when every check passes, 1 on a mismatch, 2 on a HIP error.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "sscan.h"

static int fails = 0;

static void expect_status(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: status %d (%s), expected %d\n", what, got, sscan_status_str(got), want);
    ++fails;
  } else if (want != SSCAN_OK && sscan_last_error()[0] == '\0') {
    printf("FAIL %s: no message from sscan_last_error\n", what);
    ++fails;
  }
}

static void expect_close(const char* name, const float* got, const double* want, int n) {
  double num = 0.0, den = 0.0;
  for (int i = 0; i < n; ++i) {
    if (fabs(got[i] - want[i]) > num) num = fabs(got[i] - want[i]);
    if (fabs(want[i]) > den) den = fabs(want[i]);
  }
  const double rel = den > 0.0 ? num / den : num;
  printf("%-7s max rel err %.2e\n", name, rel);
  if (!(rel < 1e-6)) ++fails;
}

#define HIP_CHECK(call)                                                       \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      return 2;                                                               \
    }                                                                         \
  } while (0)

static int validate(void) {
  sscan_desc d;
  memset(&d, 0, sizeof(d));
  d.B = 1; d.T = 3; d.D = 1; d.DS = 2; d.io = SSCAN_F32;
  size_t n = 0;
  expect_status("workspace query", sscan_fwd_workspace(&d, NULL, &n), SSCAN_OK);
  const float fake_in[4] __attribute__((aligned(16))) = {0};
  float fake_out[4] __attribute__((aligned(16)));
  expect_status("NULL y", sscan_fwd(&d, NULL, fake_in, fake_in, fake_in, fake_in, fake_in, NULL, NULL, NULL, NULL,
                                    NULL, 0, NULL), SSCAN_ERR_NULL);
  d.T = -1;
  expect_status("negative T", sscan_fwd(&d, NULL, fake_in, fake_in, fake_in, fake_in, fake_in, NULL, fake_out, NULL,
                                        NULL, NULL, 0, NULL), SSCAN_ERR_SHAPE);
  d.T = 3; d.DS = 3;
  expect_status("DS = 3", sscan_fwd_workspace(&d, NULL, &n), SSCAN_ERR_UNSUPPORTED);
  d.DS = 2; d.io = 7;
  expect_status("unknown dtype", sscan_fwd_workspace(&d, NULL, &n), SSCAN_ERR_DTYPE);
  printf("library version %d, %s\n", sscan_version(), fails ? "validation FAILED" : "validation ok");
  return fails ? 1 : 0;
}

static int run(void) {
  const double ln2 = log(2.0);
  /* B = 1, T = 3, D = 1, DS = 2 */
  const float x[3] = {2, -1, 4}, delta[3] = {1, 2, 1}, dy[3] = {1, -2, 0.5f};
  const float A[2] = {(float)-ln2, (float)(-2 * ln2)};
  const float b[6] = {1, 2, 0.5f, -1, 3, 0}, c[6] = {1, 1, 2, 0.5f, -1, 2};
  const float h0[2] = {4, -8}, dhT[2] = {1, -1};
  const double y_ref[3] = {6.0, 1.0625, -10.9375}, hT_ref[2] = {12.0, 0.53125};
  const double H_ref[6] = {4, 2, 0, 2.125, 12, 0.53125};
  const double gx_ref[3] = {1.9375, -1.75, 1.5};
  const double gdelta_ref[3] = {3.625 * ln2 + 3.875, 4 * ln2 + 0.875, 6.0};
  const double gb_ref[6] = {0.125, 1.875, 7.5, 2.0, 2.0, 0.0}, gc_ref[6] = {4.0, 2.0, 0.0, -4.25, 6.0, 0.265625};
  const double gA_ref[2] = {-7.375, -2.125}, gh0_ref[2] = {0.03125, 0.234375};

  sscan_desc d;
  memset(&d, 0, sizeof(d));
  d.B = 1; d.T = 3; d.D = 1; d.DS = 2; d.io = SSCAN_F32;

  float *dx, *dd, *dA, *db, *dc, *dh0, *ddy, *ddhT, *y, *hT, *H, *gx, *gdl, *gb, *gc, *gA, *gh0;
  float** bufs[] = {&dx, &dd, &dA, &db, &dc, &dh0, &ddy, &ddhT, &y, &hT, &H, &gx, &gdl, &gb, &gc, &gA, &gh0};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_CHECK(hipMalloc((void**)bufs[i], 64));
  HIP_CHECK(hipMemcpy(dx, x, sizeof(x), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dd, delta, sizeof(delta), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dA, A, sizeof(A), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(db, b, sizeof(b), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dc, c, sizeof(c), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dh0, h0, sizeof(h0), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(ddy, dy, sizeof(dy), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(ddhT, dhT, sizeof(dhT), hipMemcpyHostToDevice));

  size_t nf = 0, nb = 0;
  expect_status("forward workspace", sscan_fwd_workspace(&d, NULL, &nf), SSCAN_OK);
  expect_status("backward workspace", sscan_bwd_workspace(&d, NULL, &nb), SSCAN_OK);
  void* ws = NULL;
  const size_t nws = nf > nb ? nf : nb;
  if (nws > 0) HIP_CHECK(hipMalloc(&ws, nws));
  hipStream_t s;
  HIP_CHECK(hipStreamCreate(&s));
  expect_status("forward", sscan_fwd(&d, NULL, dx, dd, dA, db, dc, dh0, y, hT, H, ws, nf, s), SSCAN_OK);
  expect_status("backward", sscan_bwd(&d, NULL, ddy, ddhT, dx, dd, dA, db, dc, dh0, H, gx, gdl, gb, gc, gA, gh0, ws,
                                      nb, s), SSCAN_OK);
  HIP_CHECK(hipStreamSynchronize(s));

  float out[6];
  HIP_CHECK(hipMemcpy(out, y, 3 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("y", out, y_ref, 3);
  HIP_CHECK(hipMemcpy(out, hT, 2 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("hT", out, hT_ref, 2);
  HIP_CHECK(hipMemcpy(out, H, 6 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("H", out, H_ref, 6);
  HIP_CHECK(hipMemcpy(out, gx, 3 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("gx", out, gx_ref, 3);
  HIP_CHECK(hipMemcpy(out, gdl, 3 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("gdelta", out, gdelta_ref, 3);
  HIP_CHECK(hipMemcpy(out, gb, 6 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("gb", out, gb_ref, 6);
  HIP_CHECK(hipMemcpy(out, gc, 6 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("gc", out, gc_ref, 6);
  HIP_CHECK(hipMemcpy(out, gA, 2 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("gA", out, gA_ref, 2);
  HIP_CHECK(hipMemcpy(out, gh0, 2 * sizeof(float), hipMemcpyDeviceToHost)); expect_close("gh0", out, gh0_ref, 2);

  HIP_CHECK(hipStreamDestroy(s));
  if (ws != NULL) HIP_CHECK(hipFree(ws));
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_CHECK(hipFree(*bufs[i]));
  printf("%s\n", fails ? "worked example FAILED" : "worked example ok");
  return fails ? 1 : 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "validate") == 0) return validate();
  if (argc == 2 && strcmp(argv[1], "run") == 0) return run();
  printf("usage: %s validate|run\n", argv[0]);
  return 2;
}
