/*
 * sscan_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference for the selective diagonal state-space
 * scan.  Only the test suite, the package smoke check and the CPU-baseline leg
 * of the benchmark load it.  The GPU library neither links nor calls it, and
 * this file shares no code, header or constant with the GPU library.
 *
 * What it computes (page "pssa-100m/pssa_kernels.py", module docstring): for
 * every batch row b, channel d and state n,
 *
 *     h[t][n] = exp(delta[t] * A[d][n]) * h[t-1][n] + delta[t] * b[t][n] * x[t]
 *     y[t]    = sum_n h[t][n] * c[t][n]
 *
 * with h[-1] = h0 (zero when h0 is absent) and hT = h[T-1].  The forward loop
 * has the shape of that page's scan_fwd; the backward is the reverse adjoint
 * sweep of that page's scan_bwd (including the gradient of an optional
 * upstream dhT, which seeds the sweep), evaluated with a locally recomputed
 * state history, never with one produced elsewhere.
 *
 * Every input and output is double.  Callers convert fp32 / bf16 inputs to
 * double, which is exact.  Work is split into items of (batch row, block of
 * ORACLE_DBLK channels); each item writes its own outputs or its own partial
 * sums, and partial sums are combined in a fixed order afterwards, so the
 * result does not depend on the number of threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_DBLK 16

typedef struct {
  int64_t B, T, D, DS;
  const double *x, *delta, *A, *b, *c, *h0; /* h0 may be NULL */
  /* forward outputs */
  double *y, *hT, *H; /* hT, H may be NULL */
  /* backward inputs / outputs */
  const double *dy, *dhT; /* dhT may be NULL */
  double *gx, *gdelta, *gh0; /* gh0 may be NULL */
  double *gb_part, *gc_part, *gA_part;
  int64_t nblk; /* channel blocks per batch row */
  int64_t nitems;
  int64_t next; /* shared work counter */
  int failed;
} problem;

static void item_range(const problem* p, int64_t item, int64_t* bb, int64_t* d0, int64_t* d1) {
  *bb = item / p->nblk;
  *d0 = (item % p->nblk) * ORACLE_DBLK;
  *d1 = *d0 + ORACLE_DBLK;
  if (*d1 > p->D) *d1 = p->D;
}

/* Forward over one item.  If Hloc is given it receives the item's states,
 * laid out [t][channel-in-block][n]. */
static void fwd_item(const problem* p, int64_t item, double* h, double* Hloc) {
  const int64_t T = p->T, D = p->D, DS = p->DS;
  int64_t bb, d0, d1;
  item_range(p, item, &bb, &d0, &d1);
  const int64_t nd = d1 - d0;

  for (int64_t k = 0; k < nd; ++k)
    for (int64_t n = 0; n < DS; ++n)
      h[k * DS + n] = p->h0 ? p->h0[(bb * D + d0 + k) * DS + n] : 0.0;

  for (int64_t t = 0; t < T; ++t) {
    const double* bt = p->b + (bb * T + t) * DS;
    const double* ct = p->c + (bb * T + t) * DS;
    for (int64_t k = 0; k < nd; ++k) {
      const int64_t d = d0 + k;
      const int64_t e = (bb * T + t) * D + d;
      const double xv = p->x[e];
      const double dl = p->delta[e];
      double yv = 0.0;
      for (int64_t n = 0; n < DS; ++n) {
        const double a = exp(dl * p->A[d * DS + n]);
        h[k * DS + n] = a * h[k * DS + n] + dl * bt[n] * xv;
        yv += h[k * DS + n] * ct[n];
      }
      if (p->y) p->y[e] = yv;
      if (p->H)
        for (int64_t n = 0; n < DS; ++n) p->H[e * DS + n] = h[k * DS + n];
      if (Hloc)
        for (int64_t n = 0; n < DS; ++n) Hloc[(t * ORACLE_DBLK + k) * DS + n] = h[k * DS + n];
    }
  }
  if (p->hT)
    for (int64_t k = 0; k < nd; ++k)
      for (int64_t n = 0; n < DS; ++n) p->hT[(bb * D + d0 + k) * DS + n] = h[k * DS + n];
}

/* Backward over one item: recompute the item's states, then sweep t downward.
 * G holds the adjoint carried into step t from step t+1, i.e. exp(delta[t+1] A) * g[t+1]
 * (or dhT at the last step).  Per step:
 *   g       = dy[t] * c[t] + G
 *   gx[t]   = delta[t] * sum_n g b[t]
 *   gdelta[t] = sum_n g A a h[t-1]  +  x[t] * sum_n g b[t]
 *   gb[t]  += g delta[t] x[t]        (summed over channels)
 *   gc[t]  += dy[t] h[t]             (summed over channels)
 *   gA     += g h[t-1] a delta[t]    (summed over batch rows and steps)
 *   G       = a g
 * and gh0 is the carry left after step 0. */
static void bwd_item(const problem* p, int64_t item, double* h, double* Hloc, double* G) {
  const int64_t T = p->T, D = p->D, DS = p->DS;
  int64_t bb, d0, d1;
  item_range(p, item, &bb, &d0, &d1);
  const int64_t nd = d1 - d0;

  fwd_item(p, item, h, Hloc);

  double* gbp = p->gb_part + item * T * DS;
  double* gcp = p->gc_part + item * T * DS;
  double* gAp = p->gA_part + item * ORACLE_DBLK * DS;

  for (int64_t k = 0; k < nd; ++k)
    for (int64_t n = 0; n < DS; ++n)
      G[k * DS + n] = p->dhT ? p->dhT[(bb * D + d0 + k) * DS + n] : 0.0;

  for (int64_t t = T - 1; t >= 0; --t) {
    const double* bt = p->b + (bb * T + t) * DS;
    const double* ct = p->c + (bb * T + t) * DS;
    for (int64_t k = 0; k < nd; ++k) {
      const int64_t d = d0 + k;
      const int64_t e = (bb * T + t) * D + d;
      const double xv = p->x[e];
      const double dl = p->delta[e];
      const double dyv = p->dy[e];
      double S = 0.0, gd = 0.0;
      for (int64_t n = 0; n < DS; ++n) {
        const double An = p->A[d * DS + n];
        const double a = exp(dl * An);
        double hp;
        if (t > 0)
          hp = Hloc[((t - 1) * ORACLE_DBLK + k) * DS + n];
        else
          hp = p->h0 ? p->h0[(bb * D + d) * DS + n] : 0.0;
        const double g = dyv * ct[n] + G[k * DS + n];
        S += g * bt[n];
        gd += g * hp * a * An;
        gbp[t * DS + n] += g * dl * xv;
        gcp[t * DS + n] += dyv * Hloc[(t * ORACLE_DBLK + k) * DS + n];
        gAp[k * DS + n] += g * hp * a * dl;
        G[k * DS + n] = a * g;
      }
      p->gx[e] = dl * S;
      p->gdelta[e] = gd + xv * S;
    }
  }
  if (p->gh0)
    for (int64_t k = 0; k < nd; ++k)
      for (int64_t n = 0; n < DS; ++n) p->gh0[(bb * D + d0 + k) * DS + n] = G[k * DS + n];
}

typedef struct {
  problem* p;
  int backward;
} worker_arg;

static void* worker(void* arg_) {
  worker_arg* arg = (worker_arg*)arg_;
  problem* p = arg->p;
  const int64_t DS = p->DS;
  double* h = (double*)malloc(sizeof(double) * ORACLE_DBLK * DS);
  double* G = (double*)malloc(sizeof(double) * ORACLE_DBLK * DS);
  double* Hloc = NULL;
  if (arg->backward) Hloc = (double*)malloc(sizeof(double) * (size_t)(p->T > 0 ? p->T : 1) * ORACLE_DBLK * DS);
  if (!h || !G || (arg->backward && !Hloc)) {
    __atomic_store_n(&p->failed, 1, __ATOMIC_SEQ_CST);
  } else {
    for (;;) {
      const int64_t item = __atomic_fetch_add(&p->next, 1, __ATOMIC_SEQ_CST);
      if (item >= p->nitems) break;
      if (arg->backward)
        bwd_item(p, item, h, Hloc, G);
      else
        fwd_item(p, item, h, NULL);
    }
  }
  free(h);
  free(G);
  free(Hloc);
  return NULL;
}

static int run_items(problem* p, int backward, int nthreads) {
  p->nblk = (p->D + ORACLE_DBLK - 1) / ORACLE_DBLK;
  p->nitems = p->B * p->nblk;
  p->next = 0;
  p->failed = 0;
  if (p->nitems == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > p->nitems) nthreads = (int)p->nitems;
  worker_arg arg = {p, backward};
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, worker, &arg) != 0) break;
    ++started;
  }
  if (started == 0) worker(&arg); /* no threads available: run inline */
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  return p->failed ? -2 : 0;
}

static int check_dims(int64_t B, int64_t T, int64_t D, int64_t DS) {
  return (B < 0 || T < 0 || D < 0 || DS < 1) ? -1 : 0;
}

/* Forward.  y: (B,T,D); hT: (B,D,DS) or NULL; H: (B,T,D,DS) or NULL.
 * Returns 0, -1 on bad sizes, -2 on allocation failure. */
int sscan_oracle_fwd(int64_t B, int64_t T, int64_t D, int64_t DS, const double* x, const double* delta,
                     const double* A, const double* b, const double* c, const double* h0, double* y,
                     double* hT, double* H, int nthreads) {
  if (check_dims(B, T, D, DS)) return -1;
  problem p;
  memset(&p, 0, sizeof(p));
  p.B = B; p.T = T; p.D = D; p.DS = DS;
  p.x = x; p.delta = delta; p.A = A; p.b = b; p.c = c; p.h0 = h0;
  p.y = y; p.hT = hT; p.H = H;
  return run_items(&p, 0, nthreads);
}

/* Backward.  dy: (B,T,D); dhT: (B,D,DS) or NULL.
 * Outputs: gx, gdelta (B,T,D); gb, gc (B,T,DS); gA (D,DS); gh0 (B,D,DS) or NULL.
 * Every output is overwritten.  Returns 0, -1 on bad sizes, -2 on allocation failure. */
int sscan_oracle_bwd(int64_t B, int64_t T, int64_t D, int64_t DS, const double* dy, const double* dhT,
                     const double* x, const double* delta, const double* A, const double* b,
                     const double* c, const double* h0, double* gx, double* gdelta, double* gb,
                     double* gc, double* gA, double* gh0, int nthreads) {
  if (check_dims(B, T, D, DS)) return -1;
  problem p;
  memset(&p, 0, sizeof(p));
  p.B = B; p.T = T; p.D = D; p.DS = DS;
  p.x = x; p.delta = delta; p.A = A; p.b = b; p.c = c; p.h0 = h0;
  p.dy = dy; p.dhT = dhT;
  p.gx = gx; p.gdelta = gdelta; p.gh0 = gh0;
  const int64_t nblk = (D + ORACLE_DBLK - 1) / ORACLE_DBLK;
  const int64_t nitems = B * nblk;
  const size_t nbc = (size_t)(nitems > 0 ? nitems : 1) * (size_t)(T > 0 ? T : 1) * (size_t)DS;
  p.gb_part = (double*)calloc(nbc, sizeof(double));
  p.gc_part = (double*)calloc(nbc, sizeof(double));
  p.gA_part = (double*)calloc((size_t)(nitems > 0 ? nitems : 1) * ORACLE_DBLK * (size_t)DS, sizeof(double));
  int rc = -2;
  if (p.gb_part && p.gc_part && p.gA_part) rc = run_items(&p, 1, nthreads);
  if (rc == 0) {
    /* gb, gc: per batch row, sum the channel-block partials in ascending block order. */
    for (int64_t bb = 0; bb < B; ++bb)
      for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < DS; ++n) {
          double sb = 0.0, sc = 0.0;
          for (int64_t k = 0; k < nblk; ++k) {
            const int64_t item = bb * nblk + k;
            sb += p.gb_part[(item * T + t) * DS + n];
            sc += p.gc_part[(item * T + t) * DS + n];
          }
          gb[(bb * T + t) * DS + n] = sb;
          gc[(bb * T + t) * DS + n] = sc;
        }
    /* gA: sum the per-item partials over batch rows in ascending order. */
    for (int64_t d = 0; d < D; ++d)
      for (int64_t n = 0; n < DS; ++n) {
        double s = 0.0;
        for (int64_t bb = 0; bb < B; ++bb) {
          const int64_t item = bb * nblk + d / ORACLE_DBLK;
          s += p.gA_part[(item * ORACLE_DBLK + d % ORACLE_DBLK) * DS + n];
        }
        gA[d * DS + n] = s;
      }
  }
  free(p.gb_part);
  free(p.gc_part);
  free(p.gA_part);
  return rc;
}
