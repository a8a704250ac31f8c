/*
 * sanitize_check.c -- runs every entry point of gdn_oracle.c on small inputs
 * held in exact-size heap buffers, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only; see oracle/build.py).  It also
 * checks that the recurrent and chunkwise forms agree and that a decode step
 * equals the recurrence over one token, so a run that only stays inside its
 * buffers but computes nonsense still fails.
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle itself.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_ref_recurrent(long B, long T, int Hk, int Hv, int dk, int dv, int gate_mode,
                      const double* q, const double* k, const double* v,
                      const double* beta_or_b, const double* w, const double* g,
                      double scale, const double* state_in, double* state_out, double* o,
                      int nthreads);
int gdn_ref_chunkwise(long B, long T, int Hk, int Hv, int dk, int dv, int gate_mode,
                      const double* q, const double* k, const double* v,
                      const double* beta_or_b, const double* w, const double* g,
                      double scale, const double* state_in, double* state_out, double* o,
                      int C, int nthreads);
int gdn_ref_decode(long N, int Hk, int Hv, int dk, int dv, int gate_mode, const double* q,
                   const double* k, const double* v, const double* beta_or_b, const double* w,
                   const double* g, double scale, double* state, double* o, int nthreads);
int gdn_ref_backward(long B, long T, int Hk, int Hv, int dk, int dv, int gate_mode,
                     const double* q, const double* k, const double* v,
                     const double* beta_or_b, const double* w, const double* g, double scale,
                     const double* state_in, const double* d_o, const double* d_state_out,
                     double* dq, double* dk_out, double* dv_out, double* db, double* dw,
                     double* dg, double* d_state_in, int nthreads);

static unsigned long long rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in [0, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0;
}
static double* buf(long n, double lo, double hi) {  /* exact size, never 0 bytes */
  double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  for (long i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
  return p;
}
static int finite_all(const double* p, long n) {
  for (long i = 0; i < n; ++i) if (!isfinite(p[i])) return 0;
  return 1;
}
static double maxdiff(const double* a, const double* b, long n) {
  double m = 0.0;
  for (long i = 0; i < n; ++i) { double d = fabs(a[i] - b[i]); if (d > m) m = d; }
  return m;
}

static int fails = 0;
#define CHECK(cond, ...) do { if (!(cond)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); ++fails; } } while (0)

static void one_case(long B, long T, int Hk, int Hv, int dk, int dv, int mode, int with_g,
                     int with_s0, int C) {
  const long nqk = B * T * Hk * dk, nv = B * T * Hv * dv;
  const long ng = mode ? B * T * Hv * dk : B * T * Hv, ns = B * Hv * dk * dv;
  double *q = buf(nqk, -0.3, 0.3), *k = buf(nqk, -0.3, 0.3), *v = buf(nv, -1, 1);
  double *b = buf(ng, 0, 1), *w = mode ? buf(nv, 0, 1) : NULL;
  double *g = with_g ? buf(ng, -1.5, 0) : NULL, *s0 = with_s0 ? buf(ns, -0.5, 0.5) : NULL;
  double *o1 = buf(nv, 0, 0), *o2 = buf(nv, 0, 0), *s1 = buf(ns, 0, 0), *s2 = buf(ns, 0, 0);
  CHECK(gdn_ref_recurrent(B, T, Hk, Hv, dk, dv, mode, q, k, v, b, w, g, 0.7, s0, s1, o1, 1) == 0,
        "recurrent rejected B%ld T%ld", B, T);
  CHECK(gdn_ref_chunkwise(B, T, Hk, Hv, dk, dv, mode, q, k, v, b, w, g, 0.7, s0, s2, o2, C, 1) == 0,
        "chunkwise rejected B%ld T%ld C%d", B, T, C);
  CHECK(finite_all(o1, nv) && finite_all(s1, ns), "recurrent not finite T%ld", T);
  CHECK(maxdiff(o1, o2, nv) < 1e-9 && maxdiff(s1, s2, ns) < 1e-9,
        "recurrent and chunkwise differ T%ld C%d mode%d: %g %g", T, C, mode,
        maxdiff(o1, o2, nv), maxdiff(s1, s2, ns));
  /* backward, with and without an upstream state gradient */
  double *d_o = buf(nv, -1, 1), *dsT = buf(ns, -1, 1);
  double *dq = buf(nqk, 0, 0), *dkk = buf(nqk, 0, 0), *dvv = buf(nv, 0, 0), *db = buf(ng, 0, 0);
  double *dw = mode ? buf(nv, 0, 0) : NULL, *dg = with_g ? buf(ng, 0, 0) : NULL;
  double *ds0 = buf(ns, 0, 0);
  for (int use_dsT = 0; use_dsT < 2; ++use_dsT) {
    CHECK(gdn_ref_backward(B, T, Hk, Hv, dk, dv, mode, q, k, v, b, w, g, 0.7, s0, d_o,
                           use_dsT ? dsT : NULL, dq, dkk, dvv, db, dw, dg, ds0, 1) == 0,
          "backward rejected T%ld", T);
    CHECK(finite_all(dq, nqk) && finite_all(dkk, nqk) && finite_all(dvv, nv) &&
              finite_all(db, ng) && (!dw || finite_all(dw, nv)) && (!dg || finite_all(dg, ng)) &&
              finite_all(ds0, ns),
          "backward not finite T%ld", T);
  }
  /* one decode step = the recurrence over the first token of every sequence */
  if (T >= 1) {
    const long N = B;
    double *qd = buf(N * Hk * dk, 0, 0), *kd = buf(N * Hk * dk, 0, 0), *vd = buf(N * Hv * dv, 0, 0);
    double *bd = buf(mode ? N * Hv * dk : N * Hv, 0, 0), *wd = mode ? buf(N * Hv * dv, 0, 0) : NULL;
    double *gd = with_g ? buf(mode ? N * Hv * dk : N * Hv, 0, 0) : NULL;
    double *st = buf(ns, 0, 0), *od = buf(N * Hv * dv, 0, 0);
    for (long n = 0; n < N; ++n) {
      memcpy(qd + n * Hk * dk, q + n * T * Hk * dk, sizeof(double) * Hk * dk);
      memcpy(kd + n * Hk * dk, k + n * T * Hk * dk, sizeof(double) * Hk * dk);
      memcpy(vd + n * Hv * dv, v + n * T * Hv * dv, sizeof(double) * Hv * dv);
      const long gw = mode ? Hv * dk : Hv;
      memcpy(bd + n * gw, b + n * T * gw, sizeof(double) * gw);
      if (gd) memcpy(gd + n * gw, g + n * T * gw, sizeof(double) * gw);
      if (wd) memcpy(wd + n * Hv * dv, w + n * T * Hv * dv, sizeof(double) * Hv * dv);
    }
    if (s0) memcpy(st, s0, sizeof(double) * ns); else memset(st, 0, sizeof(double) * ns);
    CHECK(gdn_ref_decode(N, Hk, Hv, dk, dv, mode, qd, kd, vd, bd, wd, gd, 0.7, st, od, 1) == 0,
          "decode rejected");
    double *o3 = buf(N * Hv * dv, 0, 0), *s3 = buf(ns, 0, 0);
    /* the first token alone, through the recurrence */
    CHECK(gdn_ref_recurrent(N, 1, Hk, Hv, dk, dv, mode, qd, kd, vd, bd, wd, gd, 0.7, s0, s3, o3, 1) == 0,
          "recurrent T1 rejected");
    CHECK(maxdiff(od, o3, N * Hv * dv) < 1e-12 && maxdiff(st, s3, ns) < 1e-12, "decode differs");
    free(qd); free(kd); free(vd); free(bd); free(wd); free(gd); free(st); free(od); free(o3); free(s3);
  }
  free(q); free(k); free(v); free(b); free(w); free(g); free(s0);
  free(o1); free(o2); free(s1); free(s2); free(d_o); free(dsT);
  free(dq); free(dkk); free(dvv); free(db); free(dw); free(dg); free(ds0);
}

int main(void) {
  const long Ts[] = {1, 2, 15, 17, 33, 70};
  int cases = 0;
  for (int ti = 0; ti < 6; ++ti)
    for (int mode = 0; mode < 2; ++mode)
      for (int with_g = 0; with_g < 2; ++with_g)
        for (int with_s0 = 0; with_s0 < 2; ++with_s0) {
          one_case(2, Ts[ti], 1, 2, 8, 4, mode, with_g, with_s0, ti % 2 ? 16 : 7);
          ++cases;
        }
  /* the argument checks reject bad shapes without touching memory */
  CHECK(gdn_ref_recurrent(1, 1, 2, 3, 8, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, 1.0, NULL,
                          NULL, NULL, 1) != 0, "H_v %% H_k accepted");
  CHECK(gdn_ref_chunkwise(1, 1, 1, 1, 8, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, 1.0, NULL,
                          NULL, NULL, 0, 1) != 0, "C = 0 accepted");
  if (fails) { fprintf(stderr, "%d check(s) failed\n", fails); return 1; }
  printf("ok %d cases\n", cases);
  return 0;
}
