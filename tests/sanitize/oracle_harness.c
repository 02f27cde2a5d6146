/*
 * Host-only harness that drives the fp64 oracle (oracle/gdn_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: every entry point on small
 * problems, threaded, with exact checks that need no reference values:
 *   - beta = 0: the state only decays, h_T = e^{sum g} h0 and
 *     o_t = e^{G_t} h0^T q_t;
 *   - the fold of the whole sequence as one group, applied to h0 by the
 *     prefix, gives the forward's final state;
 *   - the prefix of the per-group pairs reproduces the forward's state at
 *     every group boundary (run on the prefix of the sequence);
 *   - argument checks reject bad sizes.
 * Exit status 0 when every check holds (the sanitizers abort on the first
 * error they find).  Test infrastructure: built and run by
 * tests/test_sanitizers.py.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_fwd(int B, int T, int Hqk, int Hv, int dk, int dv, int dtype, const void *q, const void *k,
                   const void *v, const float *g, const float *beta, const float *h0, int hv_lo, int hv_hi,
                   int col_lo, int col_hi, double *o, double *hT, int nthreads);
int gdn_oracle_fold(int B, int T, int Hqk, int Hv, int dk, int dv, int dtype, int ngroups, const void *k,
                    const void *v, const float *g, const float *beta, double *A, double *Bm, int nthreads);
int gdn_oracle_prefix(int BH, int n, int dk, int dv, const float *A, const float *Bm, const float *h_init,
                      double *h_in, double *h_final);

static unsigned long long rng = 88172645463325252ULL;
static float urand(void) {   /* xorshift64 in [-1, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (float)((rng >> 11) * (1.0 / 9007199254740992.0)) * 2.f - 1.f;
}

static int fails = 0;
static void check(int ok, const char *what) {
  if (!ok) { fprintf(stderr, "FAILED: %s\n", what); fails++; }
}

int main(void) {
  enum { B = 2, T = 24, Hqk = 2, Hv = 4, dk = 16, dv = 12, G = 3 };
  const size_t nq = (size_t)B * T * Hqk * dk, nv = (size_t)B * T * Hv * dv, ns = (size_t)B * T * Hv;
  const size_t nh = (size_t)B * Hv * dk * dv;
  float *q = malloc(nq * sizeof(float)), *k = malloc(nq * sizeof(float)), *v = malloc(nv * sizeof(float));
  float *g = malloc(ns * sizeof(float)), *beta = malloc(ns * sizeof(float)), *h0 = malloc(nh * sizeof(float));
  for (size_t i = 0; i < nq; i++) { q[i] = urand(); k[i] = 0.25f * urand(); }
  for (size_t i = 0; i < nv; i++) v[i] = urand();
  for (size_t i = 0; i < ns; i++) { g[i] = -0.1f + 0.05f * urand(); beta[i] = 0.5f + 0.4f * urand(); }
  for (size_t i = 0; i < nh; i++) h0[i] = 0.1f * urand();

  double *o = malloc((size_t)B * T * Hv * dv * sizeof(double)), *hT = malloc(nh * sizeof(double));
  /* beta = 0: pure decay */
  float *b0 = calloc(ns, sizeof(float));
  check(gdn_oracle_fwd(B, T, Hqk, Hv, dk, dv, 0, q, k, v, g, b0, h0, 0, Hv, 0, dv, o, hT, 4) == 0, "fwd runs");
  double err = 0;
  for (int b = 0; b < B; b++)
    for (int h = 0; h < Hv; h++) {
      double G_ = 0;
      for (int t = 0; t < T; t++) {
        G_ += g[((size_t)b * T + t) * Hv + h];
        for (int c = 0; c < dv; c++) {
          double ref = 0;
          for (int i = 0; i < dk; i++)
            ref += (double)h0[(((size_t)b * Hv + h) * dk + i) * dv + c] * q[(((size_t)b * T + t) * Hqk + h / 2) * dk + i];
          ref *= exp(G_);
          err = fmax(err, fabs(o[(((size_t)b * T + t) * Hv + h) * dv + c] - ref));
        }
      }
      for (int i = 0; i < dk * dv; i++)
        err = fmax(err, fabs(hT[((size_t)b * Hv + h) * dk * dv + i] - exp(G_) * h0[((size_t)b * Hv + h) * dk * dv + i]));
    }
  if (err >= 1e-12) fprintf(stderr, "beta = 0: max error %g\n", err);
  check(err < 1e-12, "beta = 0 closed form");

  /* the fold of the whole sequence, applied to h0, is the forward's h_T */
  check(gdn_oracle_fwd(B, T, Hqk, Hv, dk, dv, 0, q, k, v, g, beta, h0, 0, Hv, 0, dv, o, hT, 3) == 0, "fwd runs");
  double *A = malloc((size_t)B * Hv * G * dk * dk * sizeof(double)), *Bm = malloc((size_t)B * Hv * G * dk * dv * sizeof(double));
  check(gdn_oracle_fold(B, T, Hqk, Hv, dk, dv, 0, 1, k, v, g, beta, A, Bm, 2) == 0, "fold runs");
  float *Af = malloc((size_t)B * Hv * G * dk * dk * sizeof(float)), *Bf = malloc((size_t)B * Hv * G * dk * dv * sizeof(float));
  for (size_t i = 0; i < (size_t)B * Hv * dk * dk; i++) Af[i] = (float)A[i];
  for (size_t i = 0; i < (size_t)B * Hv * dk * dv; i++) Bf[i] = (float)Bm[i];
  double *hin = malloc((size_t)B * Hv * G * dk * dv * sizeof(double)), *hfin = malloc(nh * sizeof(double));
  check(gdn_oracle_prefix(B * Hv, 1, dk, dv, Af, Bf, h0, hin, hfin) == 0, "prefix runs");
  err = 0;
  for (size_t i = 0; i < nh; i++) err = fmax(err, fabs(hfin[i] - hT[i]) / (1.0 + fabs(hT[i])));
  check(err < 1e-5, "fold + prefix = forward (fp32 pairs)");

  /* three groups: the prefix's incoming states are the forward's states at
     the group boundaries */
  check(gdn_oracle_fold(B, T, Hqk, Hv, dk, dv, 0, G, k, v, g, beta, A, Bm, 4) == 0, "fold runs");
  for (size_t i = 0; i < (size_t)B * Hv * G * dk * dk; i++) Af[i] = (float)A[i];
  for (size_t i = 0; i < (size_t)B * Hv * G * dk * dv; i++) Bf[i] = (float)Bm[i];
  check(gdn_oracle_prefix(B * Hv, G, dk, dv, Af, Bf, h0, hin, hfin) == 0, "prefix runs");
  err = 0;
  for (int j = 1; j < G; j++) {
    const int Tj = j * (T / G);
    /* forward over the first Tj tokens of every (batch, head): a sub-problem
       of its own, copied out of the packed arrays */
    float *qs = malloc((size_t)B * Tj * Hqk * dk * sizeof(float)), *ks = malloc((size_t)B * Tj * Hqk * dk * sizeof(float));
    float *vs = malloc((size_t)B * Tj * Hv * dv * sizeof(float));
    float *gs = malloc((size_t)B * Tj * Hv * sizeof(float)), *bs = malloc((size_t)B * Tj * Hv * sizeof(float));
    for (int b = 0; b < B; b++) {
      memcpy(qs + (size_t)b * Tj * Hqk * dk, q + (size_t)b * T * Hqk * dk, (size_t)Tj * Hqk * dk * sizeof(float));
      memcpy(ks + (size_t)b * Tj * Hqk * dk, k + (size_t)b * T * Hqk * dk, (size_t)Tj * Hqk * dk * sizeof(float));
      memcpy(vs + (size_t)b * Tj * Hv * dv, v + (size_t)b * T * Hv * dv, (size_t)Tj * Hv * dv * sizeof(float));
      memcpy(gs + (size_t)b * Tj * Hv, g + (size_t)b * T * Hv, (size_t)Tj * Hv * sizeof(float));
      memcpy(bs + (size_t)b * Tj * Hv, beta + (size_t)b * T * Hv, (size_t)Tj * Hv * sizeof(float));
    }
    check(gdn_oracle_fwd(B, Tj, Hqk, Hv, dk, dv, 0, qs, ks, vs, gs, bs, h0, 0, Hv, 0, dv, NULL, hT, 4) == 0, "fwd runs");
    for (int bh = 0; bh < B * Hv; bh++)
      for (int i = 0; i < dk * dv; i++) {
        const double x = hin[((size_t)bh * G + j) * dk * dv + i], y = hT[(size_t)bh * dk * dv + i];
        err = fmax(err, fabs(x - y) / (1.0 + fabs(y)));
      }
    free(qs); free(ks); free(vs); free(gs); free(bs);
  }
  check(err < 1e-5, "prefix = forward at group boundaries");

  /* argument checks */
  check(gdn_oracle_fwd(B, T, Hqk, 3, dk, dv, 0, q, k, v, g, beta, h0, 0, 3, 0, dv, o, hT, 1) == -1, "H_v % H_qk");
  check(gdn_oracle_fwd(B, T, Hqk, Hv, dk, dv, 0, q, k, v, g, beta, h0, 2, 1, 0, dv, o, hT, 1) == -1, "head range");
  check(gdn_oracle_fold(B, T, Hqk, Hv, dk, dv, 0, 5, k, v, g, beta, A, Bm, 1) == -1, "groups divide T");
  check(gdn_oracle_prefix(0, 1, dk, dv, Af, Bf, h0, hin, hfin) == -1, "prefix sizes");

  free(q); free(k); free(v); free(g); free(beta); free(h0); free(o); free(hT); free(b0);
  free(A); free(Bm); free(Af); free(Bf); free(hin); free(hfin);
  if (fails) return 1;
  printf("oracle harness: all checks passed\n");
  return 0;
}
