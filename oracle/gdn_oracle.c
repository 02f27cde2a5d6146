/*
 * gdn_oracle.c -- fp64 CPU oracle for the Gated DeltaNet forward recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (plain definitions, no blocking, no chunking):
 *
 *  gdn_oracle_fwd     The per-token gated delta rule, one token at a time:
 *                        S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *                        o_t = S_t^T q_t
 *                     S is d_k x d_v per value head.  This rule is the one
 *                     whose chunk-level image is the inter-chunk step
 *                     h' = (exp(g_last) I - k_g^T w) h + k_g^T u printed in
 *                     "Shard the GatedDeltaNet sequence under
 *                     ici_context_parallelism" (PR description) and in
 *                     "GatedDeltaNet does not support ici_context_parallelism"
 *                     (section "The recurrence is affine ...").
 *
 *  gdn_oracle_fold    For each group of consecutive tokens, the affine map
 *                     h -> A h + B that the group applies to the state: A is
 *                     the ordered product of the per-token maps
 *                     exp(g_t)(I - beta_t k_t k_t^T) (latest token on the
 *                     left), B is the state reached from h = 0: the per-group
 *                     affine map of "GatedDeltaNet does not support
 *                     ici_context_parallelism", section "The recurrence is
 *                     affine, so it can be parallelized".
 *
 *  gdn_oracle_prefix  The exclusive prefix of a list of affine pairs applied
 *                     to an initial state: h_in[0] = h_init,
 *                     h_in[j+1] = A_j h_in[j] + B_j, final = h_in[n].  This is
 *                     the composition law (A2,B2)o(A1,B1) = (A2 A1, A2 B1 + B2)
 *                     of the issue page, applied one pair at a time, with the
 *                     exclusive pick of the incoming-state routine in the
 *                     code-review suggestion on the PR page.
 *
 * Inputs are read in their stored type (fp32, or bf16 as raw 16-bit words)
 * and widened to double, so a bf16 workload is evaluated on exactly the
 * rounded values the GPU receives.  All arithmetic is fp64.
 *
 * Layouts (row-major, contiguous):
 *   q, k  [B, T, Hqk, dk]      v  [B, T, Hv, dv]      g, beta [B, T, Hv] fp32
 *   h0    [B, Hv, dk, dv] fp32 (NULL = zero state)
 *   value head hv reads query/key head hv / (Hv / Hqk).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

static double load_elem(const void *p, int dtype, size_t i) {
  if (dtype == ORACLE_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float *)p)[i];
}

/* ------------------------------------------------------------------------ */
/* Work splitting: a fixed list of independent units handed out by a        */
/* shared counter under a mutex.                                            */

typedef struct {
  pthread_mutex_t lock;
  long next, total;
  void (*run)(void *ctx, long unit);
  void *ctx;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  for (;;) {
    pthread_mutex_lock(&p->lock);
    long u = p->next < p->total ? p->next++ : -1;
    pthread_mutex_unlock(&p->lock);
    if (u < 0) break;
    p->run(p->ctx, u);
  }
  return NULL;
}

static int run_units(long total, int nthreads, void (*run)(void *, long), void *ctx) {
  pool_t p;
  pthread_mutex_init(&p.lock, NULL);
  p.next = 0;
  p.total = total;
  p.run = run;
  p.ctx = ctx;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > total) nthreads = (int)(total > 0 ? total : 1);
  pthread_t tid[256];
  int started = 0;
  for (int i = 1; i < nthreads; i++)
    if (pthread_create(&tid[started], NULL, pool_worker, &p) == 0) started++;
  pool_worker(&p);
  for (int i = 0; i < started; i++) pthread_join(tid[i], NULL);
  pthread_mutex_destroy(&p.lock);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token recurrence.                                                    */

typedef struct {
  int B, T, Hqk, Hv, dk, dv, dtype;
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  int hv_lo, nh, col_lo, nc, col_block;
  int nblk;
  double *o, *hT;
} fwd_ctx;

static void fwd_unit(void *vctx, long unit) {
  fwd_ctx *c = (fwd_ctx *)vctx;
  const int blk = (int)(unit % c->nblk);
  const int hh = (int)((unit / c->nblk) % c->nh);
  const int b = (int)(unit / ((long)c->nblk * c->nh));
  const int hv = c->hv_lo + hh;
  const int hq = hv / (c->Hv / c->Hqk);
  const int j0 = c->col_lo + blk * c->col_block;
  int j1 = j0 + c->col_block;
  if (j1 > c->col_lo + c->nc) j1 = c->col_lo + c->nc;
  const int w = j1 - j0;
  const int dk = c->dk, dv = c->dv;

  double *S = (double *)calloc((size_t)dk * w, sizeof(double));
  double *kt = (double *)malloc(sizeof(double) * dk);
  double *qt = (double *)malloc(sizeof(double) * dk);
  double *p = (double *)malloc(sizeof(double) * w);
  if (c->h0) {
    const float *h0 = c->h0 + ((size_t)b * c->Hv + hv) * dk * dv;
    for (int i = 0; i < dk; i++)
      for (int j = 0; j < w; j++) S[(size_t)i * w + j] = (double)h0[(size_t)i * dv + j0 + j];
  }
  for (int t = 0; t < c->T; t++) {
    const size_t qk_off = (((size_t)b * c->T + t) * c->Hqk + hq) * dk;
    const size_t v_off = (((size_t)b * c->T + t) * c->Hv + hv) * dv;
    const size_t s_off = ((size_t)b * c->T + t) * c->Hv + hv;
    const double a = exp((double)c->g[s_off]);
    const double be = (double)c->beta[s_off];
    for (int i = 0; i < dk; i++) {
      kt[i] = load_elem(c->k, c->dtype, qk_off + i);
      qt[i] = load_elem(c->q, c->dtype, qk_off + i);
    }
    /* p = k_t^T S_{t-1} */
    for (int j = 0; j < w; j++) p[j] = 0.0;
    for (int i = 0; i < dk; i++)
      for (int j = 0; j < w; j++) p[j] += kt[i] * S[(size_t)i * w + j];
    /* S_t = a (S - beta k p) + beta k v^T */
    for (int i = 0; i < dk; i++)
      for (int j = 0; j < w; j++) {
        const double vj = load_elem(c->v, c->dtype, v_off + j0 + j);
        double *s = &S[(size_t)i * w + j];
        *s = a * (*s - be * kt[i] * p[j]) + be * kt[i] * vj;
      }
    /* o_t = S_t^T q_t */
    if (c->o) {
      double *orow = c->o + (((size_t)b * c->T + t) * c->nh + hh) * c->nc + (j0 - c->col_lo);
      for (int j = 0; j < w; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++) acc += S[(size_t)i * w + j] * qt[i];
        orow[j] = acc;
      }
    }
  }
  if (c->hT) {
    double *hT = c->hT + ((size_t)b * c->nh + hh) * dk * c->nc;
    for (int i = 0; i < dk; i++)
      for (int j = 0; j < w; j++) hT[(size_t)i * c->nc + (j0 - c->col_lo) + j] = S[(size_t)i * w + j];
  }
  free(S);
  free(kt);
  free(qt);
  free(p);
}

/*
 * Per-token forward over value heads [hv_lo, hv_hi) and state columns
 * [col_lo, col_hi).  The rule is column-separable in d_v, so a column subset
 * is computed exactly as in a full run.
 *   o  [B, T, hv_hi-hv_lo, col_hi-col_lo] fp64   (may be NULL)
 *   hT [B, hv_hi-hv_lo, dk, col_hi-col_lo] fp64  (may be NULL)
 * Returns 0, or -1 on a bad argument.
 */
int gdn_oracle_fwd(int B, int T, int Hqk, int Hv, int dk, int dv, int dtype, const void *q,
                   const void *k, const void *v, const float *g, const float *beta,
                   const float *h0, int hv_lo, int hv_hi, int col_lo, int col_hi, double *o,
                   double *hT, int nthreads) {
  if (B < 1 || T < 0 || Hqk < 1 || Hv < 1 || Hv % Hqk || dk < 1 || dv < 1) return -1;
  if (hv_lo < 0 || hv_hi > Hv || hv_lo >= hv_hi || col_lo < 0 || col_hi > dv || col_lo >= col_hi)
    return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  fwd_ctx c;
  c.B = B; c.T = T; c.Hqk = Hqk; c.Hv = Hv; c.dk = dk; c.dv = dv; c.dtype = dtype;
  c.q = q; c.k = k; c.v = v; c.g = g; c.beta = beta; c.h0 = h0;
  c.hv_lo = hv_lo; c.nh = hv_hi - hv_lo; c.col_lo = col_lo; c.nc = col_hi - col_lo;
  c.col_block = 16;
  c.nblk = (c.nc + c.col_block - 1) / c.col_block;
  c.o = o; c.hT = hT;
  return run_units((long)B * c.nh * c.nblk, nthreads, fwd_unit, &c);
}

/* ------------------------------------------------------------------------ */
/* Group fold: the affine map of each group of consecutive tokens.          */

typedef struct {
  int B, T, Hqk, Hv, dk, dv, dtype, ngroups;
  const void *k, *v;
  const float *g, *beta;
  double *A, *Bm;
} fold_ctx;

static void fold_unit(void *vctx, long unit) {
  fold_ctx *c = (fold_ctx *)vctx;
  const int grp = (int)(unit % c->ngroups);
  const int hv = (int)((unit / c->ngroups) % c->Hv);
  const int b = (int)(unit / ((long)c->ngroups * c->Hv));
  const int hq = hv / (c->Hv / c->Hqk);
  const int dk = c->dk, dv = c->dv;
  const int len = c->T / c->ngroups;
  double *A = c->A + (((size_t)b * c->Hv + hv) * c->ngroups + grp) * dk * dk;
  double *Bm = c->Bm + (((size_t)b * c->Hv + hv) * c->ngroups + grp) * dk * dv;
  double *kt = (double *)malloc(sizeof(double) * dk);
  double *pa = (double *)malloc(sizeof(double) * dk);
  double *pb = (double *)malloc(sizeof(double) * dv);
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dk; j++) A[(size_t)i * dk + j] = (i == j) ? 1.0 : 0.0;
  memset(Bm, 0, sizeof(double) * dk * dv);
  for (int t = grp * len; t < (grp + 1) * len; t++) {
    const size_t k_off = (((size_t)b * c->T + t) * c->Hqk + hq) * dk;
    const size_t v_off = (((size_t)b * c->T + t) * c->Hv + hv) * dv;
    const size_t s_off = ((size_t)b * c->T + t) * c->Hv + hv;
    const double a = exp((double)c->g[s_off]);
    const double be = (double)c->beta[s_off];
    for (int i = 0; i < dk; i++) kt[i] = load_elem(c->k, c->dtype, k_off + i);
    /* A <- a (I - be k k^T) A ;  B <- a (I - be k k^T) B + be k v^T */
    for (int j = 0; j < dk; j++) pa[j] = 0.0;
    for (int j = 0; j < dv; j++) pb[j] = 0.0;
    for (int i = 0; i < dk; i++) {
      for (int j = 0; j < dk; j++) pa[j] += kt[i] * A[(size_t)i * dk + j];
      for (int j = 0; j < dv; j++) pb[j] += kt[i] * Bm[(size_t)i * dv + j];
    }
    for (int i = 0; i < dk; i++) {
      for (int j = 0; j < dk; j++) {
        double *s = &A[(size_t)i * dk + j];
        *s = a * (*s - be * kt[i] * pa[j]);
      }
      for (int j = 0; j < dv; j++) {
        const double vj = load_elem(c->v, c->dtype, v_off + j);
        double *s = &Bm[(size_t)i * dv + j];
        *s = a * (*s - be * kt[i] * pb[j]) + be * kt[i] * vj;
      }
    }
  }
  free(kt);
  free(pa);
  free(pb);
}

/*
 * A  [B, Hv, ngroups, dk, dk] fp64,  Bm [B, Hv, ngroups, dk, dv] fp64.
 * Group j covers tokens [j*T/ngroups, (j+1)*T/ngroups).
 */
int gdn_oracle_fold(int B, int T, int Hqk, int Hv, int dk, int dv, int dtype, int ngroups,
                    const void *k, const void *v, const float *g, const float *beta, double *A,
                    double *Bm, int nthreads) {
  if (B < 1 || T < 1 || Hqk < 1 || Hv < 1 || Hv % Hqk || dk < 1 || dv < 1) return -1;
  if (ngroups < 1 || T % ngroups) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  fold_ctx c;
  c.B = B; c.T = T; c.Hqk = Hqk; c.Hv = Hv; c.dk = dk; c.dv = dv; c.dtype = dtype;
  c.ngroups = ngroups; c.k = k; c.v = v; c.g = g; c.beta = beta; c.A = A; c.Bm = Bm;
  return run_units((long)B * Hv * ngroups, nthreads, fold_unit, &c);
}

/* ------------------------------------------------------------------------ */
/* Exclusive prefix of affine pairs applied to an initial state.            */

/*
 * A [BH, n, dk, dk] fp32, Bm [BH, n, dk, dv] fp32, h_init [BH, dk, dv] fp32 or NULL.
 * h_in [BH, n, dk, dv] fp64 (exclusive: h_in[0] = h_init), h_final [BH, dk, dv] fp64.
 */
int gdn_oracle_prefix(int BH, int n, int dk, int dv, const float *A, const float *Bm,
                      const float *h_init, double *h_in, double *h_final) {
  if (BH < 1 || n < 1 || dk < 1 || dv < 1) return -1;
  double *h = (double *)malloc(sizeof(double) * dk * dv);
  double *hn = (double *)malloc(sizeof(double) * dk * dv);
  for (int bh = 0; bh < BH; bh++) {
    for (size_t e = 0; e < (size_t)dk * dv; e++)
      h[e] = h_init ? (double)h_init[(size_t)bh * dk * dv + e] : 0.0;
    for (int j = 0; j < n; j++) {
      const float *Aj = A + ((size_t)bh * n + j) * dk * dk;
      const float *Bj = Bm + ((size_t)bh * n + j) * dk * dv;
      if (h_in) memcpy(h_in + ((size_t)bh * n + j) * dk * dv, h, sizeof(double) * dk * dv);
      for (int i = 0; i < dk; i++)
        for (int c = 0; c < dv; c++) {
          double acc = (double)Bj[(size_t)i * dv + c];
          for (int m = 0; m < dk; m++) acc += (double)Aj[(size_t)i * dk + m] * h[(size_t)m * dv + c];
          hn[(size_t)i * dv + c] = acc;
        }
      memcpy(h, hn, sizeof(double) * dk * dv);
    }
    if (h_final) memcpy(h_final + (size_t)bh * dk * dv, h, sizeof(double) * dk * dv);
  }
  free(h);
  free(hn);
  return 0;
}
