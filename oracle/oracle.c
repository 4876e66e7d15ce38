/*
 * oracle.c -- plain fp64 CPU reference for attention forward and backward and row softmax.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * Everything here is the textbook definition written out, in double precision
 * with libm exp/log, one row at a time, with no blocking or fusion:
 *
 *   softmax   -- the three-pass "safe softmax" (max, then sum of exp(x - max),
 *                then exp(x - max)/sum): infra-guide "5.2 CUDA Online
 *                Softmax", section 1.1.
 *   attention -- O = softmax(scale * Q K^T) V, computed by materialising one
 *                row of scores at a time (the double-precision host reference
 *                of "100 Days of GPU, Day 97", section "Two paths, one head,
 *                one reference"); the causal rule lets query i see keys
 *                j <= i ("Online Softmax: Tiling Across a Reduction", the
 *                paragraphs on causal attention).  The per-row statistic is
 *                the natural-log logsumexp of the scaled scores, lse = m + ln l.
 *
 * Two further routines restate the online forms the pages derive, so tests
 * can check that each equals the definition (the pages assert exact
 * equality):
 *
 *   oracle_online_normaliser   -- the scalar recurrence of the infra-guide
 *                                 page, section 2.1 (step 1: new max, step 2:
 *                                 rescale the old sum and add the new term).
 *   oracle_attention_tiled_row -- the per-tile update equations of "Online
 *                                 softmax, and the register that can't move",
 *                                 section "Online softmax": m, l and O all
 *                                 rescaled by exp(m_old - m_new), O/l once at
 *                                 the end.  It records every rescale factor.
 *
 * The masked forms are the same definition over an explicit visible set:
 *
 *   oracle_attention_ranged   -- the same with an explicit key range per query
 *                                (sliding windows and document boundaries of
 *                                "Online Softmax: Tiling Across a Reduction").
 *
 *   oracle_attention_keyset   -- the same with an explicit key list per query
 *                                (block-sparse masks, same paragraph).
 *
 * The backward pass (gradients of O with respect to Q, K and V for an
 * upstream gradient dO) is the chain rule through that definition:
 *
 *   oracle_attention_backward -- dV = P^T dO, dP = dO V^T,
 *                                dS = P o (dP - D) with D_i = sum_j P_ij dP_ij
 *                                (= <dO_i, O_i>; optionally from a given O),
 *                                dQ = scale dS K, dK = scale dS^T Q,
 *                                in the order the backward-pass paragraphs of
 *                                "Online Softmax: Tiling Across a Reduction"
 *                                describe: the forward statistics of
 *                                every row first, then every score recomputed
 *                                from Q and K and normalised with the saved
 *                                statistic in one step (no running update).
 *
 * All arrays are row-major and owned by the caller.  Threads split rows (or,
 * in the second backward pass, key columns) only.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* a minimal parallel-for over rows                                         */
/* ------------------------------------------------------------------------ */
typedef void (*row_fn)(void* ctx, long r, double* scratch);

typedef struct {
  row_fn fn;
  void* ctx;
  long begin, end;
  long scratch_len;
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  double* scratch = j->scratch_len ? (double*)malloc(sizeof(double) * (size_t)j->scratch_len) : NULL;
  for (long r = j->begin; r < j->end; ++r) j->fn(j->ctx, r, scratch);
  free(scratch);
  return NULL;
}

static void parallel_rows(row_fn fn, void* ctx, long nrows, long scratch_len, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* tid = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  long per = (nrows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].begin = t * per < nrows ? t * per : nrows;
    jobs[t].end = (t + 1) * per < nrows ? (t + 1) * per : nrows;
    jobs[t].scratch_len = scratch_len;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&tid[t], NULL, run_job, &jobs[t]);
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(tid[t], NULL);
  free(jobs);
  free(tid);
}

/* ------------------------------------------------------------------------ */
/* row softmax: three passes over the row                                   */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double* x;
  double* y;
  long cols;
} softmax_ctx;

static void softmax_one_row(void* p, long r, double* scratch) {
  (void)scratch;
  softmax_ctx* c = (softmax_ctx*)p;
  const double* x = c->x + r * c->cols;
  double* y = c->y + r * c->cols;
  double m = -INFINITY;
  for (long j = 0; j < c->cols; ++j)          /* pass 1: the row maximum */
    if (x[j] > m) m = x[j];
  double l = 0.0;
  for (long j = 0; j < c->cols; ++j)          /* pass 2: sum of exp(x - m) */
    l += exp(x[j] - m);
  for (long j = 0; j < c->cols; ++j)          /* pass 3: normalise */
    y[j] = exp(x[j] - m) / l;
}

void oracle_softmax_rows(const double* x, double* y, long rows, long cols, int nthreads) {
  softmax_ctx c = {x, y, cols};
  parallel_rows(softmax_one_row, &c, rows, 0, nthreads);
}

/* ------------------------------------------------------------------------ */
/* attention: one materialised row of scores per query                      */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double *q, *k, *v;
  long n, d;
  double scale;
  int causal;
  const long* rows;  /* query indices to compute */
  double* o;         /* [nrows][d] */
  double* lse;       /* [nrows] */
} attn_ctx;

/* number of keys query i may attend to */
static long visible_keys(long i, long n, int causal) { return causal ? i + 1 : n; }

/* s[j] = scale * <q_i, k_j> for the visible keys; returns their count */
static long score_row(const attn_ctx* c, long i, double* s) {
  long nvis = visible_keys(i, c->n, c->causal);
  const double* qi = c->q + i * c->d;
  for (long j = 0; j < nvis; ++j) {
    const double* kj = c->k + j * c->d;
    double acc = 0.0;
    for (long e = 0; e < c->d; ++e) acc += qi[e] * kj[e];
    s[j] = c->scale * acc;
  }
  return nvis;
}

static void attention_one_row(void* p, long r, double* s) {
  attn_ctx* c = (attn_ctx*)p;
  long i = c->rows[r];
  long nvis = score_row(c, i, s);
  double m = -INFINITY;
  for (long j = 0; j < nvis; ++j)             /* pass 1: the row maximum */
    if (s[j] > m) m = s[j];
  double l = 0.0;
  for (long j = 0; j < nvis; ++j)             /* pass 2: sum of exp(s - m) */
    l += exp(s[j] - m);
  double* o = c->o + r * c->d;
  for (long e = 0; e < c->d; ++e) o[e] = 0.0;
  for (long j = 0; j < nvis; ++j) {           /* pass 3: P = exp(s - m)/l, O = P V */
    double pij = exp(s[j] - m) / l;
    const double* vj = c->v + j * c->d;
    for (long e = 0; e < c->d; ++e) o[e] += pij * vj[e];
  }
  c->lse[r] = m + log(l);
}

void oracle_attention_rows(const double* q, const double* k, const double* v, long n, long d,
                           double scale, int causal, const long* rows, long nrows, double* o,
                           double* lse, int nthreads) {
  attn_ctx c = {q, k, v, n, d, scale, causal, rows, o, lse};
  parallel_rows(attention_one_row, &c, nrows, n, nthreads);
}

/* Attention where query i sees exactly the keys lo[i] .. hi[i] (inclusive): the
 * structured masks of "Online Softmax: Tiling Across a Reduction" (the paragraph
 * on sliding windows, block sparsity and document masks) written as an explicit
 * key range per query.  Same three passes as above over that range. */
typedef struct {
  const double *q, *k, *v;
  long n, d;
  double scale;
  const long *lo, *hi, *rows;
  double *o, *lse;
} ranged_ctx;

static void ranged_one_row(void* p, long r, double* s) {
  ranged_ctx* c = (ranged_ctx*)p;
  const long i = c->rows[r], j0 = c->lo[i], j1 = c->hi[i];
  const double* qrow = c->q + i * c->d;
  for (long j = j0; j <= j1; ++j) {
    const double* kj = c->k + j * c->d;
    double acc = 0.0;
    for (long e = 0; e < c->d; ++e) acc += qrow[e] * kj[e];
    s[j - j0] = c->scale * acc;
  }
  const long cnt = j1 - j0 + 1;
  double m = -INFINITY;
  for (long t = 0; t < cnt; ++t)              /* pass 1: the row maximum */
    if (s[t] > m) m = s[t];
  double l = 0.0;
  for (long t = 0; t < cnt; ++t) l += exp(s[t] - m);   /* pass 2: the sum */
  double* o = c->o + r * c->d;
  for (long e = 0; e < c->d; ++e) o[e] = 0.0;
  for (long t = 0; t < cnt; ++t) {            /* pass 3: P V */
    const double pij = exp(s[t] - m) / l;
    const double* vj = c->v + (j0 + t) * c->d;
    for (long e = 0; e < c->d; ++e) o[e] += pij * vj[e];
  }
  c->lse[r] = log(l) + m;
}

/* lo[i] <= hi[i] must hold for every i (an empty range has no softmax) */
void oracle_attention_ranged(const double* q, const double* k, const double* v, long n, long d,
                             double scale, const long* lo, const long* hi, const long* rows,
                             long nrows, double* o, double* lse, int nthreads) {
  ranged_ctx c = {q, k, v, n, d, scale, lo, hi, rows, o, lse};
  parallel_rows(ranged_one_row, &c, nrows, n, nthreads);
}

/* Attention where query rows[r] sees exactly the keys keys[ptr[r]] .. keys[ptr[r+1] - 1]
 * (any set, in any order): the block-sparse masks of "Online Softmax: Tiling Across a
 * Reduction" (the paragraph on sliding windows, block sparsity and document masks)
 * written as an explicit key list per query.  The same three passes over that list.
 * A query whose list is empty has no softmax: its output row is zero and its
 * logsumexp is -inf. */
typedef struct {
  const double *q, *k, *v;
  long d;
  double scale;
  const long *ptr, *keys, *rows;
  double *o, *lse;
} keyset_ctx;

static void keyset_one_row(void* p, long r, double* sc) {
  keyset_ctx* c = (keyset_ctx*)p;
  const long b0 = c->ptr[r], cnt = c->ptr[r + 1] - c->ptr[r];
  const double* qv = c->q + c->rows[r] * c->d;
  double* out = c->o + r * c->d;
  for (long e = 0; e < c->d; ++e) out[e] = 0.0;
  if (cnt == 0) {
    c->lse[r] = -INFINITY;
    return;
  }
  double mx = -INFINITY;
  for (long t = 0; t < cnt; ++t) {            /* scores; pass 1: their maximum */
    const double* kk = c->k + c->keys[b0 + t] * c->d;
    double dot = 0.0;
    for (long e = 0; e < c->d; ++e) dot += kk[e] * qv[e];
    sc[t] = dot * c->scale;
    if (sc[t] > mx) mx = sc[t];
  }
  double den = 0.0;
  for (long t = 0; t < cnt; ++t) den += exp(sc[t] - mx);   /* pass 2: the sum */
  for (long t = 0; t < cnt; ++t) {                          /* pass 3: P V */
    const double w = exp(sc[t] - mx) / den;
    const double* vv = c->v + c->keys[b0 + t] * c->d;
    for (long e = 0; e < c->d; ++e) out[e] += w * vv[e];
  }
  c->lse[r] = mx + log(den);
}

/* max_keys bounds ptr[r+1] - ptr[r] (the score scratch of one row) */
void oracle_attention_keyset(const double* q, const double* k, const double* v, long d, double scale,
                             const long* ptr, const long* keys, const long* rows, long nrows,
                             long max_keys, double* o, double* lse, int nthreads) {
  keyset_ctx c = {q, k, v, d, scale, ptr, keys, rows, o, lse};
  parallel_rows(keyset_one_row, &c, nrows, max_keys > 0 ? max_keys : 1, nthreads);
}

/* the probability row p_ij = exp(s_ij - m_i)/l_i (zero for hidden keys) */
void oracle_attention_probs(const double* q, const double* k, long n, long d, double scale,
                            int causal, long i, double* p) {
  attn_ctx c = {q, k, NULL, n, d, scale, causal, NULL, NULL, NULL};
  long nvis = score_row(&c, i, p);
  double m = -INFINITY;
  for (long j = 0; j < nvis; ++j)
    if (p[j] > m) m = p[j];
  double l = 0.0;
  for (long j = 0; j < nvis; ++j) l += exp(p[j] - m);
  for (long j = 0; j < nvis; ++j) p[j] = exp(p[j] - m) / l;
  for (long j = nvis; j < n; ++j) p[j] = 0.0;
}

/* ------------------------------------------------------------------------ */
/* online forms                                                             */
/* ------------------------------------------------------------------------ */

/* Scalar online normaliser: after element j, m is the max of x[0..j] and dsum
 * is the sum of exp(x - m) over the same elements. */
void oracle_online_normaliser(const double* x, long n, double* m_out, double* d_out) {
  double m = -INFINITY, dsum = 0.0;
  for (long j = 0; j < n; ++j) {
    double m_next = x[j] > m ? x[j] : m;                  /* step 1: new max */
    dsum = dsum * exp(m - m_next) + exp(x[j] - m_next);   /* step 2: rescale, add */
    m = m_next;
  }
  *m_out = m;
  *d_out = dsum;
}

/* Tile-wise attention for query row i with key tiles of `tile` keys.
 * alphas[t] receives exp(m_old - m_new) of tile t; returns the tile count. */
long oracle_attention_tiled_row(const double* q, const double* k, const double* v, long n, long d,
                                double scale, int causal, long i, long tile, double* o,
                                double* lse, double* alphas) {
  attn_ctx c = {q, k, v, n, d, scale, causal, NULL, NULL, NULL};
  long nvis = visible_keys(i, n, causal);
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  score_row(&c, i, s);
  double m = -INFINITY, l = 0.0;
  for (long e = 0; e < d; ++e) o[e] = 0.0;
  long t = 0;
  for (long j0 = 0; j0 < nvis; j0 += tile, ++t) {
    long j1 = j0 + tile < nvis ? j0 + tile : nvis;
    double rowmax = -INFINITY;
    for (long j = j0; j < j1; ++j)
      if (s[j] > rowmax) rowmax = s[j];
    double m_new = rowmax > m ? rowmax : m;               /* m_new = max(m_old, rowmax) */
    double alpha = exp(m - m_new);                        /* exp(m_old - m_new) */
    double psum = 0.0;
    for (long j = j0; j < j1; ++j) psum += exp(s[j] - m_new);
    l = l * alpha + psum;                                 /* l rescaled, tile sum added */
    for (long e = 0; e < d; ++e) o[e] = o[e] * alpha;     /* O rescaled ... */
    for (long j = j0; j < j1; ++j) {                      /* ... plus exp(S - m_new) V */
      double pj = exp(s[j] - m_new);
      const double* vj = v + j * d;
      for (long e = 0; e < d; ++e) o[e] += pj * vj[e];
    }
    m = m_new;
    alphas[t] = alpha;
  }
  for (long e = 0; e < d; ++e) o[e] = o[e] / l;           /* O / l once, at the end */
  *lse = m + log(l);
  free(s);
  return t;
}

/* ------------------------------------------------------------------------ */
/* backward pass by recomputation                                            */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double *q, *k, *v, *dout;
  long n, d;
  double scale;
  int causal;
  double *dq, *dk, *dv; /* [n][d] each */
  double *lse, *dd;     /* [n] each: saved row statistic and D_i */
  const double* o_in;   /* [n][d] or NULL: the forward output a caller holds */
  double *mq, *mk, *mv; /* [n][d] each or NULL: sums of the absolute values of the terms */
} bwd_ctx;

/* pass 1, query row i: scores, their statistics (lse_i), dP_ij = <dO_i, v_j>,
 * D_i = sum_j P_ij dP_ij and dQ_i = scale sum_j P_ij (dP_ij - D_i) k_j */
static void backward_row(void* p, long i, double* scratch) {
  bwd_ctx* c = (bwd_ctx*)p;
  const long n = c->n, d = c->d;
  double* s = scratch;       /* scores of row i */
  double* dp = scratch + n;  /* dP of row i */
  attn_ctx ac = {c->q, c->k, c->v, n, d, c->scale, c->causal, NULL, NULL, NULL};
  const long nvis = score_row(&ac, i, s);
  double m = -INFINITY;
  for (long j = 0; j < nvis; ++j)
    if (s[j] > m) m = s[j];
  double l = 0.0;
  for (long j = 0; j < nvis; ++j) l += exp(s[j] - m);
  const double* doi = c->dout + i * d;
  for (long j = 0; j < nvis; ++j) {
    const double* vj = c->v + j * d;
    double acc = 0.0;
    for (long e = 0; e < d; ++e) acc += doi[e] * vj[e];
    dp[j] = acc;
  }
  double di = 0.0;
  if (c->o_in) { /* D_i = <dO_i, O_i> with the O the caller holds */
    const double* oi = c->o_in + i * d;
    for (long e = 0; e < d; ++e) di += doi[e] * oi[e];
  } else {
    for (long j = 0; j < nvis; ++j) di += exp(s[j] - m) / l * dp[j];
  }
  double* dqi = c->dq + i * d;
  double* mqi = c->mq ? c->mq + i * d : NULL;
  for (long e = 0; e < d; ++e) dqi[e] = 0.0;
  if (mqi)
    for (long e = 0; e < d; ++e) mqi[e] = 0.0;
  for (long j = 0; j < nvis; ++j) {
    const double ds = exp(s[j] - m) / l * (dp[j] - di);
    const double* kj = c->k + j * d;
    for (long e = 0; e < d; ++e) dqi[e] += c->scale * ds * kj[e];
    if (mqi)
      for (long e = 0; e < d; ++e) mqi[e] += c->scale * fabs(ds * kj[e]);
  }
  c->lse[i] = m + log(l);
  c->dd[i] = di;
}

/* pass 2, key column j: for every query i that sees key j, the score is
 * recomputed and normalised with the saved statistic, P_ij = exp(s_ij - lse_i);
 * dV_j = sum_i P_ij dO_i and dK_j = scale sum_i P_ij (dP_ij - D_i) q_i */
static void backward_col(void* p, long j, double* scratch) {
  (void)scratch;
  bwd_ctx* c = (bwd_ctx*)p;
  const long n = c->n, d = c->d;
  const double* kj = c->k + j * d;
  const double* vj = c->v + j * d;
  double* dkj = c->dk + j * d;
  double* dvj = c->dv + j * d;
  double* mkj = c->mk ? c->mk + j * d : NULL;
  double* mvj = c->mv ? c->mv + j * d : NULL;
  for (long e = 0; e < d; ++e) dkj[e] = dvj[e] = 0.0;
  if (mkj)
    for (long e = 0; e < d; ++e) mkj[e] = mvj[e] = 0.0;
  for (long i = c->causal ? j : 0; i < n; ++i) {
    const double* qi = c->q + i * d;
    const double* doi = c->dout + i * d;
    double sij = 0.0, dpij = 0.0;
    for (long e = 0; e < d; ++e) {
      sij += qi[e] * kj[e];
      dpij += doi[e] * vj[e];
    }
    const double pij = exp(c->scale * sij - c->lse[i]);
    const double ds = pij * (dpij - c->dd[i]);
    for (long e = 0; e < d; ++e) {
      dvj[e] += pij * doi[e];
      dkj[e] += c->scale * ds * qi[e];
    }
    if (mkj)
      for (long e = 0; e < d; ++e) {
        mvj[e] += fabs(pij * doi[e]);
        mkj[e] += c->scale * fabs(ds * qi[e]);
      }
  }
}

/* o_in may be NULL (D from the definition) or the forward output a caller holds,
 * rounded as it is stored: D_i = <dO_i, O_i> then uses it, as a backward pass that
 * receives O does; everything else is unchanged.  mq, mk, mv may be NULL, or
 * receive the same sums over absolute values of their terms (scale sum_j |dS_ij k_j|,
 * scale sum_i |dS_ij q_i|, sum_i |P_ij dO_i|): the magnitudes that rounding errors
 * of P and dS scale with. */
void oracle_attention_backward(const double* q, const double* k, const double* v,
                               const double* dout, const double* o_in, long n, long d,
                               double scale, int causal, double* dq, double* dk, double* dv,
                               double* lse, double* dd, double* mq, double* mk, double* mv,
                               int nthreads) {
  bwd_ctx c = {q, k, v, dout, n, d, scale, causal, dq, dk, dv, lse, dd, o_in, mq, mk, mv};
  parallel_rows(backward_row, &c, n, 2 * n, nthreads);
  parallel_rows(backward_col, &c, n, 0, nthreads);
}
