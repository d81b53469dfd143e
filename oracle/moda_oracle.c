/*
 * moda_oracle.c -- plain fp64 CPU oracle for the Mixture-of-Depths Attention
 * (MoDA) forward, its gradients, and the depth-stream packing permutation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP path is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  The product library never links
 * it and shares no source, header, table or helper with it.
 *
 * Sources (the pages this follows):
 *   [Notes]  "Mixture-of-Depths Attention: 中文研读笔记", reading notes on
 *            arXiv 2603.15619 at cc.laoqi.cc (files/MoDA-2603.15619).
 *   [Summ]   "Mixture-of-Depths Attention", section-by-section summary at
 *            papercache.org.
 *
 * What is computed (the plain definition; no tiling, no online softmax):
 * for every batch b, token t and query head h, with G = Hq/Hk and the shared
 * KV head hk = floor(h/G) (0-based reading of phi(h) = ceil(h/G), [Summ] 2.1
 * Eq. (2)), and s = 1/sqrt(d):
 *
 *   a_j = s * <q[b,t,h,:], k_seq[b,j,hk,:]>           j in J
 *   b_i = s * <q[b,t,h,:], k_depth[b,t,i,hk,:]>       i in 0..L-1
 *   J   = {0..t} if causal else {0..T-1}              ([Summ] 2.1 Eq. (2) mask)
 *   out = (sum_j e^{a_j} v_seq[b,j,hk,:] + sum_i e^{b_i} v_depth[b,t,i,hk,:])
 *         / (sum_j e^{a_j} + sum_i e^{b_i})
 *   lse = log(sum_j e^{a_j} + sum_i e^{b_i})
 *
 * This is the unified softmax of [Notes] 二.2 (the expansion with a_j, b_i
 * and one shared denominator) and the MoDA operator of [Summ] 2.2: both
 * candidate sets compete in one softmax.  The depth set is the L slots that
 * earlier layers wrote for the same token position t.  Exponentials are
 * taken relative to the row maximum m (a change of variables that leaves the
 * quotient unchanged); lse is reported as m + log(Z).
 *
 * The depth tensors are read in the generation layout [B][T][L][Hk][d]
 * (position t's L slots stored together, [Summ] 3.2 "flash-compatible"
 * layout, with the KV heads innermost as in [Summ] 2.1), NOT in the packed
 * layout the GPU kernel consumes.
 *
 * Inputs may be fp64, fp32 or bf16 (raw 16-bit patterns); every value is
 * widened exactly to fp64 before any arithmetic.  All accumulation is fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

/* Exact widening of one stored element to fp64.  bf16 is the top half of an
 * IEEE binary32, so shifting its 16 bits up by 16 gives the same value. */
static double orc_load(const void* base, size_t idx, int kind) {
  if (kind == ORC_F64) return ((const double*)base)[idx];
  if (kind == ORC_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  const void *q, *k_seq, *v_seq, *k_depth, *v_depth;
  int kind;
  int B, T, Hq, Hk, d, L, causal;
} orc_problem;

/* Flat indices of the row-major tensors. */
static size_t ix_q(const orc_problem* p, int b, int t, int h, int c) {
  return (((size_t)b * p->T + t) * p->Hq + h) * p->d + c;
}
static size_t ix_kv(const orc_problem* p, int b, int j, int hk, int c) {
  return (((size_t)b * p->T + j) * p->Hk + hk) * p->d + c;
}
static size_t ix_depth(const orc_problem* p, int b, int t, int i, int hk, int c) {
  return ((((size_t)b * p->T + t) * p->L + i) * p->Hk + hk) * p->d + c;
}

/* One query row (b, t, h).  `work` holds T + L + d doubles. */
static void orc_row(const orc_problem* p, int b, int t, int h, double* out_row,
                    double* lse_out, double* work) {
  const int G = p->Hq / p->Hk;
  const int hk = h / G;
  const int d = p->d;
  const double s = 1.0 / sqrt((double)d);
  const int nseq = p->causal ? t + 1 : p->T;
  double* logit = work;             /* [nseq] sequence logits, then [L] depth logits */
  double* qrow = work + p->T + p->L; /* [d] */

  for (int c = 0; c < d; ++c) qrow[c] = orc_load(p->q, ix_q(p, b, t, h, c), p->kind);

  /* Logits of both candidate sets, a_j then b_i ([Notes] 二.2). */
  for (int j = 0; j < nseq; ++j) {
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += qrow[c] * orc_load(p->k_seq, ix_kv(p, b, j, hk, c), p->kind);
    logit[j] = s * dot;
  }
  for (int i = 0; i < p->L; ++i) {
    double dot = 0.0;
    for (int c = 0; c < d; ++c)
      dot += qrow[c] * orc_load(p->k_depth, ix_depth(p, b, t, i, hk, c), p->kind);
    logit[nseq + i] = s * dot;
  }
  const int ncand = nseq + p->L;

  double m = -INFINITY;
  for (int n = 0; n < ncand; ++n)
    if (logit[n] > m) m = logit[n];

  /* One shared denominator over both sets. */
  double Z = 0.0;
  for (int n = 0; n < ncand; ++n) {
    logit[n] = exp(logit[n] - m); /* now the unnormalised weight */
    Z += logit[n];
  }

  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int j = 0; j < nseq; ++j) acc += logit[j] * orc_load(p->v_seq, ix_kv(p, b, j, hk, c), p->kind);
    for (int i = 0; i < p->L; ++i)
      acc += logit[nseq + i] * orc_load(p->v_depth, ix_depth(p, b, t, i, hk, c), p->kind);
    out_row[c] = acc / Z;
  }
  *lse_out = m + log(Z);
}

/* ---- row lists and threading ------------------------------------------- */

typedef struct {
  const orc_problem* p;
  const int* rows; /* nrows triples (b, t, h) */
  long long first, last;
  double* out;  /* [nrows][d] */
  double* lse;  /* [nrows] */
} orc_job;

static void* orc_worker(void* arg) {
  orc_job* job = (orc_job*)arg;
  const orc_problem* p = job->p;
  double* work = (double*)malloc(sizeof(double) * ((size_t)p->T + p->L + p->d));
  if (!work) return (void*)1;
  for (long long r = job->first; r < job->last; ++r) {
    const int* rbth = job->rows + 3 * r;
    orc_row(p, rbth[0], rbth[1], rbth[2], job->out + r * p->d, job->lse + r, work);
  }
  free(work);
  return NULL;
}

static int orc_check(const orc_problem* p) {
  if (!p->q || !p->k_seq || !p->v_seq) return -1;
  if (p->L > 0 && (!p->k_depth || !p->v_depth)) return -1;
  if (p->B <= 0 || p->T <= 0 || p->Hq <= 0 || p->Hk <= 0 || p->d <= 0 || p->L < 0) return -2;
  if (p->Hq % p->Hk != 0) return -2;
  if (p->causal != 0 && p->causal != 1) return -2;
  if (p->kind < ORC_F64 || p->kind > ORC_BF16) return -3;
  return 0;
}

static int orc_run_rows(const orc_problem* p, const int* rows, long long nrows, double* out,
                        double* lse, int nthreads) {
  int rc = orc_check(p);
  if (rc) return rc;
  for (long long r = 0; r < nrows; ++r) {
    const int* x = rows + 3 * r;
    if (x[0] < 0 || x[0] >= p->B || x[1] < 0 || x[1] >= p->T || x[2] < 0 || x[2] >= p->Hq) return -4;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  orc_job* jobs = (orc_job*)malloc(sizeof(orc_job) * nthreads);
  if (!tid || !jobs) {
    free(tid);
    free(jobs);
    return -5;
  }
  /* Interleave rows across threads by contiguous chunks of equal count; rows
   * are independent, so the split changes nothing in the results. */
  for (int w = 0; w < nthreads; ++w) {
    jobs[w].p = p;
    jobs[w].rows = rows;
    jobs[w].first = nrows * w / nthreads;
    jobs[w].last = nrows * (w + 1) / nthreads;
    jobs[w].out = out;
    jobs[w].lse = lse;
  }
  int failed = 0;
  for (int w = 1; w < nthreads; ++w)
    if (pthread_create(&tid[w], NULL, orc_worker, &jobs[w]) != 0) {
      tid[w] = 0; /* no thread: run this share on the calling thread */
      if (orc_worker(&jobs[w]) != NULL) failed = 1;
    }
  if (orc_worker(&jobs[0]) != NULL) failed = 1;
  for (int w = 1; w < nthreads; ++w) {
    void* res = NULL;
    if (tid[w]) {
      pthread_join(tid[w], &res);
      if (res != NULL) failed = 1;
    }
  }
  free(tid);
  free(jobs);
  return failed ? -5 : 0;
}

/* ---- exported entry points ---------------------------------------------- */

/* Selected rows.  rows = nrows triples (b, t, h); out = [nrows][d] fp64,
 * lse = [nrows] fp64 (natural log).  kind: 0 fp64, 1 fp32, 2 bf16 inputs.
 * Returns 0, or a negative code for bad arguments / allocation failure. */
int moda_oracle_fwd_rows(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                         const void* v_depth, int kind, int B, int T, int Hq, int Hk, int d, int L,
                         int causal, const int* rows, long long nrows, double* out, double* lse,
                         int nthreads) {
  orc_problem p = {q, k_seq, v_seq, k_depth, v_depth, kind, B, T, Hq, Hk, d, L, causal};
  if (nrows < 0 || (nrows > 0 && (!rows || !out || !lse))) return -1;
  return orc_run_rows(&p, rows, nrows, out, lse, nthreads);
}

/* Every row.  out = [B][T][Hq][d] fp64, lse = [B][Hq][T] fp64. */
int moda_oracle_fwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, int kind, int B, int T, int Hq, int Hk, int d, int L,
                    int causal, double* out, double* lse, int nthreads) {
  orc_problem p = {q, k_seq, v_seq, k_depth, v_depth, kind, B, T, Hq, Hk, d, L, causal};
  int rc = orc_check(&p);
  if (rc) return rc;
  if (!out || !lse) return -1;
  long long nrows = (long long)B * T * Hq;
  int* rows = (int*)malloc(sizeof(int) * 3 * (size_t)nrows);
  double* lse_rows = (double*)malloc(sizeof(double) * (size_t)nrows);
  if (!rows || !lse_rows) {
    free(rows);
    free(lse_rows);
    return -5;
  }
  /* Row order b, t, h matches out's [B][T][Hq][d] layout. */
  long long r = 0;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < Hq; ++h, ++r) {
        rows[3 * r] = b;
        rows[3 * r + 1] = t;
        rows[3 * r + 2] = h;
      }
  rc = orc_run_rows(&p, rows, nrows, out, lse_rows, nthreads);
  if (rc == 0) {
    r = 0;
    for (int b = 0; b < B; ++b)
      for (int t = 0; t < T; ++t)
        for (int h = 0; h < Hq; ++h, ++r) lse[((size_t)b * Hq + h) * T + t] = lse_rows[r];
  }
  free(rows);
  free(lse_rows);
  return rc;
}

/* ---- backward ------------------------------------------------------------ */

/* Gradients of the forward map, by definition: with P_n the softmax weights of
 * row (b, t, h) over its candidates n (the visible sequence keys j, then the L
 * depth slots i), dO the output gradient of the row and
 *   dP_n = <dO, v_n>,   D = sum_n P_n dP_n,   dS_n = P_n (dP_n - D)
 * (the derivative of out = sum_n P_n v_n through the shared denominator):
 *   dq      = s * sum_n dS_n k_n
 *   dk_n   += s * dS_n q          (summed over every row that sees key n)
 *   dv_n   += P_n dO
 * Sequence keys collect contributions from the G heads of every token that
 * sees them; a depth slot of token t only from the G heads of token t.
 * One thread owns one (b, hk): all of that head's keys and the G query heads
 * that read them, so its sums need no synchronisation. */
typedef struct {
  const orc_problem* p;
  const void* dout;
  int first, last; /* (b, hk) pairs [first, last) */
  double *dq, *dk, *dv, *dkd, *dvd;
} orc_bwd_job;

static void* orc_bwd_worker(void* arg) {
  orc_bwd_job* job = (orc_bwd_job*)arg;
  const orc_problem* p = job->p;
  const int G = p->Hq / p->Hk, d = p->d, T = p->T, L = p->L;
  const double s = 1.0 / sqrt((double)p->d);
  double* w = (double*)malloc(sizeof(double) * ((size_t)3 * (T + L) + 2 * (size_t)d));
  if (!w) return (void*)1;
  double* logit = w;            /* [T + L]: logits, then P */
  double* dP = w + (T + L);     /* [T + L] */
  double* dS = w + 2 * (T + L); /* [T + L] */
  double* qrow = w + 3 * (T + L);
  double* dorow = qrow + d;
  for (int pair = job->first; pair < job->last; ++pair) {
    const int b = pair / p->Hk, hk = pair % p->Hk;
    for (int t = 0; t < T; ++t)
      for (int g = 0; g < G; ++g) {
        const int h = hk * G + g;
        const int nseq = p->causal ? t + 1 : T;
        const int ncand = nseq + L;
        for (int c = 0; c < d; ++c) {
          qrow[c] = orc_load(p->q, ix_q(p, b, t, h, c), p->kind);
          dorow[c] = orc_load(job->dout, ix_q(p, b, t, h, c), p->kind);
        }
        /* Forward recomputation: logits, the row max, P. */
        double m = -INFINITY;
        for (int n = 0; n < ncand; ++n) {
          double dot = 0.0, dpv = 0.0;
          for (int c = 0; c < d; ++c) {
            const size_t kix = n < nseq ? ix_kv(p, b, n, hk, c) : ix_depth(p, b, t, n - nseq, hk, c);
            const double kc = orc_load(n < nseq ? p->k_seq : p->k_depth, kix, p->kind);
            const double vc = orc_load(n < nseq ? p->v_seq : p->v_depth, kix, p->kind);
            dot += qrow[c] * kc;
            dpv += dorow[c] * vc;
          }
          logit[n] = s * dot;
          dP[n] = dpv;
          if (logit[n] > m) m = logit[n];
        }
        double Z = 0.0;
        for (int n = 0; n < ncand; ++n) {
          const double e = exp(logit[n] - m);
          logit[n] = e;
          Z += e;
        }
        double D = 0.0;
        for (int n = 0; n < ncand; ++n) {
          logit[n] /= Z; /* P_n */
          D += logit[n] * dP[n];
        }
        for (int n = 0; n < ncand; ++n) dS[n] = logit[n] * (dP[n] - D);
        /* Accumulate. */
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int n = 0; n < ncand; ++n) {
            const size_t kix = n < nseq ? ix_kv(p, b, n, hk, c) : ix_depth(p, b, t, n - nseq, hk, c);
            acc += dS[n] * orc_load(n < nseq ? p->k_seq : p->k_depth, kix, p->kind);
            double* dkp = n < nseq ? job->dk : job->dkd;
            double* dvp = n < nseq ? job->dv : job->dvd;
            dkp[kix] += s * dS[n] * qrow[c];
            dvp[kix] += logit[n] * dorow[c];
          }
          job->dq[ix_q(p, b, t, h, c)] = s * acc;
        }
      }
  }
  free(w);
  return NULL;
}

/* Gradients of every input for the output gradient dout ([B][T][Hq][d], same
 * kind as the inputs).  Outputs fp64, in the input layouts: dq [B][T][Hq][d];
 * dk, dv [B][T][Hk][d]; dkd, dvd [B][T][L][Hk][d].  Returns 0 or a negative code. */
int moda_oracle_bwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, const void* dout, int kind, int B, int T, int Hq, int Hk, int d,
                    int L, int causal, double* dq, double* dk, double* dv, double* dkd, double* dvd,
                    int nthreads) {
  orc_problem p = {q, k_seq, v_seq, k_depth, v_depth, kind, B, T, Hq, Hk, d, L, causal};
  int rc = orc_check(&p);
  if (rc) return rc;
  if (!dout || !dq || !dk || !dv || (L > 0 && (!dkd || !dvd))) return -1;
  memset(dq, 0, sizeof(double) * (size_t)B * T * Hq * d);
  memset(dk, 0, sizeof(double) * (size_t)B * T * Hk * d);
  memset(dv, 0, sizeof(double) * (size_t)B * T * Hk * d);
  if (L > 0) {
    memset(dkd, 0, sizeof(double) * (size_t)B * T * L * Hk * d);
    memset(dvd, 0, sizeof(double) * (size_t)B * T * L * Hk * d);
  }
  const int npairs = B * Hk;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > npairs) nthreads = npairs;
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  orc_bwd_job* jobs = (orc_bwd_job*)malloc(sizeof(orc_bwd_job) * nthreads);
  if (!tid || !jobs) {
    free(tid);
    free(jobs);
    return -5;
  }
  for (int w = 0; w < nthreads; ++w) {
    orc_bwd_job j = {&p, dout, npairs * w / nthreads, npairs * (w + 1) / nthreads, dq, dk, dv, dkd, dvd};
    jobs[w] = j;
  }
  int failed = 0;
  for (int w = 1; w < nthreads; ++w)
    if (pthread_create(&tid[w], NULL, orc_bwd_worker, &jobs[w]) != 0) {
      tid[w] = 0;
      if (orc_bwd_worker(&jobs[w]) != NULL) failed = 1;
    }
  if (orc_bwd_worker(&jobs[0]) != NULL) failed = 1;
  for (int w = 1; w < nthreads; ++w) {
    void* res = NULL;
    if (tid[w]) {
      pthread_join(tid[w], &res);
      if (res != NULL) failed = 1;
    }
  }
  free(tid);
  free(jobs);
  return failed ? -5 : 0;
}

/* ---- sampled gradients -------------------------------------------------------
 *
 * The same gradients as moda_oracle_bwd, for selected outputs only, so that
 * long sequences can be checked without the full quadratic cost:
 *   rows  (b, t, h)   -> dq[b, t, h, :]
 *   keys  (b, j, hk)  -> dk[b, j, hk, :], dv[b, j, hk, :]  (sequence keys)
 *   toks  (b, t, hk)  -> dkd[b, t, :, hk, :], dvd[b, t, :, hk, :]  (all L slots)
 * Each contributing row is evaluated exactly as in moda_oracle_bwd: its full
 * softmax over all its candidates, dP, D and dS.  A key collects from every row
 * that sees it, a depth slot from the G rows of its own token. */

/* P and dS of every candidate of row (b, t, h): P in P_out[0 .. nseq+L), dS in
 * dS_out; qrow / dorow receive the row's q and dout.  Returns nseq. */
static int orc_row_grad(const orc_problem* p, const void* dout, int b, int t, int h, double* P_out,
                        double* dS_out, double* qrow, double* dorow) {
  const int G = p->Hq / p->Hk, hk = h / G, d = p->d, L = p->L;
  const double s = 1.0 / sqrt((double)p->d);
  const int nseq = p->causal ? 1 + t : p->T;
  const int ncand = nseq + L;
  for (int c = 0; c < d; ++c) {
    qrow[c] = orc_load(p->q, ix_q(p, b, t, h, c), p->kind);
    dorow[c] = orc_load(dout, ix_q(p, b, t, h, c), p->kind);
  }
  double m = -INFINITY;
  for (int n = 0; n < ncand; ++n) {
    double dot = 0.0, dpv = 0.0;
    for (int c = 0; c < d; ++c) {
      const size_t kix = n < nseq ? ix_kv(p, b, n, hk, c) : ix_depth(p, b, t, n - nseq, hk, c);
      dot += qrow[c] * orc_load(n < nseq ? p->k_seq : p->k_depth, kix, p->kind);
      dpv += dorow[c] * orc_load(n < nseq ? p->v_seq : p->v_depth, kix, p->kind);
    }
    P_out[n] = s * dot;
    dS_out[n] = dpv; /* dP for now */
    if (P_out[n] > m) m = P_out[n];
  }
  double Z = 0.0;
  for (int n = 0; n < ncand; ++n) {
    P_out[n] = exp(P_out[n] - m);
    Z += P_out[n];
  }
  double D = 0.0;
  for (int n = 0; n < ncand; ++n) {
    P_out[n] /= Z;
    D += P_out[n] * dS_out[n];
  }
  for (int n = 0; n < ncand; ++n) dS_out[n] = P_out[n] * (dS_out[n] - D);
  return nseq;
}

typedef struct {
  const orc_problem* p;
  const void* dout;
  const int* work; /* triples (b, t, h) */
  long long first, last;
  const int *rows, *keys, *toks;
  long long nrows, nkeys, ntoks;
  double *dq, *dk, *dv, *dkd, *dvd; /* this thread's accumulators */
} orc_samp_job;

static void* orc_samp_worker(void* arg) {
  orc_samp_job* j = (orc_samp_job*)arg;
  const orc_problem* p = j->p;
  const int d = p->d, L = p->L, G = p->Hq / p->Hk;
  const double s = 1.0 / sqrt((double)p->d);
  double* w = (double*)malloc(sizeof(double) * (2 * ((size_t)p->T + L) + 2 * (size_t)d));
  if (!w) return (void*)1;
  double *P = w, *dS = w + p->T + L, *qrow = w + 2 * ((size_t)p->T + L), *dorow = qrow + d;
  for (long long r = j->first; r < j->last; ++r) {
    const int b = j->work[3 * r], t = j->work[3 * r + 1], h = j->work[3 * r + 2], hk = h / G;
    const int nseq = orc_row_grad(p, j->dout, b, t, h, P, dS, qrow, dorow);
    for (long long i = 0; i < j->nrows; ++i) /* dq of a sampled row */
      if (j->rows[3 * i] == b && j->rows[3 * i + 1] == t && j->rows[3 * i + 2] == h)
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int n = 0; n < nseq + L; ++n) {
            const size_t kix = n < nseq ? ix_kv(p, b, n, hk, c) : ix_depth(p, b, t, n - nseq, hk, c);
            acc += dS[n] * orc_load(n < nseq ? p->k_seq : p->k_depth, kix, p->kind);
          }
          j->dq[i * d + c] += s * acc;
        }
    for (long long i = 0; i < j->nkeys; ++i) { /* sampled sequence keys this row sees */
      const int kb = j->keys[3 * i], kj = j->keys[3 * i + 1], khk = j->keys[3 * i + 2];
      if (kb != b || khk != hk || kj >= nseq) continue;
      for (int c = 0; c < d; ++c) {
        j->dk[i * d + c] += s * dS[kj] * qrow[c];
        j->dv[i * d + c] += P[kj] * dorow[c];
      }
    }
    for (long long i = 0; i < j->ntoks; ++i) { /* depth slots of a sampled token */
      if (j->toks[3 * i] != b || j->toks[3 * i + 1] != t || j->toks[3 * i + 2] != hk) continue;
      for (int l = 0; l < L; ++l)
        for (int c = 0; c < d; ++c) {
          j->dkd[(i * L + l) * d + c] += s * dS[nseq + l] * qrow[c];
          j->dvd[(i * L + l) * d + c] += P[nseq + l] * dorow[c];
        }
    }
  }
  free(w);
  return NULL;
}

int moda_oracle_bwd_sampled(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                            const void* v_depth, const void* dout, int kind, int B, int T, int Hq, int Hk, int d,
                            int L, int causal, const int* rows, long long nrows, double* dq_rows, const int* keys,
                            long long nkeys, double* dk_keys, double* dv_keys, const int* toks, long long ntoks,
                            double* dkd_toks, double* dvd_toks, int nthreads) {
  orc_problem p = {q, k_seq, v_seq, k_depth, v_depth, kind, B, T, Hq, Hk, d, L, causal};
  int rc = orc_check(&p);
  if (rc) return rc;
  if (!dout || nrows < 0 || nkeys < 0 || ntoks < 0) return -1;
  if ((nrows && (!rows || !dq_rows)) || (nkeys && (!keys || !dk_keys || !dv_keys)) ||
      (ntoks && L > 0 && (!toks || !dkd_toks || !dvd_toks)))
    return -1;
  const int G = Hq / Hk;
  for (long long i = 0; i < nrows; ++i)
    if (rows[3 * i] < 0 || rows[3 * i] >= B || rows[3 * i + 1] < 0 || rows[3 * i + 1] >= T || rows[3 * i + 2] < 0 ||
        rows[3 * i + 2] >= Hq)
      return -2;
  for (long long i = 0; i < nkeys + ntoks; ++i) {
    const int* e = i < nkeys ? keys + 3 * i : toks + 3 * (i - nkeys);
    if (e[0] < 0 || e[0] >= B || e[1] < 0 || e[1] >= T || e[2] < 0 || e[2] >= Hk) return -2;
  }
  /* Mark every row that contributes to a requested output. */
  unsigned char* need = (unsigned char*)calloc((size_t)B * T * Hq, 1);
  if (!need) return -5;
#define NEED(b, t, h) need[((size_t)(b) * T + (t)) * Hq + (h)]
  for (long long i = 0; i < nrows; ++i) NEED(rows[3 * i], rows[3 * i + 1], rows[3 * i + 2]) = 1;
  for (long long i = 0; i < nkeys; ++i)
    for (int t = causal ? keys[3 * i + 1] : 0; t < T; ++t)
      for (int g = 0; g < G; ++g) NEED(keys[3 * i], t, keys[3 * i + 2] * G + g) = 1;
  for (long long i = 0; i < ntoks; ++i)
    for (int g = 0; g < G; ++g) NEED(toks[3 * i], toks[3 * i + 1], toks[3 * i + 2] * G + g) = 1;
  long long nwork = 0;
  for (size_t i = 0; i < (size_t)B * T * Hq; ++i) nwork += need[i];
  int* work = (int*)malloc(sizeof(int) * 3 * (size_t)(nwork > 0 ? nwork : 1));
  if (!work) {
    free(need);
    return -5;
  }
  long long wi = 0;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < Hq; ++h)
        if (NEED(b, t, h)) {
          work[3 * wi] = b;
          work[3 * wi + 1] = t;
          work[3 * wi + 2] = h;
          ++wi;
        }
#undef NEED
  free(need);
  if (nthreads < 1) nthreads = 1;
  if (nwork < nthreads) nthreads = nwork > 0 ? (int)nwork : 1;
  const size_t nq = (size_t)nrows * d, nk = (size_t)nkeys * d, nt = (size_t)ntoks * L * d;
  const size_t per = nq + 2 * nk + 2 * nt;
  double* acc = (double*)calloc((size_t)nthreads * (per > 0 ? per : 1), sizeof(double));
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  orc_samp_job* jobs = (orc_samp_job*)malloc(sizeof(orc_samp_job) * nthreads);
  if (!acc || !tid || !jobs) {
    free(acc);
    free(tid);
    free(jobs);
    free(work);
    return -5;
  }
  for (int w = 0; w < nthreads; ++w) {
    double* a = acc + (size_t)w * per;
    orc_samp_job jb = {&p, dout, work, nwork * w / nthreads, nwork * (w + 1) / nthreads, rows, keys, toks, nrows,
                       nkeys, L > 0 ? ntoks : 0, a, a + nq, a + nq + nk, a + nq + 2 * nk, a + nq + 2 * nk + nt};
    jobs[w] = jb;
  }
  int failed = 0;
  for (int w = 1; w < nthreads; ++w)
    if (pthread_create(&tid[w], NULL, orc_samp_worker, &jobs[w]) != 0) {
      tid[w] = 0;
      if (orc_samp_worker(&jobs[w]) != NULL) failed = 1;
    }
  if (orc_samp_worker(&jobs[0]) != NULL) failed = 1;
  for (int w = 1; w < nthreads; ++w) {
    void* res = NULL;
    if (tid[w]) {
      pthread_join(tid[w], &res);
      if (res != NULL) failed = 1;
    }
  }
  /* Reduce the per-thread partial sums in thread order. */
  for (size_t e = 0; e < nq; ++e) {
    double x = 0.0;
    for (int w = 0; w < nthreads; ++w) x += jobs[w].dq[e];
    dq_rows[e] = x;
  }
  for (size_t e = 0; e < nk; ++e) {
    double x = 0.0, y = 0.0;
    for (int w = 0; w < nthreads; ++w) {
      x += jobs[w].dk[e];
      y += jobs[w].dv[e];
    }
    dk_keys[e] = x;
    dv_keys[e] = y;
  }
  for (size_t e = 0; e < nt; ++e) {
    double x = 0.0, y = 0.0;
    for (int w = 0; w < nthreads; ++w) {
      x += jobs[w].dkd[e];
      y += jobs[w].dvd[e];
    }
    dkd_toks[e] = x;
    dvd_toks[e] = y;
  }
  free(acc);
  free(tid);
  free(jobs);
  free(work);
  return failed ? -5 : 0;
}

/* ---- depth write: KV projection ------------------------------------------------
 *
 * A layer's depth KV comes from the attention branch (its own K, V) or from a KV
 * projection of the FFN input ([Notes] 二.3).  Either is a projection of a
 * token's hidden state x [Dm] by a fused weight w [2*Hk*d][Dm] (output channel n
 * = row n: K channels first, then V), by definition
 *   k[b,t,hk,c] = sum_m x[b,t,m] * w[hk*d + c][m]
 *   v[b,t,hk,c] = sum_m x[b,t,m] * w[Hk*d + hk*d + c][m]
 * Outputs fp64 [B][T][Hk][d]. */
int moda_oracle_kv_project(const void* x, const void* w, int kind, int B, int T, int Dm, int Hk, int d, double* k_out,
                           double* v_out) {
  if (!x || !w || !k_out || !v_out) return -1;
  if (B <= 0 || T <= 0 || Dm <= 0 || Hk <= 0 || d <= 0) return -2;
  if (kind < ORC_F64 || kind > ORC_BF16) return -3;
  const int N = Hk * d;
  for (long long bt = 0; bt < (long long)B * T; ++bt)
    for (int n = 0; n < 2 * N; ++n) {
      double acc = 0.0;
      for (int m = 0; m < Dm; ++m)
        acc += orc_load(x, (size_t)bt * Dm + m, kind) * orc_load(w, (size_t)n * Dm + m, kind);
      double* dst = n < N ? k_out : v_out;
      dst[(size_t)bt * N + (n % N)] = acc;
    }
  return 0;
}

/* Depth-stream packing, by definition: dst[b][t][hk][l][:] = src[b][t][l][hk][:]
 * for elements of elem_bytes bytes.  This is the reorganisation that keeps
 * each position's L depth states together ([Summ] 3.2), with the KV head
 * moved outside the slot index so one (token, KV head) pair's L slots form
 * one contiguous run. */
int moda_oracle_pack_depth(const void* src, void* dst, int B, int T, int L, int Hk, int d,
                           int elem_bytes) {
  if (!src || !dst) return -1;
  if (B <= 0 || T <= 0 || L <= 0 || Hk <= 0 || d <= 0 || elem_bytes <= 0) return -2;
  const unsigned char* s = (const unsigned char*)src;
  unsigned char* o = (unsigned char*)dst;
  const size_t row = (size_t)d * elem_bytes;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int hk = 0; hk < Hk; ++hk)
        for (int l = 0; l < L; ++l) {
          size_t from = ((((size_t)b * T + t) * L + l) * Hk + hk) * row;
          size_t to = ((((size_t)b * T + t) * Hk + hk) * L + l) * row;
          memcpy(o + to, s + from, row);
        }
  return 0;
}

/* Write one layer's K or V, kv[b][t][hk][:], into slot `slot` of a packed
 * depth tensor: dst[b][t][hk][slot][:] = kv[b][t][hk][:] (the "write" step of
 * [Summ] 2.2: a layer appends its KV to the depth stream). */
int moda_oracle_append_depth_slot(const void* kv, void* dst, int slot, int B, int T, int L, int Hk,
                                  int d, int elem_bytes) {
  if (!kv || !dst) return -1;
  if (B <= 0 || T <= 0 || L <= 0 || Hk <= 0 || d <= 0 || elem_bytes <= 0) return -2;
  if (slot < 0 || slot >= L) return -2;
  const unsigned char* s = (const unsigned char*)kv;
  unsigned char* o = (unsigned char*)dst;
  const size_t row = (size_t)d * elem_bytes;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int hk = 0; hk < Hk; ++hk) {
        size_t from = (((size_t)b * T + t) * Hk + hk) * row;
        size_t to = ((((size_t)b * T + t) * Hk + hk) * L + slot) * row;
        memcpy(o + to, s + from, row);
      }
  return 0;
}
