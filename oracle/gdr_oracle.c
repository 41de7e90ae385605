/*
 * gdr_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU reference for the gated delta rule (the recurrence at
 * the heart of Gated DeltaNet / GDN linear attention, the method the FlashQLA
 * pages accelerate: FlashQLA curated summary, sections "中文摘要" and
 * "GDN Chunked Prefill的效率問題"; blog "FlashQLA：Qwen 把線性注意力推進 DGX
 * Spark 的 2-3× 加速 kernel", section "FlashQLA 解的是什麼").
 *
 * Only tests/, the smoke entry and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (token by token, no chunking, no reformulation):
 *   per sequence n and value head h (query/key head hk = h / G, G = Hv / Hq):
 *     S = initial_state[n, h]  (or zero)                        -- [K, V]
 *     for each token t of sequence n, in order:
 *       S   <- exp(g[t, h]) * S                                  (gate decay)
 *       p   <- S^T k[t, hk]                                      (read before write)
 *       u   <- beta[t, h] * (v[t, h] - p)                        (delta)
 *       S   <- S + k[t, hk] u^T                                  (rank-1 write)
 *       o[t, h] <- scale * S^T q[t, hk]                          (read after write)
 *     final_state[n, h] <- S
 *   which is S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   with o_t = scale * S_t^T q_t.
 *
 * The reverse mode walks the same recurrence backwards (adjoint of each of the
 * five statements above, in reverse order), with the state checkpointed every
 * 64 tokens and recomputed inside each 64-token span.  The 64 is only a memory
 * device of the oracle: the arithmetic is identical for any checkpoint step.
 *
 * Layouts (row-major, fp64):
 *   q, k      [Ttot, Hq, K]       v, o, do  [Ttot, Hv, V]
 *   g, beta   [Ttot, Hv]          h0, ht, dht, dh0  [N, Hv, K, V]
 *   cu        [N + 1] token offsets of the N sequences (int64)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t N, Hq, Hv, K, V;
  const int64_t *cu;
  const double *q, *k, *v, *g, *beta, *h0, *dout, *dht;
  double scale;
  int64_t t_max;      /* <=0: whole sequence; else only the first t_max tokens */
  int64_t h_begin, h_end; /* value heads (fwd) or q/k heads (bwd) to compute */
  double *o, *ht, *u_out;
  double *dq, *dk, *dv, *dbeta, *dg, *dh0;
  /* work distribution */
  int64_t n_units;
  int64_t next_unit;  /* atomically incremented */
  int status;
} oracle_job;

static int64_t seq_len_limited(const oracle_job *J, int64_t n) {
  int64_t len = J->cu[n + 1] - J->cu[n];
  if (J->t_max > 0 && len > J->t_max) len = J->t_max;
  return len;
}

/* ---------------------------------------------------------------- forward */

static void fwd_unit(oracle_job *J, int64_t n, int64_t h, double *S, double *u) {
  const int64_t K = J->K, V = J->V, Hq = J->Hq, Hv = J->Hv;
  const int64_t G = Hv / Hq, hk = h / G;
  const int64_t t0 = J->cu[n], len = seq_len_limited(J, n);
  if (J->h0)
    memcpy(S, J->h0 + (n * Hv + h) * K * V, sizeof(double) * K * V);
  else
    memset(S, 0, sizeof(double) * K * V);
  for (int64_t t = t0; t < t0 + len; ++t) {
    const double a = exp(J->g[t * Hv + h]);
    const double b = J->beta[t * Hv + h];
    const double *kt = J->k + (t * Hq + hk) * K;
    const double *qt = J->q + (t * Hq + hk) * K;
    const double *vt = J->v + (t * Hv + h) * V;
    for (int64_t i = 0; i < K * V; ++i) S[i] *= a;
    for (int64_t j = 0; j < V; ++j) {
      double p = 0.0;
      for (int64_t i = 0; i < K; ++i) p += S[i * V + j] * kt[i];
      u[j] = b * (vt[j] - p);
    }
    for (int64_t i = 0; i < K; ++i)
      for (int64_t j = 0; j < V; ++j) S[i * V + j] += kt[i] * u[j];
    if (J->u_out) memcpy(J->u_out + (t * Hv + h) * V, u, sizeof(double) * V);
    if (J->o) {
      double *ot = J->o + (t * Hv + h) * V;
      for (int64_t j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * qt[i];
        ot[j] = J->scale * acc;
      }
    }
  }
  if (J->ht) memcpy(J->ht + (n * Hv + h) * K * V, S, sizeof(double) * K * V);
}

static void *fwd_worker(void *arg) {
  oracle_job *J = (oracle_job *)arg;
  double *S = (double *)malloc(sizeof(double) * J->K * J->V);
  double *u = (double *)malloc(sizeof(double) * J->V);
  if (!S || !u) { J->status = -3; free(S); free(u); return NULL; }
  const int64_t nh = J->h_end - J->h_begin;
  for (;;) {
    int64_t unit = __atomic_fetch_add(&J->next_unit, 1, __ATOMIC_RELAXED);
    if (unit >= J->n_units) break;
    fwd_unit(J, unit / nh, J->h_begin + unit % nh, S, u);
  }
  free(S);
  free(u);
  return NULL;
}

/* --------------------------------------------------------------- backward */

#define CKPT 64

/* One sequence n and one q/k head hk: loops over the G value heads of the
 * group so that dq and dk (shared by the group) are summed without races. */
static int bwd_unit(oracle_job *J, int64_t n, int64_t hk) {
  const int64_t K = J->K, V = J->V, Hq = J->Hq, Hv = J->Hv, KV = K * V;
  const int64_t G = Hv / Hq;
  const int64_t t0 = J->cu[n], len = seq_len_limited(J, n);
  const int64_t nck = (len + CKPT - 1) / CKPT;
  double *ck = (double *)malloc(sizeof(double) * KV * (nck > 0 ? nck : 1));
  double *Sprev = (double *)malloc(sizeof(double) * KV * CKPT); /* S_{t-1} per token */
  double *S = (double *)malloc(sizeof(double) * KV);
  double *Sp = (double *)malloc(sizeof(double) * KV);  /* S' = a S_{t-1} */
  double *St = (double *)malloc(sizeof(double) * KV);  /* S_t */
  double *dS = (double *)malloc(sizeof(double) * KV);
  double *vec = (double *)malloc(sizeof(double) * (6 * V + 2 * K));
  if (!ck || !Sprev || !S || !Sp || !St || !dS || !vec) {
    free(ck); free(Sprev); free(S); free(Sp); free(St); free(dS); free(vec);
    return -3;
  }
  double *p = vec, *delta = vec + V, *ddelta = vec + 2 * V, *dp = vec + 3 * V;
  double *vm = vec + 4 * V, *u = vec + 5 * V, *dkt = vec + 6 * V, *dqt = vec + 6 * V + K;

  for (int64_t h = hk * G; h < hk * G + G; ++h) {
    /* forward sweep: checkpoint the state entering every CKPT-token span */
    if (J->h0) memcpy(S, J->h0 + (n * Hv + h) * KV, sizeof(double) * KV);
    else memset(S, 0, sizeof(double) * KV);
    for (int64_t r = 0; r < len; ++r) {
      const int64_t t = t0 + r;
      if (r % CKPT == 0) memcpy(ck + (r / CKPT) * KV, S, sizeof(double) * KV);
      const double a = exp(J->g[t * Hv + h]), b = J->beta[t * Hv + h];
      const double *kt = J->k + (t * Hq + hk) * K, *vt = J->v + (t * Hv + h) * V;
      for (int64_t i = 0; i < KV; ++i) S[i] *= a;
      for (int64_t j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * kt[i];
        u[j] = b * (vt[j] - acc);
      }
      for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < V; ++j) S[i * V + j] += kt[i] * u[j];
    }
    /* reverse sweep */
    if (J->dht) memcpy(dS, J->dht + (n * Hv + h) * KV, sizeof(double) * KV);
    else memset(dS, 0, sizeof(double) * KV);
    for (int64_t c = nck - 1; c >= 0; --c) {
      const int64_t r0 = c * CKPT, r1 = (r0 + CKPT < len) ? r0 + CKPT : len;
      /* recompute S_{t-1} for every token of the span from its checkpoint */
      memcpy(S, ck + c * KV, sizeof(double) * KV);
      for (int64_t r = r0; r < r1; ++r) {
        const int64_t t = t0 + r;
        memcpy(Sprev + (r - r0) * KV, S, sizeof(double) * KV);
        const double a = exp(J->g[t * Hv + h]), b = J->beta[t * Hv + h];
        const double *kt = J->k + (t * Hq + hk) * K, *vt = J->v + (t * Hv + h) * V;
        for (int64_t i = 0; i < KV; ++i) S[i] *= a;
        for (int64_t j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * kt[i];
          u[j] = b * (vt[j] - acc);
        }
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) S[i * V + j] += kt[i] * u[j];
      }
      for (int64_t r = r1 - 1; r >= r0; --r) {
        const int64_t t = t0 + r;
        const double a = exp(J->g[t * Hv + h]), b = J->beta[t * Hv + h];
        const double *kt = J->k + (t * Hq + hk) * K, *qt = J->q + (t * Hq + hk) * K;
        const double *vt = J->v + (t * Hv + h) * V, *dot = J->dout + (t * Hv + h) * V;
        const double *Sm1 = Sprev + (r - r0) * KV;
        /* rebuild the forward quantities of token t */
        for (int64_t i = 0; i < KV; ++i) Sp[i] = a * Sm1[i];
        for (int64_t j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int64_t i = 0; i < K; ++i) acc += Sp[i * V + j] * kt[i];
          p[j] = acc;
          vm[j] = vt[j] - acc;
          delta[j] = b * vm[j];
        }
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) St[i * V + j] = Sp[i * V + j] + kt[i] * delta[j];
        /* o_t = scale * S_t^T q_t */
        for (int64_t i = 0; i < K; ++i) {
          double acc = 0.0;
          for (int64_t j = 0; j < V; ++j) {
            dS[i * V + j] += J->scale * qt[i] * dot[j];
            acc += St[i * V + j] * dot[j];
          }
          dqt[i] = J->scale * acc;
        }
        /* S_t = S' + k delta^T */
        for (int64_t i = 0; i < K; ++i) {
          double acc = 0.0;
          for (int64_t j = 0; j < V; ++j) acc += dS[i * V + j] * delta[j];
          dkt[i] = acc;
        }
        for (int64_t j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int64_t i = 0; i < K; ++i) acc += dS[i * V + j] * kt[i];
          ddelta[j] = acc;
        }
        /* delta = beta (v - p) */
        double db = 0.0;
        for (int64_t j = 0; j < V; ++j) {
          db += ddelta[j] * vm[j];
          J->dv[(t * Hv + h) * V + j] = b * ddelta[j];
          dp[j] = -b * ddelta[j];
        }
        J->dbeta[t * Hv + h] = db;
        /* p = S'^T k : dS' = dS + k dp^T, dk += S' dp */
        for (int64_t i = 0; i < K; ++i) {
          double acc = 0.0;
          for (int64_t j = 0; j < V; ++j) {
            dS[i * V + j] += kt[i] * dp[j];
            acc += Sp[i * V + j] * dp[j];
          }
          dkt[i] += acc;
        }
        /* S' = a S_{t-1}: dg = <dS', S'>, dS_{t-1} = a dS' */
        double dgt = 0.0;
        for (int64_t i = 0; i < KV; ++i) {
          dgt += dS[i] * Sp[i];
          dS[i] *= a;
        }
        J->dg[t * Hv + h] = dgt;
        for (int64_t i = 0; i < K; ++i) {
          J->dq[(t * Hq + hk) * K + i] += dqt[i];
          J->dk[(t * Hq + hk) * K + i] += dkt[i];
        }
      }
    }
    if (J->dh0) memcpy(J->dh0 + (n * Hv + h) * KV, dS, sizeof(double) * KV);
  }
  free(ck); free(Sprev); free(S); free(Sp); free(St); free(dS); free(vec);
  return 0;
}

static void *bwd_worker(void *arg) {
  oracle_job *J = (oracle_job *)arg;
  const int64_t nh = J->h_end - J->h_begin;
  for (;;) {
    int64_t unit = __atomic_fetch_add(&J->next_unit, 1, __ATOMIC_RELAXED);
    if (unit >= J->n_units) break;
    if (bwd_unit(J, unit / nh, J->h_begin + unit % nh) != 0) J->status = -3;
  }
  return NULL;
}

static int run_threads(oracle_job *J, void *(*fn)(void *), int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > J->n_units) nthreads = (int)(J->n_units > 0 ? J->n_units : 1);
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[started], NULL, fn, J) != 0) break;
    ++started;
  }
  fn(J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  return J->status;
}

static int check_common(const oracle_job *J) {
  if (J->N < 0 || J->Hq <= 0 || J->Hv <= 0 || J->K <= 0 || J->V <= 0) return -1;
  if (J->Hv % J->Hq != 0) return -1;
  for (int64_t n = 0; n < J->N; ++n)
    if (J->cu[n + 1] < J->cu[n]) return -1;
  return 0;
}

/* Forward.  Computes value heads [h_begin, h_end) of every sequence; o, ht
 * and u_out may be NULL.  u_out [Ttot, Hv, V] receives the delta vector u that
 * each token writes.  With t_max > 0 only the first t_max tokens of each
 * sequence are processed (ht is then the state after that prefix). */
int oracle_gdr_fwd(int64_t N, const int64_t *cu, int64_t Hq, int64_t Hv, int64_t K,
                   int64_t V, const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale, const double *h0,
                   int64_t t_max, int64_t h_begin, int64_t h_end, double *o, double *ht,
                   double *u_out, int nthreads) {
  oracle_job J;
  memset(&J, 0, sizeof J);
  J.N = N; J.cu = cu; J.Hq = Hq; J.Hv = Hv; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.scale = scale; J.h0 = h0;
  J.t_max = t_max; J.o = o; J.ht = ht; J.u_out = u_out;
  if (check_common(&J) != 0) return -1;
  if (h_begin < 0 || h_end > Hv || h_begin > h_end) return -1;
  J.h_begin = h_begin; J.h_end = h_end;
  J.n_units = N * (h_end - h_begin);
  if (J.n_units == 0) return 0;
  return run_threads(&J, fwd_worker, nthreads);
}

/* Reverse mode of the forward above for the loss <o, dout> + <ht, dht>.
 * Computes q/k heads [hk_begin, hk_end) (and their G value heads).  dq and dk
 * must be zero-initialised by the caller (they are accumulated over the G
 * value heads of a group).  dht and h0 may be NULL (zero). */
int oracle_gdr_bwd(int64_t N, const int64_t *cu, int64_t Hq, int64_t Hv, int64_t K,
                   int64_t V, const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale, const double *h0,
                   const double *dout, const double *dht, int64_t t_max,
                   int64_t hk_begin, int64_t hk_end, double *dq, double *dk, double *dv,
                   double *dbeta, double *dg, double *dh0, int nthreads) {
  oracle_job J;
  memset(&J, 0, sizeof J);
  J.N = N; J.cu = cu; J.Hq = Hq; J.Hv = Hv; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.scale = scale; J.h0 = h0;
  J.dout = dout; J.dht = dht; J.t_max = t_max;
  J.dq = dq; J.dk = dk; J.dv = dv; J.dbeta = dbeta; J.dg = dg; J.dh0 = dh0;
  if (check_common(&J) != 0) return -1;
  if (!dout || !dq || !dk || !dv || !dbeta || !dg) return -1;
  if (hk_begin < 0 || hk_end > Hq || hk_begin > hk_end) return -1;
  J.h_begin = hk_begin; J.h_end = hk_end;
  J.n_units = N * (hk_end - hk_begin);
  if (J.n_units == 0) return 0;
  return run_threads(&J, bwd_worker, nthreads);
}
