/*
 * Oracle for the gated delta rule recurrence: plain, slow, FP64, CPU only.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline of the benchmark may load this library. The product path (the HIP
 * library) never calls it, and it shares no code with that path.
 *
 * What it computes. The Megatron-LM pull request "fold q/k L2-norm into the
 * gated_delta_rule kernel" (section What) and the flash-linear-attention pull
 * request on the fused q/k/v short conv (Benchmark section) name the operation
 * (FLA's gated_delta_rule / chunk_gated_delta_rule) without printing its
 * formula. Reading: it is the gated delta rule of Gated DeltaNet (Yang, Kautz
 * and Hatamizadeh, ICLR 2025):
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * with S_0 = 0 unless an initial state is given.
 *
 * S is dv x dk (rows follow the value dimension, columns the key dimension).
 * Written row by row: with S' = exp(g_t) S_{t-1}, row i of S' (I - b k k^T) is
 * S'_i - b (S'_i . k) k^T, so
 *
 *     S_t[i] = S'_i + beta_t (v_t[i] - S'_i . k_t) k_t^T.
 *
 * Every row evolves independently of the others, which is the only reason
 * the work is split over threads by (sequence, value head, block of rows);
 * each row is updated token by token in order, with no blocking or chunking.
 *
 * Layouts (all row-major, FP64):
 *   q, k          [T_total, Hqk, dk]   already L2-normalised by the caller
 *                                      when the normalisation is on
 *   v             [T_total, Hv, dv]
 *   g, beta       [T_total, Hv]
 *   cu_seqlens    [n_seqs + 1]         sequence n is tokens [cu[n], cu[n+1])
 *   initial_state [n_seqs, Hv, dv, dk] or NULL (zero state)
 *   out_o         [T_total, Hv, dv]
 *   final_state   [n_seqs, Hv, dv, dk] or NULL
 * Value head h reads query/key head h / (Hv / Hqk) (heads are repeated in
 * groups of Hv/Hqk consecutive value heads).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const double *q, *k, *v, *g, *beta;
  const int64_t *cu;
  int64_t n_seqs, Hqk, Hv, dk, dv, rows_per_unit, units_per_head;
  double scale;
  const double *init;
  double *o, *fin;
  int64_t n_units;
  int64_t next; /* guarded by lock */
  pthread_mutex_t lock;
  int failed;
} job_t;

static void run_unit(job_t *J, int64_t unit, double *S) {
  const int64_t per_seq = J->Hv * J->units_per_head;
  const int64_t n = unit / per_seq;
  const int64_t h = (unit % per_seq) / J->units_per_head;
  const int64_t r0 = (unit % J->units_per_head) * J->rows_per_unit;
  int64_t r1 = r0 + J->rows_per_unit;
  if (r1 > J->dv) r1 = J->dv;
  const int64_t dk = J->dk, dv = J->dv, Hv = J->Hv, Hqk = J->Hqk;
  const int64_t hk = h / (Hv / Hqk);

  /* S rows r0..r1-1 of (sequence n, head h) */
  for (int64_t i = r0; i < r1; ++i)
    for (int64_t j = 0; j < dk; ++j)
      S[(i - r0) * dk + j] =
          J->init ? J->init[((n * Hv + h) * dv + i) * dk + j] : 0.0;

  for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
    const double *kt = J->k + (t * Hqk + hk) * dk;
    const double *qt = J->q + (t * Hqk + hk) * dk;
    const double *vt = J->v + (t * Hv + h) * dv;
    const double decay = exp(J->g[t * Hv + h]);
    const double b = J->beta[t * Hv + h];
    for (int64_t i = r0; i < r1; ++i) {
      double *Si = S + (i - r0) * dk;
      for (int64_t j = 0; j < dk; ++j) Si[j] *= decay; /* S' = e^g S */
      double sk = 0.0;
      for (int64_t j = 0; j < dk; ++j) sk += Si[j] * kt[j]; /* S'_i . k */
      const double u = b * (vt[i] - sk);
      for (int64_t j = 0; j < dk; ++j) Si[j] += u * kt[j];
      double sq = 0.0;
      for (int64_t j = 0; j < dk; ++j) sq += Si[j] * qt[j]; /* S_t q */
      J->o[(t * Hv + h) * dv + i] = J->scale * sq;
    }
  }
  if (J->fin)
    for (int64_t i = r0; i < r1; ++i)
      for (int64_t j = 0; j < dk; ++j)
        J->fin[((n * Hv + h) * dv + i) * dk + j] = S[(i - r0) * dk + j];
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  double *S = (double *)malloc(sizeof(double) * J->rows_per_unit * J->dk);
  if (!S) {
    pthread_mutex_lock(&J->lock);
    J->failed = 1;
    pthread_mutex_unlock(&J->lock);
    return NULL;
  }
  for (;;) {
    pthread_mutex_lock(&J->lock);
    const int64_t u = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (u >= J->n_units) break;
    run_unit(J, u, S);
  }
  free(S);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int oracle_gated_delta_rule(const double *q, const double *k, const double *v,
                            const double *g, const double *beta,
                            const int64_t *cu_seqlens, int64_t n_seqs,
                            int64_t Hqk, int64_t Hv, int64_t dk, int64_t dv,
                            double scale, const double *initial_state,
                            double *out_o, double *final_state,
                            int64_t rows_per_unit, int n_threads) {
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !out_o) return -1;
  if (n_seqs < 1 || Hqk < 1 || Hv < 1 || dk < 1 || dv < 1) return -1;
  if (Hv % Hqk != 0) return -1;
  if (rows_per_unit < 1) rows_per_unit = dv;
  if (n_threads < 1) n_threads = 1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.cu = cu_seqlens;
  J.n_seqs = n_seqs; J.Hqk = Hqk; J.Hv = Hv; J.dk = dk; J.dv = dv;
  J.scale = scale; J.init = initial_state; J.o = out_o; J.fin = final_state;
  J.rows_per_unit = rows_per_unit;
  J.units_per_head = (dv + rows_per_unit - 1) / rows_per_unit;
  J.n_units = n_seqs * Hv * J.units_per_head;
  pthread_mutex_init(&J.lock, NULL);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
  if (!th) return -2;
  int started = 0;
  for (int i = 0; i < n_threads; ++i) {
    if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
    ++started;
  }
  if (started == 0) worker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return J.failed ? -2 : 0;
}
