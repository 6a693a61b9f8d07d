/*
 * kda_oracle.c -- CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP path.
 *
 * What it computes.  KDA is the gated delta rule with a decay per key channel
 * (page "spike(kimi-linear): chunk_kda prefill AOT port", section
 * Delivered).  For one (sequence, head) the state S is a
 * dk x dv matrix (rows: key channels, columns: value channels).  One token t
 * with query q, key k, value v, log-decay g (one per key channel) and write
 * strength beta updates it as
 *
 *     S <- (I - beta k k^T) Diag(exp(g)) S + beta k v^T
 *     o  = scale * S^T q            (read from the state after the update)
 *
 * Expanding the product gives the form evaluated below:
 *     S' = Diag(exp(g)) S                    decay, row i scaled by exp(g_i)
 *     u  = beta * (v - S'^T k)               the delta-rule error
 *     S  = S' + k u^T                        the write
 *     o  = scale * S^T q
 * The prefill runs this token by token from the initial state h0 (zero when
 * absent) and returns the final state; the decode step is the same body run
 * once on a carried state: after one prefill over the prompt, each new token
 * updates the state it inherits from the previous call (page "Kimi-Linear:
 * paged-incremental decode (prefill-once + carried-state decode)", squash
 * commit).
 *
 * Arithmetic is fp64 throughout.  Every (sequence, head) chain is independent,
 * so OpenMP runs the chains in parallel; inside a chain the order of
 * operations is fixed, so results do not depend on the thread count.
 *
 * Layouts (row-major, last index contiguous):
 *   q, k, g  [T, H, dk]      v, o  [T, H, dv]      beta  [T, H]
 *   h0, ht   [N, H, dk, dv]  cu_seqlens [N + 1] (token offsets of each sequence)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on a dk x dv state S (in place); writes o[dv].
 * u is caller-provided scratch of length dv. */
static void kda_token_step(int64_t dk, int64_t dv, double* S, const double* q,
                           const double* k, const double* v, const double* g,
                           double beta, double scale, double* u, double* o) {
  /* decay: row i of S is multiplied by exp(g_i) */
  for (int64_t i = 0; i < dk; ++i) {
    const double d = exp(g[i]);
    double* row = S + i * dv;
    for (int64_t j = 0; j < dv; ++j) row[j] *= d;
  }
  /* u = beta * (v - S^T k) */
  for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
  for (int64_t i = 0; i < dk; ++i) {
    const double ki = k[i];
    const double* row = S + i * dv;
    for (int64_t j = 0; j < dv; ++j) u[j] += row[j] * ki;
  }
  for (int64_t j = 0; j < dv; ++j) u[j] = beta * (v[j] - u[j]);
  /* S += k u^T */
  for (int64_t i = 0; i < dk; ++i) {
    const double ki = k[i];
    double* row = S + i * dv;
    for (int64_t j = 0; j < dv; ++j) row[j] += ki * u[j];
  }
  /* o = scale * S^T q */
  for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
  for (int64_t i = 0; i < dk; ++i) {
    const double qi = q[i];
    const double* row = S + i * dv;
    for (int64_t j = 0; j < dv; ++j) o[j] += row[j] * qi;
  }
  for (int64_t j = 0; j < dv; ++j) o[j] *= scale;
}

int kda_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads later calls use (n >= 1); no effect without OpenMP. */
void kda_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Token-by-token prefill over packed sequences.
 * cu_seqlens: host array [n_seqs + 1], non-decreasing, cu[0] = 0.
 * h0 may be NULL (zero initial state); ht may be NULL (final state dropped).
 * Returns 0, or -1 on a bad argument. */
int kda_oracle_prefill_f64(int64_t n_seqs, int64_t n_heads, int64_t dk, int64_t dv,
                           const int64_t* cu_seqlens, const double* q, const double* k,
                           const double* v, const double* g, const double* beta,
                           const double* h0, double scale, double* o, double* ht) {
  if (n_seqs < 0 || n_heads <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return -1;
  if (cu_seqlens[0] != 0) return -1;
  for (int64_t n = 0; n < n_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int64_t chains = n_seqs * n_heads;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t c = 0; c < chains; ++c) {
    const int64_t n = c / n_heads, h = c % n_heads;
    double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !u) {
      free(S);
      free(u);
      bad |= 1;
      continue;
    }
    if (h0)
      memcpy(S, h0 + c * dk * dv, sizeof(double) * (size_t)(dk * dv));
    else
      memset(S, 0, sizeof(double) * (size_t)(dk * dv));
    for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
      const int64_t th = t * n_heads + h;
      kda_token_step(dk, dv, S, q + th * dk, k + th * dk, v + th * dv, g + th * dk,
                     beta[th], scale, u, o + th * dv);
    }
    if (ht) memcpy(ht + c * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
    free(S);
    free(u);
  }
  return bad ? -1 : 0;
}

/* One decode step for a batch: state [N,H,dk,dv] updated in place;
 * q,k,g [N,H,dk]; v,o [N,H,dv]; beta [N,H]. */
int kda_oracle_decode_f64(int64_t n_seqs, int64_t n_heads, int64_t dk, int64_t dv,
                          double* state, const double* q, const double* k, const double* v,
                          const double* g, const double* beta, double scale, double* o) {
  if (n_seqs < 0 || n_heads <= 0 || dk <= 0 || dv <= 0 || !state) return -1;
  const int64_t chains = n_seqs * n_heads;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t c = 0; c < chains; ++c) {
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!u) {
      bad |= 1;
      continue;
    }
    kda_token_step(dk, dv, state + c * dk * dv, q + c * dk, k + c * dk, v + c * dv,
                   g + c * dk, beta[c], scale, u, o + c * dv);
    free(u);
  }
  return bad ? -1 : 0;
}
