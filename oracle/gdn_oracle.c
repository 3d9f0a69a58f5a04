/*
 * gdn_oracle.c -- plain, slow, sequential fp64 CPU oracle for the Gated
 * DeltaNet recurrence and its replay form.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.  "parity pinned": every function below is checked against
 * closed forms, explicit matrix products and invariants by the CPU test suite
 * (tests/test_oracle_gdn.py), and planted mistakes in a copy of this file
 * must fail those pins.
 *
 * The pages name Gated DeltaNet as a recurrence whose update, like Mamba-2's,
 * unrolls into a decay plus a sum, so the checkpoint-plus-log replay applies
 * to it ("Why Speculative Decoding Slows Hybrid Mamba Models at Large Batch
 * Sizes", section "When Replaying the Inputs Is the Wrong Tool"), but they do
 * not write the update out.  It is taken from its published definition (the
 * gated delta rule of Gated Delta Networks, Yang, Kautz and Hatamizadeh,
 * 2024), per value head h with key group g = h / (H/G):
 *
 *     alpha_t = exp(dt_t[h] * A[h])                  the gate (Mamba-2's decay form)
 *     S_t     = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t     = S_t q_t
 *
 * S is [P, N]: P value rows, N key columns (the same [S,H,P,N] layout as the
 * Mamba-2 state), v_t = v[t,h,:] (P), k_t, q_t = k[t,g,:], q[t,g,:] (N),
 * beta_t = beta[t,h].  Written per row p of S:
 *     d_p    = sum_n S_{t-1}[p,n] k_t[n]           (the row read at key k_t)
 *     S_t[p,n] = alpha_t * (S_{t-1}[p,n] - beta_t d_p k_t[n]) + beta_t v_t[p] k_t[n]
 *     o_t[p] = sum_n S_t[p,n] q_t[n]
 * Sums over n run in increasing n; compile with -ffp-contract=off.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_INVALID_CHUNK (-2)

typedef void (*unit_fn)(void *ctx, int64_t unit);
typedef struct {
  unit_fn fn;
  void *ctx;
  int64_t n_units;
  int n_threads;
  int tid;
} pf_arg;

static void *pf_worker(void *p) {
  pf_arg *a = (pf_arg *)p;
  for (int64_t u = a->tid; u < a->n_units; u += a->n_threads) a->fn(a->ctx, u);
  return NULL;
}

static void parallel_for(unit_fn fn, void *ctx, int64_t n_units, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > n_units) n_threads = (int)(n_units > 0 ? n_units : 1);
  if (n_threads == 1) {
    for (int64_t u = 0; u < n_units; ++u) fn(ctx, u);
    return;
  }
  pthread_t th[256];
  pf_arg args[256];
  for (int i = 0; i < n_threads; ++i) {
    args[i].fn = fn;
    args[i].ctx = ctx;
    args[i].n_units = n_units;
    args[i].n_threads = n_threads;
    args[i].tid = i;
    pthread_create(&th[i], NULL, pf_worker, &args[i]);
  }
  for (int i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
}

static int all_finite(const double *v, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(v[i])) return 0;
  return 1;
}

/* One token for one head: s[P,N] in place, o[P] the output. */
static void gdn_step_head(int P, int N, double alpha, double beta, const double *v /*[P]*/,
                          const double *k /*[N]*/, const double *q /*[N]*/, double *s,
                          double *o /*[P]*/) {
  for (int p = 0; p < P; ++p) {
    double *row = s + (int64_t)p * N;
    double d = 0.0;
    for (int n = 0; n < N; ++n) d += row[n] * k[n];
    for (int n = 0; n < N; ++n) row[n] = alpha * (row[n] - beta * d * k[n]) + beta * v[p] * k[n];
    double acc = 0.0;
    for (int n = 0; n < N; ++n) acc += row[n] * q[n];
    o[p] = acc;
  }
}

/* ------------------------------------------------------------------------ */
/* scan: one stream, L tokens, optional per-token reset                      */
/* ------------------------------------------------------------------------ */
typedef struct {
  int H, P, N, G;
  int64_t L;
  const double *v, *dt, *beta, *k, *q, *A;
  const uint8_t *reset;
  double *state, *o;
} scan_ctx;

static void scan_unit(void *vctx, int64_t h) {
  scan_ctx *c = (scan_ctx *)vctx;
  const int H = c->H, P = c->P, N = c->N, G = c->G;
  const int g = (int)(h / (H / G));
  const int64_t PN = (int64_t)P * N;
  double *s = c->state + h * PN;
  for (int64_t t = 0; t < c->L; ++t) {
    if (c->reset && c->reset[t]) memset(s, 0, sizeof(double) * PN);
    const double alpha = exp(c->dt[t * H + h] * c->A[h]);
    gdn_step_head(P, N, alpha, c->beta[t * H + h], c->v + (t * H + h) * P,
                  c->k + (t * G + g) * N, c->q + (t * G + g) * N, s, c->o + (t * H + h) * P);
  }
}

/*
 * oracle_gdn_scan: advance one stream by L tokens.
 *   v[L,H,P] dt[L,H] beta[L,H] k,q[L,G,N] A[H]; reset[L] or NULL (zero the
 *   state and the position before token t); state[H,P,N] carry-in/out;
 *   pos in/out; o[L,H,P].  ORC_E_INVALID_CHUNK (nothing written) for a
 *   non-finite input.
 */
int oracle_gdn_scan(int H, int P, int N, int G, int64_t L, const double *v, const double *dt,
                    const double *beta, const double *k, const double *q, const double *A,
                    const uint8_t *reset, double *state, int64_t *pos, double *o, int n_threads) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || L < 0) return ORC_E_ARG;
  if (!all_finite(v, L * H * P) || !all_finite(dt, L * H) || !all_finite(beta, L * H) ||
      !all_finite(k, L * G * N) || !all_finite(q, L * G * N))
    return ORC_E_INVALID_CHUNK;
  scan_ctx c = {H, P, N, G, L, v, dt, beta, k, q, A, reset, state, o};
  parallel_for(scan_unit, &c, H, n_threads);
  int64_t p = *pos;
  for (int64_t t = 0; t < L; ++t) {
    if (reset && reset[t]) p = 0;
    p += 1;
  }
  *pos = p;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* speculative verify with rollback: the step-by-step recurrence            */
/* ------------------------------------------------------------------------ */
typedef struct {
  int H, P, N, G, batch, n_in;
  const int32_t *slot, *accepted;
  const double *v, *dt, *beta, *k, *q, *A;
  double *state, *o;
} spec_ctx;

static void spec_unit(void *vctx, int64_t u) {
  spec_ctx *c = (spec_ctx *)vctx;
  const int H = c->H, P = c->P, N = c->N, G = c->G, n_in = c->n_in;
  const int64_t b = u / H, h = u % H;
  const int g = (int)(h / (H / G));
  const int64_t PN = (int64_t)P * N;
  double *s = c->state + ((int64_t)c->slot[b] * H + h) * PN;
  double *work = (double *)malloc(sizeof(double) * PN);
  double *kept = (double *)malloc(sizeof(double) * PN);
  memcpy(work, s, sizeof(double) * PN);
  const int a = c->accepted[b];
  for (int i = 0; i < n_in; ++i) {
    const int64_t bk = b * n_in + i;
    const double alpha = exp(c->dt[bk * H + h] * c->A[h]);
    gdn_step_head(P, N, alpha, c->beta[bk * H + h], c->v + (bk * H + h) * P,
                  c->k + (bk * G + g) * N, c->q + (bk * G + g) * N, work,
                  c->o + (bk * H + h) * P);
    if (i == a - 1) memcpy(kept, work, sizeof(double) * PN);
  }
  memcpy(s, kept, sizeof(double) * PN);
  free(work);
  free(kept);
}

/*
 * oracle_gdn_spec_step: verify n_in in-flight tokens per slot (the real token
 * plus drafts) with the plain recurrence, emit every token's output, keep the
 * state after the first accepted[b] tokens and drop the rest (rejected drafts
 * never reach the state: "Why Speculative Decoding Slows ...", section "The
 * Fix: Log the Inputs, Checkpoint the State").  1 <= accepted[b] <= n_in.
 *   v[batch,n_in,H,P] dt,beta[batch,n_in,H] k,q[batch,n_in,G,N] o[batch,n_in,H,P]
 */
int oracle_gdn_spec_step(int S, int H, int P, int N, int G, int batch, const int32_t *slot,
                         int n_in, const double *v, const double *dt, const double *beta,
                         const double *k, const double *q, const double *A,
                         const int32_t *accepted, double *state, int64_t *pos, double *o,
                         int n_threads) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || batch < 0 || n_in < 1)
    return ORC_E_ARG;
  for (int b = 0; b < batch; ++b) {
    if (slot[b] < 0 || slot[b] >= S) return ORC_E_ARG;
    if (accepted[b] < 1 || accepted[b] > n_in) return ORC_E_ARG;
    for (int b2 = 0; b2 < b; ++b2)
      if (slot[b2] == slot[b]) return ORC_E_ARG;
  }
  const int64_t nt = (int64_t)batch * n_in;
  if (!all_finite(v, nt * H * P) || !all_finite(dt, nt * H) || !all_finite(beta, nt * H) ||
      !all_finite(k, nt * G * N) || !all_finite(q, nt * G * N))
    return ORC_E_INVALID_CHUNK;
  spec_ctx c = {H, P, N, G, batch, n_in, slot, accepted, v, dt, beta, k, q, A, state, o};
  parallel_for(spec_unit, &c, (int64_t)batch * H, n_threads);
  for (int b = 0; b < batch; ++b) pos[slot[b]] += accepted[b];
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* test-only: the replay form (checkpoint + logged inputs)                   */
/* ------------------------------------------------------------------------ */
/*
 * Write A_j = alpha_j (I - beta_j k_j k_j^T) (an N x N matrix).  Unrolled, the
 * state after entries 1..m is
 *     S_m = S_0 A_1 A_2 ... A_m + sum_j beta_j v_j k_j^T A_{j+1} ... A_m,
 * a product of the checkpoint with the entries' factors plus one term per
 * entry: the decay-plus-sum shape the replay trick needs, with matrix factors
 * in place of Mamba-2's scalar decays.
 *
 * oracle_gdn_replay_unrolled computes, for one slot, from the checkpoint
 * ckpt[H,P,N] and a combined list of entries (n_log committed, then n_in
 * in-flight; per entry dt[H], beta[H], v[H,P], k[G,N], q[G,N]):
 *   o[i] for every in-flight entry m = n_log + i, by carrying q_m backwards
 *        through the factors: w <- q_m; for j = m down to 0:
 *        c_j = beta_j (k_j . w), w <- alpha_j (w - c_j k_j); then
 *        o_m = ckpt . w + sum_j c_j v_j  (the state is never formed);
 *   fold_out = S after the n_log committed entries, with the factor product
 *        formed as an explicit N x N matrix T = A_{j+1} ... A_{n_log} while j
 *        runs down: fold = ckpt T_0 + sum_j beta_j v_j (k_j^T T_j).
 */
int oracle_gdn_replay_unrolled(int H, int P, int N, int G, int n_log, int n_in,
                               const double *ckpt, const double *dt_all, const double *beta_all,
                               const double *v_all, const double *k_all, const double *q_all,
                               const double *A, double *o /*[n_in,H,P]*/,
                               double *fold_out /*[H,P,N] or NULL*/) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || n_log < 0 || n_in < 0)
    return ORC_E_ARG;
  const int M = n_log + n_in;
  double *w = (double *)malloc(sizeof(double) * N);
  double *c = (double *)malloc(sizeof(double) * (M > 0 ? M : 1));
  double *T = (double *)malloc(sizeof(double) * N * N);
  double *T2 = (double *)malloc(sizeof(double) * N * N);
  double *r = (double *)malloc(sizeof(double) * N);
  for (int h = 0; h < H; ++h) {
    const int g = h / (H / G);
    const double *S0 = ckpt + (int64_t)h * P * N;
    for (int i = 0; i < n_in; ++i) {
      const int m = n_log + i;
      memcpy(w, q_all + ((int64_t)m * G + g) * N, sizeof(double) * N);
      for (int j = m; j >= 0; --j) {
        const double *kj = k_all + ((int64_t)j * G + g) * N;
        const double alpha = exp(dt_all[(int64_t)j * H + h] * A[h]);
        double kw = 0.0;
        for (int n = 0; n < N; ++n) kw += kj[n] * w[n];
        c[j] = beta_all[(int64_t)j * H + h] * kw;
        for (int n = 0; n < N; ++n) w[n] = alpha * (w[n] - c[j] * kj[n]);
      }
      for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int n = 0; n < N; ++n) acc += S0[(int64_t)p * N + n] * w[n];
        for (int j = 0; j <= m; ++j) acc += c[j] * v_all[((int64_t)j * H + h) * P + p];
        o[((int64_t)i * H + h) * P + p] = acc;
      }
    }
    if (fold_out) {
      double *F = fold_out + (int64_t)h * P * N;
      memset(F, 0, sizeof(double) * P * N);
      for (int a = 0; a < N; ++a)
        for (int b = 0; b < N; ++b) T[a * N + b] = a == b ? 1.0 : 0.0;
      for (int j = n_log - 1; j >= 0; --j) {
        const double *kj = k_all + ((int64_t)j * G + g) * N;
        const double alpha = exp(dt_all[(int64_t)j * H + h] * A[h]);
        const double beta = beta_all[(int64_t)j * H + h];
        /* the entry's own term: beta_j v_j (k_j^T T) */
        for (int b = 0; b < N; ++b) {
          double acc = 0.0;
          for (int a = 0; a < N; ++a) acc += kj[a] * T[a * N + b];
          r[b] = acc;
        }
        for (int p = 0; p < P; ++p)
          for (int b = 0; b < N; ++b)
            F[(int64_t)p * N + b] += beta * v_all[((int64_t)j * H + h) * P + p] * r[b];
        /* T <- A_j T = alpha_j (T - beta_j k_j (k_j^T T)) */
        for (int a = 0; a < N; ++a)
          for (int b = 0; b < N; ++b) T2[a * N + b] = alpha * (T[a * N + b] - beta * kj[a] * r[b]);
        memcpy(T, T2, sizeof(double) * N * N);
      }
      for (int p = 0; p < P; ++p)
        for (int b = 0; b < N; ++b) {
          double acc = 0.0;
          for (int a = 0; a < N; ++a) acc += S0[(int64_t)p * N + a] * T[a * N + b];
          F[(int64_t)p * N + b] += acc;
        }
    }
  }
  free(w);
  free(c);
  free(T);
  free(T2);
  free(r);
  return ORC_OK;
}
