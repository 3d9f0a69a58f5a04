/*
 * ssm_oracle.c -- plain, slow, sequential fp64 CPU oracle for the Mamba-2
 * streaming-state recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.  "parity pinned": every function below is checked against the
 * pages and closed forms by the CPU test suite (see tests/test_oracle_*.py).
 *
 * What it computes (the plain definition, in this order, per head h and
 * group g = h / (H/G)):
 *
 *     a_t   = exp(dt_t[h] * A[h])                     decay of the old state
 *     s    <- a_t * s + dt_t[h] * x_t[h,:] (outer) B_t[g,:]
 *     y_t[h,p] = sum_n s[p,n] * C_t[g,n]  +  D[h] * x_t[h,p]
 *
 * This is the Mamba-2 selective-scan recurrence (each token scales the old
 * state by its decay and adds its own term: "Why Speculative Decoding Slows
 * Hybrid Mamba Models at Large Batch Sizes", section "The Fix: Log the Inputs,
 * Checkpoint the State"; the SSD dual view is named in "Mamba Streaming State
 * That Survives Chunking", section "Separate Mamba-2 algebra from kernel
 * behavior").  The output uses the post-update state.  A reset flag on token
 * t zeroes the state and the position before token t is applied ("Runnable
 * artifact" of the same page: resetBefore restores the initial state).
 *
 * Everything is fp64; inputs arrive already widened (exactly) from fp32 or
 * bf16.  Sums over n run in increasing n.  Compile with -ffp-contract=off so
 * the operation order is exactly the one written here, which makes a chunked
 * scan bit-identical to the full scan (section "Let the full scan define
 * legal chunking": a scalar CPU check may insist on exact equality).
 *
 * Threads only split independent (head) or (slot, head) units; each unit is a
 * strictly sequential loop over tokens, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_INVALID_CHUNK (-2) /* a non-finite input: nothing is changed */

/* ------------------------------------------------------------------------ */
/* a tiny parallel-for over independent units                               */
/* ------------------------------------------------------------------------ */
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

/* One token of the recurrence for one head: s[P,N] is updated in place and
 * y[P] receives the output.  decay is a_t (already exp(dt*A) or injected). */
static void step_head(int P, int N, double decay, double dt, const double *x /*[P]*/,
                      const double *Bg /*[N]*/, const double *Cg /*[N]*/, double Dh,
                      double *s /*[P,N]*/, double *y /*[P]*/) {
  for (int p = 0; p < P; ++p) {
    double u = dt * x[p];
    double *row = s + (int64_t)p * N;
    for (int n = 0; n < N; ++n) row[n] = decay * row[n] + u * Bg[n];
    double acc = 0.0;
    for (int n = 0; n < N; ++n) acc += row[n] * Cg[n];
    y[p] = acc + Dh * x[p];
  }
}

/* ------------------------------------------------------------------------ */
/* chunk scan: one stream, L tokens, optional per-token reset, checkpoints  */
/* ------------------------------------------------------------------------ */
typedef struct {
  int H, P, N, G;
  int64_t L;
  const double *x, *dt, *B, *C, *A, *D, *decay;
  const uint8_t *reset;
  double *state, *y;
  int n_ckpt;
  const int64_t *ckpt_at;
  double *ckpt_out;
} scan_ctx;

static void scan_unit(void *vctx, int64_t h) {
  scan_ctx *c = (scan_ctx *)vctx;
  const int H = c->H, P = c->P, N = c->N, G = c->G;
  const int g = (int)(h / (H / G));
  const int64_t PN = (int64_t)P * N;
  double *s = c->state + h * PN;
  int next_ck = 0;
  for (int64_t t = 0; t < c->L; ++t) {
    if (c->reset && c->reset[t]) memset(s, 0, sizeof(double) * PN);
    double dt = c->dt[t * H + h];
    double decay = c->decay ? c->decay[t * H + h] : exp(dt * c->A[h]);
    step_head(P, N, decay, dt, c->x + (t * H + h) * P, c->B + (t * G + g) * N,
              c->C + (t * G + g) * N, c->D[h], s, c->y + (t * H + h) * P);
    while (next_ck < c->n_ckpt && c->ckpt_at[next_ck] == t) {
      memcpy(c->ckpt_out + ((int64_t)next_ck * H + h) * PN, s, sizeof(double) * PN);
      ++next_ck;
    }
  }
}

/*
 * oracle_scan: advance one stream by L tokens.
 *   x[L,H,P] dt[L,H] B[L,G,N] C[L,G,N] A[H] D[H]    inputs (fp64)
 *   decay[L,H] or NULL      test-only: use a_t = decay[t,h] instead of exp(dt*A)
 *   reset[L] or NULL        reset before token t (state and position to 0)
 *   state[H,P,N]            carry-in on entry, carry-out on return
 *   pos                     position on entry / return (tokens since reset)
 *   y[L,H,P]                outputs
 *   ckpt_at[n_ckpt]         strictly increasing token indices; the state right
 *                           after token ckpt_at[i] is copied to ckpt_out[i,H,P,N]
 * Returns ORC_E_INVALID_CHUNK, with nothing written, if any input is not finite
 * (the artifact's "invalid_chunk").  L == 0 is legal and changes nothing.
 */
int oracle_scan(int H, int P, int N, int G, int64_t L, const double *x, const double *dt,
                const double *B, const double *C, const double *A, const double *D,
                const double *decay, const uint8_t *reset, double *state, int64_t *pos,
                double *y, int n_ckpt, const int64_t *ckpt_at, double *ckpt_out,
                int n_threads) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || L < 0 || n_ckpt < 0)
    return ORC_E_ARG;
  for (int i = 0; i < n_ckpt; ++i) {
    if (ckpt_at[i] < 0 || ckpt_at[i] >= L) return ORC_E_ARG;
    if (i > 0 && ckpt_at[i] <= ckpt_at[i - 1]) return ORC_E_ARG;
  }
  if (!all_finite(x, L * H * P) || !all_finite(dt, L * H) || !all_finite(B, L * G * N) ||
      !all_finite(C, L * G * N))
    return ORC_E_INVALID_CHUNK;
  if (decay && !all_finite(decay, L * H)) return ORC_E_INVALID_CHUNK;
  scan_ctx c = {H, P, N, G, L, x, dt, B, C, A, D, decay, reset, state, y, n_ckpt, ckpt_at,
                ckpt_out};
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
/* batched decode: one token for each of `batch` slots                      */
/* ------------------------------------------------------------------------ */
typedef struct {
  int H, P, N, G, batch;
  const int32_t *slot;
  const double *x, *dt, *B, *C, *A, *D;
  const uint8_t *reset;
  double *state, *y;
} dec_ctx;

static void dec_unit(void *vctx, int64_t u) {
  dec_ctx *c = (dec_ctx *)vctx;
  const int H = c->H, P = c->P, N = c->N, G = c->G;
  const int64_t b = u / H, h = u % H;
  const int g = (int)(h / (H / G));
  const int64_t PN = (int64_t)P * N;
  double *s = c->state + ((int64_t)c->slot[b] * H + h) * PN;
  if (c->reset && c->reset[b]) memset(s, 0, sizeof(double) * PN);
  double dt = c->dt[b * H + h];
  step_head(P, N, exp(dt * c->A[h]), dt, c->x + (b * H + h) * P, c->B + (b * G + g) * N,
            c->C + (b * G + g) * N, c->D[h], s, c->y + (b * H + h) * P);
}

/*
 * oracle_decode: one token per slot (decode moves many streams forward by a
 * token each: section "Separate Mamba-2 algebra from kernel behavior").
 *   slot[batch] distinct slot indices into state[S,H,P,N] and pos[S]
 *   x[batch,H,P] dt[batch,H] B,C[batch,G,N]; reset[batch] or NULL
 *   y[batch,H,P]
 */
int oracle_decode(int S, int H, int P, int N, int G, int batch, const int32_t *slot,
                  const double *x, const double *dt, const double *B, const double *C,
                  const double *A, const double *D, const uint8_t *reset, double *state,
                  int64_t *pos, double *y, int n_threads) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || batch < 0) return ORC_E_ARG;
  for (int b = 0; b < batch; ++b) {
    if (slot[b] < 0 || slot[b] >= S) return ORC_E_ARG;
    for (int b2 = 0; b2 < b; ++b2)
      if (slot[b2] == slot[b]) return ORC_E_ARG;
  }
  if (!all_finite(x, (int64_t)batch * H * P) || !all_finite(dt, (int64_t)batch * H) ||
      !all_finite(B, (int64_t)batch * G * N) || !all_finite(C, (int64_t)batch * G * N))
    return ORC_E_INVALID_CHUNK;
  dec_ctx c = {H, P, N, G, batch, slot, x, dt, B, C, A, D, reset, state, y};
  parallel_for(dec_unit, &c, (int64_t)batch * H, n_threads);
  for (int b = 0; b < batch; ++b) {
    if (reset && reset[b]) pos[slot[b]] = 0;
    pos[slot[b]] += 1;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* speculative verify with rollback: the step-by-step recurrence            */
/* ------------------------------------------------------------------------ */
typedef struct {
  int H, P, N, G, batch, n_in;
  const int32_t *slot, *accepted;
  const double *x, *dt, *B, *C, *A, *D;
  double *state, *y;
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
  for (int k = 0; k < n_in; ++k) {
    int64_t bk = b * n_in + k;
    double dt = c->dt[bk * H + h];
    step_head(P, N, exp(dt * c->A[h]), dt, c->x + (bk * H + h) * P, c->B + (bk * G + g) * N,
              c->C + (bk * G + g) * N, c->D[h], work, c->y + (bk * H + h) * P);
    if (k == a - 1) memcpy(kept, work, sizeof(double) * PN);
  }
  memcpy(s, kept, sizeof(double) * PN);
  free(work);
  free(kept);
}

/*
 * oracle_spec_step: verify n_in in-flight tokens per slot (the real token plus
 * drafts) with the plain recurrence, emit every token's output, then keep the
 * state after the first accepted[b] tokens and drop the rest ("Why Speculative
 * Decoding Slows ...", sections "The Problem" and "The Fix": rejected drafts
 * never reach the state).  1 <= accepted[b] <= n_in.
 *   x[batch,n_in,H,P] dt[batch,n_in,H] B,C[batch,n_in,G,N] y[batch,n_in,H,P]
 */
int oracle_spec_step(int S, int H, int P, int N, int G, int batch, const int32_t *slot,
                     int n_in, const double *x, const double *dt, const double *B,
                     const double *C, const double *A, const double *D,
                     const int32_t *accepted, double *state, int64_t *pos, double *y,
                     int n_threads) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || batch < 0 || n_in < 1)
    return ORC_E_ARG;
  for (int b = 0; b < batch; ++b) {
    if (slot[b] < 0 || slot[b] >= S) return ORC_E_ARG;
    if (accepted[b] < 1 || accepted[b] > n_in) return ORC_E_ARG;
    for (int b2 = 0; b2 < b; ++b2)
      if (slot[b2] == slot[b]) return ORC_E_ARG;
  }
  int64_t nt = (int64_t)batch * n_in;
  if (!all_finite(x, nt * H * P) || !all_finite(dt, nt * H) || !all_finite(B, nt * G * N) ||
      !all_finite(C, nt * G * N))
    return ORC_E_INVALID_CHUNK;
  spec_ctx c = {H, P, N, G, batch, n_in, slot, accepted, x, dt, B, C, A, D, state, y};
  parallel_for(spec_unit, &c, (int64_t)batch * H, n_threads);
  for (int b = 0; b < batch; ++b) pos[slot[b]] += accepted[b];
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* test-only: the replay form written out (checkpoint + logged inputs)       */
/* ------------------------------------------------------------------------ */
/*
 * oracle_replay_unrolled: outputs and folded state computed from a checkpoint
 * and a log of per-token inputs without stepping the state: the output is the
 * decayed checkpoint's read-out plus every logged token's term, each decayed
 * by the tokens that followed it (section "The Fix: Log the Inputs, Checkpoint
 * the State").  Used by the tests
 * to pin the recurrence against the rearranged form; one head group, one slot.
 *
 * Entries 0..n_log-1 are the committed log, entries n_log..n_log+n_in-1 the
 * in-flight tokens.  For an in-flight token at combined index m:
 *   y_m[h,p] = exp(A_h * sum_{i<=m} dt_i) * sum_n ckpt[h,p,n] C_m[n]
 *            + sum_{j<=m} exp(A_h * sum_{j<i<=m} dt_i) * dt_j * x_j[h,p] * (B_j . C_m)
 *            + D_h x_m[h,p]
 * fold_out[h,p,n] = state after the n_log committed entries:
 *   exp(A_h sum_{i<n_log} dt_i) ckpt + sum_{j<n_log} exp(A_h sum_{j<i<n_log} dt_i) dt_j x_j B_j
 *   dt_all[n_log+n_in,H] x_all[n_log+n_in,H,P] B_all,C_all[n_log+n_in,G,N]
 *   (C_all rows for log entries are unused)
 */
int oracle_replay_unrolled(int H, int P, int N, int G, int n_log, int n_in,
                           const double *ckpt, const double *dt_all, const double *x_all,
                           const double *B_all, const double *C_all, const double *A,
                           const double *D, double *y /*[n_in,H,P]*/,
                           double *fold_out /*[H,P,N] or NULL*/) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || n_log < 0 || n_in < 0)
    return ORC_E_ARG;
  for (int h = 0; h < H; ++h) {
    const int g = h / (H / G);
    for (int k = 0; k < n_in; ++k) {
      const int m = n_log + k;
      const double *Cm = C_all + ((int64_t)m * G + g) * N;
      double total = 0.0;
      for (int i = 0; i <= m; ++i) total += dt_all[(int64_t)i * H + h];
      double lam = exp(A[h] * total);
      for (int p = 0; p < P; ++p) {
        const double *row = ckpt + ((int64_t)h * P + p) * N;
        double dotc = 0.0;
        for (int n = 0; n < N; ++n) dotc += row[n] * Cm[n];
        double acc = lam * dotc;
        for (int j = 0; j <= m; ++j) {
          double suffix = 0.0;
          for (int i = j + 1; i <= m; ++i) suffix += dt_all[(int64_t)i * H + h];
          const double *Bj = B_all + ((int64_t)j * G + g) * N;
          double bc = 0.0;
          for (int n = 0; n < N; ++n) bc += Bj[n] * Cm[n];
          acc += exp(A[h] * suffix) * dt_all[(int64_t)j * H + h] *
                 x_all[((int64_t)j * H + h) * P + p] * bc;
        }
        y[((int64_t)k * H + h) * P + p] = acc + D[h] * x_all[((int64_t)m * H + h) * P + p];
      }
    }
    if (fold_out) {
      double total = 0.0;
      for (int i = 0; i < n_log; ++i) total += dt_all[(int64_t)i * H + h];
      double lam = exp(A[h] * total);
      for (int p = 0; p < P; ++p)
        for (int n = 0; n < N; ++n) {
          double v = lam * ckpt[((int64_t)h * P + p) * N + n];
          for (int j = 0; j < n_log; ++j) {
            double suffix = 0.0;
            for (int i = j + 1; i < n_log; ++i) suffix += dt_all[(int64_t)i * H + h];
            v += exp(A[h] * suffix) * dt_all[(int64_t)j * H + h] *
                 x_all[((int64_t)j * H + h) * P + p] * B_all[((int64_t)j * G + g) * N + n];
          }
          fold_out[((int64_t)h * P + p) * N + n] = v;
        }
    }
  }
  return ORC_OK;
}
