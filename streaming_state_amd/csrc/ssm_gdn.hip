// ssm_gdn.hip -- verify kernels of the Gated DeltaNet recurrence: ReplaySSM
// (checkpoint plus a log of per-token inputs) and the copy-state-per-draft
// baseline it replaces.
//
// The recurrence, per value head h with key group g (the gated delta rule):
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
//   alpha_t = exp(dt_t A_h),
// with S [P value rows, N key columns] fp32 in the same [S, H, P, N] layout as
// the Mamba-2 state (x carries v, B carries k, C carries q).  The pages list it
// among the recurrences whose update unrolls into a decay plus a sum, so that
// a checkpoint and a log of per-token inputs can stand in for per-draft state
// copies ("Why Speculative Decoding Slows Hybrid Mamba Models at Large Batch
// Sizes", section "When Replaying the Inputs Is the Wrong Tool"); they do not
// write the update out, and the published gated delta rule is used.
//
// Unrolled over the entries 1..m after the checkpoint S_0, with the rank-1
// factors A_j = alpha_j (I - beta_j k_j k_j^T):
//   o_m = S_0 (A_1 ... A_m q_m) + sum_j beta_j v_j k_j^T (A_{j+1} ... A_m q_m).
// Carrying the query backwards through the factors (w <- q_m; for j = m..1:
// c_j = beta_j (k_j . w), w <- alpha_j (w - c_j k_j)) turns an output into one
// read of the checkpoint at u_m = w plus sum_j c_j v_j.  The checkpoint is read
// once for all in-flight tokens and written only when the log is full and is
// folded in (the state stepped through the committed entries).  Where Mamba-2
// needs scalar decay weights, this needs one length-N vector per in-flight
// token, computed per (slot, head) from the log in LDS.
#include "ssm_device.h"

namespace ssm {
namespace {

__device__ __forceinline__ float4 gz4() { return make_float4(0.f, 0.f, 0.f, 0.f); }
__device__ __forceinline__ float tofl(float v) { return v; }
__device__ __forceinline__ float tofl(bf16_t v) { return bf16_to_f(v); }

// Entry j of half `half` of slot `slot` (the Mamba-2 verify kernels' layout).
struct GdnLogIdx {
  int W;
  __device__ __forceinline__ size_t ent(int slot, int half, int j) const {
    return ((size_t)slot * 2 + half) * W + j;
  }
};

// ===========================================================================
// copy-per-draft baseline: read once, then per token update, write a copy,
// emit the output
// ===========================================================================
constexpr int kGdnCopyR = 4;

template <typename T, int R>
__global__ __launch_bounds__(kThreads) void gdn_copy_kernel(CopyArgs a, CopyMeta m) {
  const TileR<R> tl;
  const Dims d = a.d;
  constexpr int kTileRows = 8 * R;
  const int pt_n = (d.P + kTileRows - 1) / kTileRows;
  int bid = blockIdx.x;
  const int pt = bid % pt_n;
  bid /= pt_n;
  const int h = bid % d.H;
  const int e = bid / d.H;
  const int slot = m.slot[e];
  const int src = m.src[e];
  const int g = h / (d.H / d.G);
  const int prow0 = pt * kTileRows;
  const bool colok = 4 * tl.c < d.N;
  const size_t PN = (size_t)d.P * d.N;
  const size_t tile_off = (size_t)prow0 * d.N + 4 * tl.c;
  const float *in = (src < 0 ? a.state + ((size_t)slot * d.H + h) * PN
                             : a.copies + (((size_t)slot * a.n_in_max + src) * d.H + h) * PN) +
                    tile_off;
  float4 hv[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const bool ok = colok && (prow0 + tl.row(i) < d.P);
    hv[i] = ok ? nt_load4(in + (size_t)tl.row(i) * d.N) : gz4();
  }
  const float Ah = a.A[h];
  for (int k = 0; k < a.n_in; ++k) {
    const size_t ek = (size_t)e * a.n_in + k;
    const T *v = (const T *)a.x + (ek * d.H + h) * d.P + prow0;
    const float al = expf(Io<T>::ld((const T *)a.dt + ek * d.H + h) * Ah);
    const float be = Io<T>::ld((const T *)a.beta + ek * d.H + h);
    float4 kv = gz4(), qv = gz4();
    if (colok) {
      kv = Io<T>::ld4((const T *)a.B + (ek * d.G + g) * d.N + 4 * tl.c);
      qv = Io<T>::ld4((const T *)a.C + (ek * d.G + g) * d.N + 4 * tl.c);
    }
    float *out = a.copies + (((size_t)slot * a.n_in_max + k) * d.H + h) * PN + tile_off;
    float rd[R];
#pragma unroll
    for (int i = 0; i < R; ++i) rd[i] = allsum32(dot4(hv[i], kv));  // (S k)[row]
    float part[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const bool rowok = prow0 + tl.row(i) < d.P;
      const float vv = rowok ? Io<T>::ld(v + tl.row(i)) : 0.f;
      hv[i] = fma4(al, hv[i], be * (vv - al * rd[i]), kv);
      if (rowok && colok) nt_store4(out + (size_t)tl.row(i) * d.N, hv[i]);
      part[i] = dot4(hv[i], qv);
    }
    const float yv = row_totals<R>(part, tl.lane);
    const int r = tl.reduced_row();
    if (tl.reduced_writer() && prow0 + r < d.P)
      Io<T>::st((T *)a.y + (ek * d.H + h) * d.P + prow0 + r, yv);
  }
}

// ===========================================================================
// ReplaySSM verify
// ===========================================================================
constexpr int kGdnR = 8;  // float4 per lane: two state rows of four 16-byte chunks

// LDS carve-up (byte offsets; W window, n_in in-flight tokens, xs the LDS stride
// of an entry's v rows, rows the tile's row count, es the io element size).
// A step folds F <= W entries and starts its live half empty (J = n_in), or
// folds none (J <= W), so key rows never exceed W + 2 n_in and v rows W + n_in.
//   K [W + 2 n_in][N] io   fold k rows, then combined k rows, then in-flight q
//   x [W + n_in][xs] io    combined v rows, then fold v rows
//   alpha, beta [W] (combined), fla = log2(alpha), fbeta [W] (fold), coef [W][n_in],
//   u [n_in][N], dot [n_in][rows]   (fp32)
struct GdnSmem {
  int K, x, alpha, beta, fla, fbeta, coef, u, dot, total;
  __host__ __device__ GdnSmem(int W, int n_in, int N, int xs, int rows, int es) {
    auto up16 = [](int b) { return (b + 15) & ~15; };
    K = 0;
    x = up16(K + (W + 2 * n_in) * N * es);
    alpha = up16(x + (W + n_in) * xs * es);
    beta = alpha + 4 * W;
    fla = beta + 4 * W;
    fbeta = fla + 4 * W;
    coef = fbeta + 4 * W;
    u = up16(coef + 4 * W * n_in);
    dot = u + 4 * n_in * N;
    total = dot + 4 * n_in * rows;
  }
};

// One (batch entry, head, 16 kWaves-row tile) per workgroup of kWaves waves:
// eight waves (128 rows, a whole P = 128 head) share one query sweep and one
// copy of the key rows per head; four serve heads of fewer rows.  The state
// tile lives in registers in the Mamba-2 verify kernel's layout (ReplayTile:
// two rows of four 16-byte chunks per lane, eight lanes per row).  kFull: P a
// multiple of the tile height and N = 128 (no per-lane predicates); eight
// waves per SIMD for it on 128-row tiles (64 registers: the fp32 fold spills
// one, measured faster than six waves without the spill), six on 64-row
// tiles, four for the instantiations that carry the predicates.
template <typename T, int R, bool kFull, int kWaves>
__global__ __launch_bounds__(64 * kWaves, kFull ? (kWaves == 8 ? 8 : 6) : 4) void gdn_replay_kernel(ReplayArgs a,
                                                                               ReplayMeta m,
                                                                               LogLayout lay) {
  extern __shared__ float4 gd_smem4[];
  char *sb = reinterpret_cast<char *>(gd_smem4);
  static_assert(R == 8, "two rows of four 16-byte chunks per lane");
  static_assert(kWaves == 4 || kWaves == 8, "64- or 128-row tiles");
  const ReplayTile tl;
  constexpr int kRows = 16 * kWaves;
  constexpr int kNT = 64 * kWaves;  // threads
  constexpr int E = 16 / (int)sizeof(T);  // io elements per 16-byte chunk
  constexpr int es = (int)sizeof(T);
  const Dims d = a.d;
  const int W = a.W, n_in = a.n_in;
  const int N = kFull ? 4 * 32 : d.N;
  const int pt = blockIdx.x, e = blockIdx.z;
  // Two value heads per key group (H a multiple of 16): the heads of group g
  // are placed eight workgroup slots apart, so that the round-robin dispatch
  // over the eight XCDs puts both on one XCD and the second one's key rows are
  // hits in that XCD's L2.  Otherwise heads in order.
  const int h = (d.H == 2 * d.G && d.H % 16 == 0)
                    ? (blockIdx.y & ~15) + 2 * (blockIdx.y & 7) + ((blockIdx.y >> 3) & 1)
                    : (int)blockIdx.y;
  const int slot = m.slot[e];
  const uint32_t info = m.info[e];
  const int F = info_fold(info);
  const int base = info_base(info);
  const int rh = info_fold_half(info), wh = info_live_half(info);
  const int J = base + n_in;
  const int hpg = d.H / d.G;
  const int g = d.G == 1 ? 0 : h / hpg;
  const int prow0 = pt * kRows;
  const int rv = kFull ? kRows : min(kRows, d.P - prow0);
  const bool whole_chunks = (d.P * es) % 16 == 0 && (N * es) % 16 == 0 &&
                            (((uintptr_t)a.x | (uintptr_t)a.B | (uintptr_t)a.C) & 15) == 0;
  const int xs = whole_chunks ? rv : (rv + 7) & ~7;
  auto colok = [&](int q) { return kFull || tl.col(q) < N; };
  const size_t PN = (size_t)d.P * N;
  const float Ah = a.A[h];
  const float Ah2 = Ah * 1.4426950408889634f;  // A in log2 units
  const GdnLogIdx li{W};
  T *logdt = (T *)((char *)a.log + lay.dt_off);
  T *logbeta = (T *)((char *)a.log + lay.beta_off);
  T *logx = (T *)((char *)a.log + lay.x_off);
  T *logk = (T *)((char *)a.log + lay.B_off);
  const T *inx = (const T *)a.x, *indt = (const T *)a.dt, *inbeta = (const T *)a.beta;
  const T *ink = (const T *)a.B, *inq = (const T *)a.C;
  const GdnSmem L(W, n_in, N, xs, rv, es);
  T *s_K = (T *)(sb + L.K);
  T *s_x = (T *)(sb + L.x);
  float *s_alpha = (float *)(sb + L.alpha), *s_beta = (float *)(sb + L.beta);
  float *s_fla = (float *)(sb + L.fla), *s_fbeta = (float *)(sb + L.fbeta);
  float *s_coef = (float *)(sb + L.coef), *s_u = (float *)(sb + L.u);
  float *s_dot = (float *)(sb + L.dot);

  // Row sources, each a run at a fixed stride (consecutive log entries of a
  // slot and half are consecutive in the log).
  const size_t xstride = (size_t)d.H * d.P, kstride = (size_t)d.G * N;
  const T *x_com = logx + (li.ent(slot, wh, 0) * d.H + h) * d.P + prow0;
  const T *x_new = inx + ((size_t)e * n_in * d.H + h) * d.P + prow0;
  const T *x_fold = logx + (li.ent(slot, rh, 0) * d.H + h) * d.P + prow0;
  const T *k_fold = logk + li.ent(slot, rh, 0) * kstride + (size_t)g * N;
  const T *k_com = logk + li.ent(slot, wh, 0) * kstride + (size_t)g * N;
  const T *k_new = ink + (size_t)e * n_in * kstride + (size_t)g * N;
  const T *q_new = inq + (size_t)e * n_in * kstride + (size_t)g * N;
  if (whole_chunks) {
    const int cx = rv / E, cv = N / E;
    const FastDiv fx(cx), fv(cv);
    auto run = [&](char *lds, const T *src, size_t stride, int rows, int chunks, FastDiv f) {
      stage_lds<kWaves>(lds, rows * chunks, [&](int i) {
        const int j = f.div(i);
        return (const void *)(src + j * stride + (i - j * chunks) * E);
      });
    };
    run(sb + L.x, x_com, xstride, base, cx, fx);
    run(sb + L.x + base * xs * es, x_new, xstride, n_in, cx, fx);
    run(sb + L.x + J * xs * es, x_fold, xstride, F, cx, fx);
    run(sb + L.K, k_fold, kstride, F, cv, fv);
    run(sb + L.K + F * N * es, k_com, kstride, base, cv, fv);
    run(sb + L.K + (F + base) * N * es, k_new, kstride, n_in, cv, fv);
    run(sb + L.K + (F + J) * N * es, q_new, kstride, n_in, cv, fv);
  } else {  // rows not made of aligned 16-byte chunks: element copies
    const FastDiv frv(rv), fn(N);
    for (int i = threadIdx.x; i < (J + F) * rv; i += kNT) {
      const int j = frv.div(i), r = i - j * rv;
      const T *src = j >= J ? x_fold + (j - J) * xstride
                     : j < base ? x_com + j * xstride : x_new + (j - base) * xstride;
      s_x[j * xs + r] = src[r];
    }
    for (int i = threadIdx.x; i < (F + J + n_in) * N; i += kNT) {
      const int r = fn.div(i), col = i - r * N;
      const T *src = r < F ? k_fold + r * kstride
                     : r < F + base ? k_com + (r - F) * kstride
                     : r < F + J ? k_new + (r - F - base) * kstride
                                 : q_new + (r - F - J) * kstride;
      s_K[i] = src[col];
    }
  }

  // checkpoint tile
  float *st = a.state + ((size_t)slot * d.H + h) * PN + (size_t)prow0 * N;
  float4 hv[R];  // hv[4 i + q]: row(i), chunk q
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = colok(q) && (kFull || tl.row(i) < rv);
      hv[4 * i + q] = ok ? nt_load4(st + (size_t)tl.row(i) * N + tl.col(q)) : gz4();
    }

  // gates: combined entries (committed, then in-flight) and fold entries
  const T *dt_com = logdt + li.ent(slot, wh, 0) * d.H + h;
  const T *dt_new = indt + (size_t)e * n_in * d.H + h;
  const T *dt_fold = logdt + li.ent(slot, rh, 0) * d.H + h;
  const T *be_com = logbeta + li.ent(slot, wh, 0) * d.H + h;
  const T *be_new = inbeta + (size_t)e * n_in * d.H + h;
  const T *be_fold = logbeta + li.ent(slot, rh, 0) * d.H + h;
  for (int i = threadIdx.x; i < J + F; i += kNT) {
    if (i < J) {
      const bool com = i < base;
      const size_t o = (size_t)(com ? i : i - base) * d.H;
      s_alpha[i] = expf(Ah * tofl(com ? dt_com[o] : dt_new[o]));
      s_beta[i] = tofl(com ? be_com[o] : be_new[o]);
    } else {
      const size_t o = (size_t)(i - J) * d.H;
      s_fla[i - J] = Ah2 * tofl(dt_fold[o]);
      s_fbeta[i - J] = tofl(be_fold[o]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the LDS copies above have landed
  __syncthreads();

  // append the in-flight v (this tile), dt and beta (per head) and k (per
  // group, by its first head) to the live log half
  {
    const FastDiv frows(rv);
    T *x_app = logx + (li.ent(slot, wh, base) * d.H + h) * d.P + prow0;
    for (int i = threadIdx.x; i < n_in * rv; i += kNT) {
      const int k = frows.div(i), r = i - k * rv;
      x_app[k * xstride + r] = s_x[(base + k) * xs + r];
    }
    if (pt == 0)
      for (int k = threadIdx.x; k < n_in; k += kNT) {
        const size_t o = li.ent(slot, wh, base + k) * d.H + h;
        logdt[o] = dt_new[(size_t)k * d.H];
        logbeta[o] = be_new[(size_t)k * d.H];
      }
    if (pt == 0 && h % hpg == 0) {
      const FastDiv fn(N);
      for (int i = threadIdx.x; i < n_in * N; i += kNT) {
        const int k = fn.div(i), col = i - k * N;
        logk[li.ent(slot, wh, base + k) * kstride + (size_t)g * N + col] =
            s_K[(F + base + k) * N + col];
      }
    }
  }

  // every in-flight query carried back through the combined entries' factors,
  // newest first: two tokens per wave, one per 32-lane half, a lane holding
  // four consecutive key elements.  The decay stays out of the loop: with the
  // carried query w = rho * wh, the coefficient is c_j = rho beta_j (k_j . wh),
  // then wh <- wh - beta_j (k_j . wh) k_j and rho <- alpha_j rho.
  {
    const int half = tl.lane >> 5, n0 = 4 * (tl.lane & 31);
    const T *s_Kc = s_K + F * N, *s_q = s_K + (F + J) * N;
    auto ld_key4 = [&](const T *row, float v[4]) {
      if (kFull) {
        const float4 t = lds_ld4(row + n0);
        v[0] = t.x;
        v[1] = t.y;
        v[2] = t.z;
        v[3] = t.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = n0 + i < N ? tofl(row[n0 + i]) : 0.f;
      }
    };
    for (int kp = __builtin_amdgcn_readfirstlane(tl.wave); 2 * kp < n_in; kp += kWaves) {
      const int k = 2 * kp + half;
      const bool tok = k < n_in;
      const int mm = base + k;                             // this half's newest entry
      const int jtop = base + min(2 * kp + 1, n_in - 1);  // the wave's newest entry
      float w[4] = {0.f, 0.f, 0.f, 0.f};
      if (tok) ld_key4(s_q + k * N, w);
      float rho = 1.f;
      for (int j = jtop; j >= 0; --j) {
        float kv[4];
        ld_key4(s_Kc + j * N, kv);
        float p = w[0] * kv[0];
        p = fmaf(w[1], kv[1], p);
        p = fmaf(w[2], kv[2], p);
        p = fmaf(w[3], kv[3], p);
        const float sum = allsum32(p);  // every lane takes part in the lane moves
        const bool act = tok && j <= mm;
        const float t = act ? s_beta[j] * sum : 0.f;
        if (act && (tl.lane & 31) == 0) s_coef[j * n_in + k] = rho * t;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = fmaf(-t, kv[i], w[i]);
        rho = act ? rho * s_alpha[j] : rho;
      }
      if (tok)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kFull || n0 + i < N) s_u[k * N + n0 + i] = rho * w[i];
    }
  }

  // fold: step the checkpoint through the committed entries of the full half
  // (S <- alpha S + (beta (v - alpha S k)) k^T per entry) and write it back.
  // The decay is deferred: the registers hold Sh with S = 2^ls Sh, ls the sum
  // of log2(alpha) since the last rescale, so an entry is one multiply-add per
  // element, Sh <- Sh + beta (2^-ls v - Sh k) k^T; Sh is rescaled to S before
  // 2^-ls passes 2^32.
  if (F > 0) {
    const T *fx = s_x + J * xs + tl.row(0);  // this lane's two consecutive rows
    float ls = 0.f;
#pragma unroll 1
    for (int j = 0; j < F; ++j) {
      float4 kq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) kq[q] = colok(q) ? lds_ld4(s_K + j * N + tl.col(q)) : gz4();
      float xv[2];
      lds_ld_pair(fx + j * xs, xv);
      const float be = s_fbeta[j];
      ls += s_fla[j];
      if (!(ls >= -32.f)) {  // uniform: take the decay into the registers
        const float sc = exp2f(ls);
#pragma unroll
        for (int i = 0; i < R; ++i) hv[i] = scale4(hv[i], sc);
        ls = 0.f;
      }
      const float isig = exp2f(-ls);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // (Sh k)[row]: this lane's 16 columns, then the row's eight lanes
        float acc = hv[4 * i].x * kq[0].x;
        acc = fmaf(hv[4 * i].y, kq[0].y, acc);
        acc = fmaf(hv[4 * i].z, kq[0].z, acc);
        acc = fmaf(hv[4 * i].w, kq[0].w, acc);
#pragma unroll
        for (int q = 1; q < 4; ++q) {
          acc = fmaf(hv[4 * i + q].x, kq[q].x, acc);
          acc = fmaf(hv[4 * i + q].y, kq[q].y, acc);
          acc = fmaf(hv[4 * i + q].z, kq[q].z, acc);
          acc = fmaf(hv[4 * i + q].w, kq[q].w, acc);
        }
        const float rd = ReplayTile::row_sum(acc);
        const float vv = (kFull || tl.row(i) < rv) ? xv[i] : 0.f;
        const float u = be * fmaf(vv, isig, -rd);
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[4 * i + q] = fma4(1.f, hv[4 * i + q], u, kq[q]);
      }
    }
    if (ls != 0.f) {
      const float sc = exp2f(ls);
#pragma unroll
      for (int i = 0; i < R; ++i) hv[i] = scale4(hv[i], sc);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (colok(q) && (kFull || tl.row(i) < rv))
          nt_store4(st + (size_t)tl.row(i) * N + tl.col(q), hv[4 * i + q]);
  }
  __syncthreads();  // u and coef are complete

  // checkpoint read-out at every carried-back query
  for (int k = 0; k < n_in; ++k) {
    float part[2];  // one multiply-add chain per row over the lane's 16 columns
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 Uv =
          colok(q) ? *reinterpret_cast<const float4 *>(s_u + k * N + tl.col(q)) : gz4();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float4 hq = hv[4 * i + q];
        float acc = q == 0 ? hq.x * Uv.x : fmaf(hq.x, Uv.x, part[i]);
        acc = fmaf(hq.y, Uv.y, acc);
        acc = fmaf(hq.z, Uv.z, acc);
        part[i] = fmaf(hq.w, Uv.w, acc);
      }
    }
    const float v = tl.totals(part[0], part[1]);
    if (tl.reduced_writer() && (kFull || tl.reduced_row() < rv)) s_dot[k * rv + tl.reduced_row()] = v;
  }
  __syncthreads();

  // outputs: one wave per (in-flight token, 64 rows of the tile), lane = row
  constexpr int kParts = kRows / 64;
  for (int jb = __builtin_amdgcn_readfirstlane(tl.wave); jb < n_in * kParts; jb += kWaves) {
    const int k = jb / kParts, r = (jb % kParts) * 64 + tl.lane;
    if (r < rv) {
      const int mm = base + k;
      float acc = s_dot[k * rv + r];
#pragma unroll 4
      for (int j = 0; j <= mm; ++j) acc += s_coef[j * n_in + k] * tofl(s_x[j * xs + r]);
      Io<T>::st((T *)a.y + (((size_t)e * n_in + k) * d.H + h) * d.P + prow0 + r, acc);
    }
  }
}

}  // namespace

hipError_t launch_gdn_copy(int io, const CopyArgs &a, const CopyMeta &m, hipStream_t s) {
  const int pt_n = (a.d.P + 8 * kGdnCopyR - 1) / (8 * kGdnCopyR);
  dim3 grid(a.n * a.d.H * pt_n), block(kThreads);
  if (io == kBF16)
    hipLaunchKernelGGL((gdn_copy_kernel<bf16_t, kGdnCopyR>), grid, block, 0, s, a, m);
  else
    hipLaunchKernelGGL((gdn_copy_kernel<float, kGdnCopyR>), grid, block, 0, s, a, m);
  return hipGetLastError();
}

hipError_t launch_gdn_replay(int io, const ReplayArgs &a, const ReplayMeta &m,
                             const LogLayout &lay, hipStream_t s) {
  // 128-row tiles (eight waves) once a head has that many rows, else 64
  const bool wide = a.d.P >= 128;
  const int rows = wide ? 128 : 64;
  const int pt_n = (a.d.P + rows - 1) / rows;
  dim3 grid(pt_n, a.d.H, a.n), block(wide ? 512 : 256);
  // xs and the row count are at most the tile height: this bounds every tile
  const size_t sm = (size_t)GdnSmem(a.W, a.n_in, a.d.N, rows, rows, io == kBF16 ? 2 : 4).total;
  const bool full = a.d.P % rows == 0 && a.d.N == 4 * 32;
  auto go = [&](auto kernel) {
    hipError_t err = allow_dynamic_lds(reinterpret_cast<const void *>(kernel), sm);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kernel, grid, block, sm, s, a, m, lay);
    return hipGetLastError();
  };
  auto pick = [&](auto tag) {
    using T = decltype(tag);
    if (wide)
      return full ? go(gdn_replay_kernel<T, kGdnR, true, 8>)
                  : go(gdn_replay_kernel<T, kGdnR, false, 8>);
    return full ? go(gdn_replay_kernel<T, kGdnR, true, 4>)
                : go(gdn_replay_kernel<T, kGdnR, false, 4>);
  };
  return io == kBF16 ? pick(bf16_t{}) : pick(float{});
}

}  // namespace ssm
