// ssm_kernels.hip -- gfx950 kernels of the memory-bound verify paths:
// copy-per-draft verify (baseline), ReplaySSM verify with the fused log fold,
// and the state operations (zero, copy, checksum, finite check).  The batched
// decode kernel is in ssm_decode.hip.
//
// All three verify/decode kernels share one shape: a workgroup of 256 threads
// owns one (batch entry, head, 64-row tile) of the fp32 state, held in
// registers as 8 float4 per thread (Tile in ssm_device.h).  The state is read
// with one pass of 128-bit loads and written (when it is written at all) with
// one pass of 128-bit nontemporal stores; inputs and outputs are small.
#include "ssm_device.h"

namespace ssm {

static __device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }
static __device__ __forceinline__ float to_f(float v) { return v; }
static __device__ __forceinline__ float to_f(bf16_t v) { return bf16_to_f(v); }

// ===========================================================================
// copy-per-draft verify: read once, then per token update, write a full copy,
// and emit the output
// ===========================================================================
constexpr int kCopyR = 4;  // 16 KiB state tiles (see the decode tiles)

template <typename T, int R>
__global__ __launch_bounds__(kThreads) void copy_kernel(CopyArgs a, CopyMeta m) {
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
    hv[i] = ok ? nt_load4(in + (size_t)tl.row(i) * d.N) : zero4();
  }
  const float Ah = a.A[h], Dh = a.D[h];
  for (int k = 0; k < a.n_in; ++k) {
    const size_t ek = (size_t)e * a.n_in + k;
    const T *x = (const T *)a.x + (ek * d.H + h) * d.P + prow0;
    const float dt = Io<T>::ld((const T *)a.dt + ek * d.H + h);
    const float dA = expf(dt * Ah);
    float4 Bv = zero4(), Cv = zero4();
    if (colok) {
      Bv = Io<T>::ld4((const T *)a.B + (ek * d.G + g) * d.N + 4 * tl.c);
      Cv = Io<T>::ld4((const T *)a.C + (ek * d.G + g) * d.N + 4 * tl.c);
    }
    float *out = a.copies + (((size_t)slot * a.n_in_max + k) * d.H + h) * PN + tile_off;
    float part[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const bool rowok = prow0 + tl.row(i) < d.P;
      const float u = rowok ? dt * Io<T>::ld(x + tl.row(i)) : 0.f;
      hv[i] = fma4(dA, hv[i], u, Bv);
      if (rowok && colok) nt_store4(out + (size_t)tl.row(i) * d.N, hv[i]);
      part[i] = dot4(hv[i], Cv);
    }
    const float yv = row_totals<R>(part, tl.lane);
    const int r = tl.reduced_row();
    if (tl.reduced_writer() && prow0 + r < d.P)
      Io<T>::st((T *)a.y + (ek * d.H + h) * d.P + prow0 + r, yv + Dh * Io<T>::ld(x + r));
  }
}

hipError_t launch_copy(int io, const CopyArgs &a, const CopyMeta &m, hipStream_t s) {
  const int pt_n = (a.d.P + 8 * kCopyR - 1) / (8 * kCopyR);
  dim3 grid(a.n * a.d.H * pt_n), block(kThreads);
  if (io == kBF16)
    hipLaunchKernelGGL((copy_kernel<bf16_t, kCopyR>), grid, block, 0, s, a, m);
  else
    hipLaunchKernelGGL((copy_kernel<float, kCopyR>), grid, block, 0, s, a, m);
  return hipGetLastError();
}

// ===========================================================================
// ReplaySSM verify
// ===========================================================================
// Log of one slot: two halves of W entries each.  A fold (flush) reads the
// half that holds the committed entries while the step's in-flight entries
// are appended to the other half, so the two never overlap within a launch.
LogLayout log_layout(int io, const Dims &d, int S, int W, bool gdn) {
  const size_t es = io == kBF16 ? 2 : 4;
  const size_t ent = (size_t)S * 2 * W;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  LogLayout L;
  L.dt_off = 0;
  L.beta_off = up(L.dt_off + ent * d.H * es);
  L.x_off = gdn ? up(L.beta_off + ent * d.H * es) : L.beta_off;  // beta: Gated DeltaNet only
  L.B_off = up(L.x_off + ent * d.H * d.P * es);
  L.bc_off = up(L.B_off + ent * d.G * d.N * es);
  // Mamba-2's B.C scratch: [kBatchPerLaunch][G][kMaxInFlight][bc_stride(W)] fp32
  L.total = L.bc_off + (gdn ? 0 : (size_t)kBatchPerLaunch * d.G * kMaxInFlight * bc_stride(W) * 4);
  return L;
}

// Offsets of entry j of half `half` of slot `slot` (element units).
struct LogIdx {
  int W;
  __device__ __forceinline__ size_t ent(int slot, int half, int j) const {
    return ((size_t)slot * 2 + half) * W + j;
  }
};

// Staging loads of the verify kernels are issued in rounds of kStageU
// values per thread: every load of a round is in flight before the first
// LDS store of that round waits for it.
constexpr int kStageU = 4;

// Pass 1, per (batch entry, group): B_j . C_k for every combined entry j
// (committed log, then in-flight) and in-flight token k; these are shared by
// all heads of a group.  The rows are staged in LDS with one batch of loads
// (row stride N/4 + 1 float4, so rows start on distinct 16-byte slots), and
// the in-flight B rows are appended to the live log half on the way.
template <typename T>
__global__ __launch_bounds__(kThreads) void replay_bc_kernel(ReplayArgs a, ReplayMeta m,
                                                             LogLayout lay) {
  extern __shared__ float4 bc_smem[];
  const Dims d = a.d;
  const int g = blockIdx.x, e = blockIdx.y;
  const int slot = m.slot[e];
  const uint32_t info = m.info[e];
  const int base = info_base(info);
  const int wh = info_live_half(info);
  const int n_in = a.n_in, J = base + n_in;
  const int q = d.N >> 2, qs = q + 1;
  float4 *sB = bc_smem;                    // [J][qs]
  float4 *sC = bc_smem + (size_t)a.W * qs;  // [n_in][qs]
  const LogIdx li{a.W};
  T *logB = (T *)((char *)a.log + lay.B_off);
  const T *inB = (const T *)a.B, *inC = (const T *)a.C;
  const int total = (J + n_in) * q;
  for (int i0 = 0; i0 < total; i0 += kStageU * kThreads) {
    float4 v[kStageU];
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int i = i0 + u * kThreads + (int)threadIdx.x;
      if (i < total) {
        const int row = i / q, cq = i - row * q;
        const T *src = row < base ? logB + (li.ent(slot, wh, row) * d.G + g) * d.N
                       : row < J  ? inB + (((size_t)e * n_in + (row - base)) * d.G + g) * d.N
                                  : inC + (((size_t)e * n_in + (row - J)) * d.G + g) * d.N;
        v[u] = Io<T>::ld4(src + 4 * cq);
      }
    }
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int i = i0 + u * kThreads + (int)threadIdx.x;
      if (i < total) {
        const int row = i / q, cq = i - row * q;
        if (row < J) {
          sB[row * qs + cq] = v[u];
          if (row >= base)
            Io<T>::st4(logB + (li.ent(slot, wh, row) * d.G + g) * d.N + 4 * cq, v[u]);
        } else {
          sC[(row - J) * qs + cq] = v[u];
        }
      }
    }
  }
  __syncthreads();
  const int ws = bc_stride(a.W);
  float *bc = a.bc + ((size_t)e * d.G + g) * kMaxInFlight * ws;
  for (int p = threadIdx.x; p < J * n_in; p += kThreads) {
    const int j = p / n_in, k = p - j * n_in;
    const float4 *bj = sB + j * qs, *ck = sC + k * qs;
    float acc = 0.f;
    for (int t = 0; t < q; ++t) acc += dot4(bj[t], ck[t]);
    bc[k * ws + j] = acc;
  }
}

// Pass 2, per (entry, head, 64-row tile): read the checkpoint once; if the log
// is full, fold it in (ckpt <- Lambda ckpt + sum_j w_j x_j B_j^T) and write the
// checkpoint back -- the only state write; then emit every in-flight token's
// output from the checkpoint and the combined log:
//   y_k = Lambda_m (ckpt . C_k) + sum_{j<=m} w_{j,m} x_j (B_j . C_k) + D x_k,
// m = base + k, Lambda_m = exp(A sum_{i<=m} dt_i),
// w_{j,m} = exp(A sum_{j<i<=m} dt_i) dt_j  (direct suffix sums, at most W terms).
// Everything the tile needs besides the checkpoint (log and in-flight x, the
// fold's B rows, the in-flight C rows) is copied global -> LDS by
// global_load_lds_dwordx4, issued together with the checkpoint's loads: no
// registers hold it on the way, so the kernel keeps eight workgroups per CU,
// and a workgroup waits on global memory once; every later phase touches only
// LDS and registers.
constexpr int kReplayR = 8;  // 64-row (32 KiB) tiles

// LDS carve-up of the verify kernel (byte offsets; W window, n_in in-flight
// tokens, vrows / xrows the rows reserved for the two row regions, xs = the
// LDS stride of an entry's x rows (>= rows), rows = the tile's row count,
// es = io element size, ws = bc_stride(W)):
//   V [vrows][N] io      fold B rows (FR = vrows - n_in at a time), then the
//                        in-flight C rows (n_in)
//   x [xrows][xs] io     combined entries' x (J), then the fold rows' x (FR)
//   coef [n_in][ws]      staged B.C products, then in place the output weights
//   dt [W], fdt [W], lam [n_in], fw [W], flam [1], dot [n_in][rows]   (fp32)
// A step that folds starts its live half empty (J = n_in), one that does not
// folds nothing (F = 0), so xrows = max(W, n_in + FR) covers both.
struct ReplaySmem {
  int V, x, coef, dt, fdt, lam, fw, flam, dot, total;
  __host__ __device__ ReplaySmem(int W, int n_in, int N, int vrows, int xrows, int xs, int rows,
                                 int es) {
    auto up16 = [](int b) { return (b + 15) & ~15; };
    V = 0;
    x = up16(V + vrows * N * es);
    coef = up16(x + xrows * xs * es);
    dt = coef + 4 * n_in * bc_stride(W);
    fdt = dt + 4 * W;
    lam = fdt + 4 * W;
    fw = lam + 4 * n_in;
    flam = fw + 4 * W;
    dot = flam + 4;
    total = dot + 4 * n_in * rows;
  }
};

// Eight waves per SIMD (<= 64 VGPRs): eight workgroups, 256 KiB of checkpoint
// loads in flight per CU.  kFull: every tile has 64 rows inside the head and
// N = 128, so every lane owns rows and columns and the fold and the dot
// products need no per-lane predicates; the instantiation for ragged tiles
// carries those predicates and is given twice the registers (four waves per
// SIMD) rather than spill.
template <typename T, int R, bool kFull>
__global__ __launch_bounds__(kThreads, kFull ? 8 : 4) void replay_kernel(ReplayArgs a, ReplayMeta m,
                                                          LogLayout lay) {
  extern __shared__ float4 rp_smem4[];
  char *sb = reinterpret_cast<char *>(rp_smem4);
  static_assert(R == 8, "two rows of four 16-byte chunks per lane");
  const ReplayTile tl;
  constexpr int kRows = 64;  // state rows of this workgroup's tile
  constexpr int E = 16 / (int)sizeof(T);  // io elements per 16-byte chunk
  constexpr int kWaves = kThreads / 64;
  const Dims d = a.d;
  const int W = a.W, n_in = a.n_in;
  const int ws = bc_stride(W);
  const int N = kFull ? 4 * 32 : d.N;
  const int pt = blockIdx.x, h = blockIdx.y;
  const int slot = m.slot[blockIdx.z];
  const uint32_t info = m.info[blockIdx.z];
  const int e = info_entry(info);  // row of the launch's inputs and outputs
  const int F = info_fold(info);
  const int base = info_base(info);
  const int rh = info_fold_half(info), wh = info_live_half(info);
  const int J = base + n_in;
  const int g = d.G == 1 ? 0 : h / (d.H / d.G);
  const int prow0 = pt * kRows;
  const int rv = kFull ? kRows : min(kRows, d.P - prow0);  // rows of this tile inside the head
  const bool whole_chunks = (d.P * (int)sizeof(T)) % 16 == 0 && (N * (int)sizeof(T)) % 16 == 0 &&
                            (((uintptr_t)a.x | (uintptr_t)a.C) & 15) == 0;
  // LDS stride of an entry's x rows: rv for whole chunks (the copies are
  // contiguous), else rounded up so that every 8-row group starts 16-byte aligned
  const int xs = whole_chunks ? rv : (rv + 7) & ~7;
  auto colok = [&](int q) { return kFull || tl.col(q) < N; };
  const size_t PN = (size_t)d.P * N;
  const float Ah = a.A[h], Dh = a.D[h];
  const LogIdx li{W};
  T *logdt = (T *)((char *)a.log + lay.dt_off);
  T *logx = (T *)((char *)a.log + lay.x_off);
  const T *logB = (const T *)((const char *)a.log + lay.B_off);
  const T *inx = (const T *)a.x, *indt = (const T *)a.dt, *inC = (const T *)a.C;
  const ReplaySmem L(W, n_in, N, a.vrows, a.xrows, xs, rv, (int)sizeof(T));
  T *s_V = (T *)(sb + L.V);  // [F + n_in][N]
  T *s_x = (T *)(sb + L.x);  // [J + F][xs]
  float *s_coef = (float *)(sb + L.coef), *s_dt = (float *)(sb + L.dt);
  float *s_fdt = (float *)(sb + L.fdt), *s_lam = (float *)(sb + L.lam);
  float *s_fw = (float *)(sb + L.fw), *s_flam = (float *)(sb + L.flam);
  float *s_dot = (float *)(sb + L.dot);

  // Six row sources, each a run of rows at a fixed stride: the committed
  // and the in-flight x, the fold entries' x, the fold B rows, the in-flight
  // C rows and the B.C rows.  Consecutive log entries of a slot and half are
  // consecutive in the log, so every run is (first row, stride, count).
  const size_t xstride = (size_t)d.H * d.P, vstride = (size_t)d.G * N;
  const T *x_com = logx + (li.ent(slot, wh, 0) * d.H + h) * d.P + prow0;
  const T *x_new = inx + ((size_t)e * n_in * d.H + h) * d.P + prow0;
  const T *c_new = inC + (size_t)e * n_in * vstride + (size_t)g * N;
  const float *bc = a.bc + ((size_t)e * d.G + g) * kMaxInFlight * ws;
  stage_lds(sb + L.coef, n_in * ws / 4, [&](int i) { return (const void *)(bc + 4 * i); });
  // Fold entries are staged FR at a time (the rows the launch reserved for
  // them): the first chunk with everything else, later chunks in the fold.
  const int FR = a.vrows - n_in;
  const int es = (int)sizeof(T);
  const int cx = rv / E, cv = N / E;
  const FastDiv fx(cx), fv(cv), frv(rv), fn(N);
  auto run = [&](char *lds, const T *src, size_t stride, int rows, int chunks, FastDiv f) {
    stage_lds(lds, rows * chunks, [&](int i) {
      const int j = f.div(i);
      return (const void *)(src + j * stride + (i - j * chunks) * E);
    });
  };
  // rows not made of aligned 16-byte chunks: element copies
  auto copy_rows = [&](T *dst, int dpitch, const T *src, size_t stride, int rows, int len,
                       FastDiv f) {
    for (int i = threadIdx.x; i < rows * len; i += kThreads) {
      const int j = f.div(i), r = i - j * len;
      dst[j * dpitch + r] = src[j * stride + r];
    }
  };
  // fold entries c0 .. c0 + cnt - 1: x rows after the J combined rows, B rows
  // at the top of V
  auto stage_fold = [&](int c0, int cnt) {
    // (sources recomputed here rather than kept live across the fold)
    const size_t ec = li.ent(slot, rh, c0);
    const T *xf = logx + (ec * d.H + h) * d.P + prow0;
    const T *bf = logB + ec * vstride + (size_t)g * N;
    if (whole_chunks) {
      run(sb + L.x + J * xs * es, xf, xstride, cnt, cx, fx);
      run(sb + L.V, bf, vstride, cnt, cv, fv);
    } else {
      copy_rows(s_x + J * xs, xs, xf, xstride, cnt, rv, frv);
      copy_rows(s_V, N, bf, vstride, cnt, N, fn);
    }
  };
  T *s_C = s_V + FR * N;  // in-flight C rows, after the fold rows
  if (whole_chunks) {
    run(sb + L.x, x_com, xstride, base, cx, fx);
    run(sb + L.x + base * xs * es, x_new, xstride, n_in, cx, fx);
    run((char *)s_C, c_new, vstride, n_in, cv, fv);
  } else {
    copy_rows(s_x, xs, x_com, xstride, base, rv, frv);
    copy_rows(s_x + base * xs, xs, x_new, xstride, n_in, rv, frv);
    copy_rows(s_C, N, c_new, vstride, n_in, N, fn);
  }
  stage_fold(0, min(F, FR));

  // checkpoint tile
  float *st = a.state + ((size_t)slot * d.H + h) * PN + (size_t)prow0 * N;
  float4 hv[R];  // hv[4 i + q]: row(i), chunk q
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = colok(q) && (kFull || tl.row(i) < rv);
      hv[4 * i + q] = ok ? nt_load4(st + (size_t)tl.row(i) * N + tl.col(q)) : zero4();
    }

  // dt of the combined entries, then of the fold entries: one load per
  // thread (J + F <= 2 W <= kThreads) and a single wait for everything
  const T *dt_com = logdt + li.ent(slot, wh, 0) * d.H + h;
  const T *dt_new = indt + (size_t)e * n_in * d.H + h;
  const T *dt_fold = logdt + li.ent(slot, rh, 0) * d.H + h;
  const int tid = threadIdx.x;
  if (tid < J + F) {
    const T *src = tid < base ? dt_com + (size_t)tid * d.H
                   : tid < J  ? dt_new + (size_t)(tid - base) * d.H
                              : dt_fold + (size_t)(tid - J) * d.H;
    const float v = to_f(*src);
    if (tid < J)
      s_dt[tid] = v;
    else
      s_fdt[tid - J] = v;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the LDS copies above have landed
  __syncthreads();

  // Scalar weights.  Wave w takes the in-flight tokens w, w + kWaves, ...;
  // the last wave also the fold.
  // Lane l stands for entry j = 63 - l, so the lane prefix sum of dt_{j+1}
  // is the entry suffix sum S_j = sum_{j < i <= m} dt_i (J, F <= W <= 64).
  const int wave = __builtin_amdgcn_readfirstlane(tl.wave);
  const int jr = 63 - tl.lane;
  for (int k = wave; k < n_in; k += kWaves) {
    const int mm = base + k;
    const float S = wave_prefix_sum(jr + 1 <= mm ? s_dt[jr + 1] : 0.f);
    if (jr < ws) {
      float cf = 0.f;  // zero past the token's own entry
      if (jr <= mm) {
        cf = expf(Ah * S) * s_dt[jr] * s_coef[k * ws + jr];
        if (jr == mm) cf += Dh;  // the skip term D x_m rides on the newest entry
      }
      s_coef[k * ws + jr] = cf;
    }
    if (jr == 0) s_lam[k] = expf(Ah * (s_dt[0] + S));
  }
  if (F > 0 && wave == kWaves - 1) {
    const float S = wave_prefix_sum(jr + 1 < F ? s_fdt[jr + 1] : 0.f);
    if (jr < F) s_fw[jr] = expf(Ah * S) * s_fdt[jr];
    if (jr == 0) s_flam[0] = expf(Ah * (s_fdt[0] + S));
  }
  __syncthreads();

  // fold, then ckpt . C_k for every in-flight token
  if (F > 0) {
    const float lam = s_flam[0];
#pragma unroll
    for (int i = 0; i < R; ++i)
      hv[i] = make_float4(lam * hv[i].x, lam * hv[i].y, lam * hv[i].z, lam * hv[i].w);
    const T *fx = s_x + J * xs + tl.row(0);  // this lane's two consecutive rows
    for (int c0 = 0; c0 < F; c0 += FR) {  // uniform across the workgroup
      const int cnt = min(FR, F - c0);
      if (c0 > 0) {  // the next chunk of fold rows, once every wave is done with this one
        __syncthreads();
        stage_fold(c0, cnt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
#pragma unroll 1
      for (int j = 0; j < cnt; ++j) {
        const float w = s_fw[c0 + j];
        float xv[2];
        lds_ld_pair(fx + j * xs, xv);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 Bv = colok(q) ? lds_ld4(s_V + j * N + tl.col(q)) : zero4();
#pragma unroll
          for (int i = 0; i < 2; ++i)
            hv[4 * i + q] =
                fma4(1.f, hv[4 * i + q], (kFull || tl.row(i) < rv) ? w * xv[i] : 0.f, Bv);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (colok(q) && (kFull || tl.row(i) < rv))
          nt_store4(st + (size_t)tl.row(i) * N + tl.col(q), hv[4 * i + q]);
  }
  for (int k = 0; k < n_in; ++k) {
    float part[2];  // one multiply-add chain per row over the lane's 16 columns
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 Cv = colok(q) ? lds_ld4(s_C + k * N + tl.col(q)) : zero4();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float4 hq = hv[4 * i + q];
        float acc = q == 0 ? hq.x * Cv.x : fmaf(hq.x, Cv.x, part[i]);
        acc = fmaf(hq.y, Cv.y, acc);
        acc = fmaf(hq.z, Cv.z, acc);
        part[i] = fmaf(hq.w, Cv.w, acc);
      }
    }
    const float v = tl.totals(part[0], part[1]);
    if (tl.reduced_writer() && (kFull || tl.reduced_row() < rv))
      s_dot[k * rv + tl.reduced_row()] = v;
  }

  // append the in-flight x and dt to the live log half
  const FastDiv frows(rv);
  T *x_app = logx + (li.ent(slot, wh, base) * d.H + h) * d.P + prow0;
  for (int i = threadIdx.x; i < n_in * rv; i += kThreads) {
    const int k = frows.div(i), r = i - k * rv;
    x_app[k * xstride + r] = s_x[(base + k) * xs + r];
  }
  if (pt == 0)
    for (int k = threadIdx.x; k < n_in; k += kThreads)
      Io<T>::st(logdt + li.ent(slot, wh, base + k) * d.H + h, s_dt[base + k]);
  __syncthreads();

  // outputs: lane = row, one wave per in-flight token, so the loop over
  // entries is uniform across the wave (D x_m is inside the newest weight);
  // the weights of a token are contiguous and read four at a time
  static_assert(kRows == 64, "one lane per tile row");
  if (tl.lane < rv) {
    const int r = tl.lane;
    T *yr = (T *)a.y + ((size_t)e * n_in * d.H + h) * d.P + prow0 + r;
    for (int k = wave; k < n_in; k += kWaves) {
      const int mm = base + k;
      const float *cf = s_coef + k * ws;
      const T *xr = s_x + r;
      float acc = s_lam[k] * s_dot[k * rv + r];
      int j = 0;
      for (; j + 3 <= mm; j += 4) {
        const float4 c = *reinterpret_cast<const float4 *>(cf + j);
        acc += c.x * to_f(xr[j * xs]);
        acc += c.y * to_f(xr[(j + 1) * xs]);
        acc += c.z * to_f(xr[(j + 2) * xs]);
        acc += c.w * to_f(xr[(j + 3) * xs]);
      }
      for (; j <= mm; ++j) acc += cf[j] * to_f(xr[j * xs]);
      Io<T>::st(yr + (size_t)k * d.H * d.P, acc);
    }
  }
}

static size_t replay_smem_bytes(int io, int W, int n_in, int N, int vrows, int xrows) {
  // xs and rows are at most the tile height, so this bounds every tile's need
  return (size_t)ReplaySmem(W, n_in, N, vrows, xrows, 8 * kReplayR, 8 * kReplayR,
                            io == kBF16 ? 2 : 4)
      .total;
}

static size_t replay_bc_smem_bytes(int W, int n_in, int N) {
  return sizeof(float4) * (size_t)(W + n_in) * (N / 4 + 1);
}

template <typename K> static hipError_t allow_lds(K kernel, size_t bytes) {
  return allow_dynamic_lds(reinterpret_cast<const void *>(kernel), bytes);
}

hipError_t launch_replay(int io, const ReplayArgs &a, const ReplayMeta &m, const LogLayout &lay,
                         hipStream_t s) {
  if (a.n_in > 0) {
    dim3 g1(a.d.G, a.n), b1(kThreads);
    const size_t sm1 = replay_bc_smem_bytes(a.W, a.n_in, a.d.N);
    hipError_t err;
    if (io == kBF16) {
      err = allow_lds(replay_bc_kernel<bf16_t>, sm1);
      if (err == hipSuccess) hipLaunchKernelGGL(replay_bc_kernel<bf16_t>, g1, b1, sm1, s, a, m, lay);
    } else {
      err = allow_lds(replay_bc_kernel<float>, sm1);
      if (err == hipSuccess) hipLaunchKernelGGL(replay_bc_kernel<float>, g1, b1, sm1, s, a, m, lay);
    }
    if (err == hipSuccess) err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int pt_n = (a.d.P + 8 * kReplayR - 1) / (8 * kReplayR);
  const bool full = a.d.P % (8 * kReplayR) == 0 && a.d.N == 4 * 32;
  auto launch = [&](const ReplayArgs &la, const ReplayMeta &lm) {
    dim3 grid(pt_n, la.d.H, la.n), block(kThreads);
    const size_t sm = replay_smem_bytes(io, la.W, la.n_in, la.d.N, la.vrows, la.xrows);
    auto go = [&](auto kernel) {
      hipError_t err = allow_lds(kernel, sm);
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(kernel, grid, block, sm, s, la, lm, lay);
      return hipGetLastError();
    };
    if (io == kBF16)
      return full ? go(replay_kernel<bf16_t, kReplayR, true>)
                  : go(replay_kernel<bf16_t, kReplayR, false>);
    return full ? go(replay_kernel<float, kReplayR, true>)
                : go(replay_kernel<float, kReplayR, false>);
  };
  // One launch for every entry.  Its LDS reservation holds the in-flight C
  // rows, the largest J rows of x and FR fold rows (B and x); an entry that
  // folds more than FR entries stages them FR at a time.  FR is the largest
  // count whose reservation keeps eight workgroups per CU (160 KiB of LDS),
  // at least eight (else all of the longest fold at once).
  ReplayMeta ml;
  int maxF = 0, maxJ = a.n_in;
  for (int i = 0; i < a.n; ++i) {
    const uint32_t u = info_with_entry(m.info[i], i);
    ml.slot[i] = m.slot[i];
    ml.info[i] = u;
    maxF = max(maxF, info_fold(u));
    if (info_fold(u) == 0) maxJ = max(maxJ, info_base(u) + a.n_in);
  }
  if (a.n == 0) return hipSuccess;
  auto smem = [&](int fr) {
    return replay_smem_bytes(io, a.W, a.n_in, a.d.N, fr + a.n_in, max(maxJ, a.n_in + fr));
  };
  int FR = maxF;
  while (FR > 8 && smem(FR) > 160 * 1024 / 8) --FR;
  if (smem(FR) > 160 * 1024 / 8) FR = maxF;
  ReplayArgs la = a;
  la.vrows = FR + a.n_in;
  la.xrows = max(maxJ, a.n_in + FR);
  return launch(la, ml);
}

// ===========================================================================
// state operations
// ===========================================================================
__global__ void zero_kernel(float *dst, size_t n) {
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    reinterpret_cast<float4 *>(dst)[i] = zero4();
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = 0.f;
}

__global__ void copy_f32_kernel(float *dst, const float *src, size_t n) {
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    reinterpret_cast<float4 *>(dst)[i] = reinterpret_cast<const float4 *>(src)[i];
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void zero_u64_kernel(unsigned long long *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

__global__ void checksum_kernel(const uint32_t *w, size_t n, unsigned long long *acc) {
  unsigned long long s = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    s += (unsigned long long)w[i] * (2ull * i + 1ull);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((threadIdx.x & 63) == 0) atomicAdd(acc, s);
}

template <typename T> __global__ void finite_kernel(const T *p, size_t n, unsigned int *flag) {
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const float v = Io<T>::ld(p + i);
    bad |= !isfinite(v);
  }
  if (bad) atomicOr(flag, 1u);
}

static unsigned grid_for(size_t n, unsigned per = 4) {
  size_t g = (n / per + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (unsigned)g;
}

hipError_t launch_zero(float *dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, dst, n);
  return hipGetLastError();
}
hipError_t launch_copy_f32(float *dst, const float *src, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, dst, src, n);
  return hipGetLastError();
}
hipError_t launch_zero_u64(unsigned long long *p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3((n + 63) / 64), dim3(64), 0, s, p, n);
  return hipGetLastError();
}
hipError_t launch_checksum(const float *src, size_t n, unsigned long long *acc, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(checksum_kernel, dim3(grid_for(n, 8)), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint32_t *>(src), n, acc);
  return hipGetLastError();
}
hipError_t launch_finite_check(int io, const void *p, size_t n, unsigned int *flag,
                               hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (io == kBF16)
    hipLaunchKernelGGL(finite_kernel<bf16_t>, dim3(grid_for(n, 8)), dim3(kThreads), 0, s,
                       (const bf16_t *)p, n, flag);
  else
    hipLaunchKernelGGL(finite_kernel<float>, dim3(grid_for(n, 8)), dim3(kThreads), 0, s,
                       (const float *)p, n, flag);
  return hipGetLastError();
}

}  // namespace ssm
