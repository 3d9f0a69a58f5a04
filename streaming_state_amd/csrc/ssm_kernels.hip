// ssm_kernels.hip -- gfx950 kernels of the memory-bound paths: batched decode,
// copy-per-draft verify (baseline), ReplaySSM verify with the fused log fold,
// and the state operations (zero, copy, checksum, finite check).
//
// All three verify/decode kernels share one shape: a workgroup of 256 threads
// owns one (batch entry, head, 64-row tile) of the fp32 state, held in
// registers as 8 float4 per thread (Tile in ssm_device.h).  The state is read
// with one pass of 128-bit loads and written (when it is written at all) with
// one pass of 128-bit nontemporal stores; inputs and outputs are small.
#include "ssm_device.h"

namespace ssm {

static __device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// ===========================================================================
// decode: h <- exp(dt A) h + dt x B^T ; y = h C + D x, one token per slot
// ===========================================================================
// Decode tiles: R float4 rows per thread (a 256-thread tile covers 8R state
// rows of one head) and kDecodeTiles consecutive tiles of one slot per
// workgroup.  On MI355X an in-place read-modify-write sweep is fastest with
// 16 KiB or 128 KiB per workgroup and slowest with 32-64 KiB.
constexpr int kDecodeR = 4;
constexpr int kDecodeTiles = 2;

template <typename T, int R, int TW>
__global__ __launch_bounds__(kThreads *TW) void decode_kernel(DecodeArgs a, DecodeMeta m) {
  const TileR<R> tl;
  const Dims d = a.d;
  constexpr int kTileRows = 8 * R;
  const int pt_n = (d.P + kTileRows - 1) / kTileRows;
  const int tiles_per_entry = d.H * pt_n;
  const int groups = (tiles_per_entry + TW - 1) / TW;
  const int k = blockIdx.x / groups;
  const int tile = (blockIdx.x % groups) * TW + (int)(threadIdx.x / kThreads);
  if (tile >= tiles_per_entry) return;  // no barriers below: tiles are independent
  const int pt = tile % pt_n;
  const int h = tile / pt_n;
  const int slot = m.slot[k];
  const int e = m.ent[k];
  const bool rst = m.reset[k] != 0;
  const int g = h / (d.H / d.G);
  const int prow0 = pt * kTileRows;
  const bool colok = 4 * tl.c < d.N;

  float *st = a.state + (((size_t)slot * d.H + h) * d.P + prow0) * d.N + 4 * tl.c;
  // state first: the only large read, issued before anything else
  float4 hv[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const bool ok = colok && (prow0 + tl.row(i) < d.P) && !rst;
    hv[i] = ok ? nt_load4(st + (size_t)tl.row(i) * d.N) : zero4();
  }
  const T *x = (const T *)a.x + ((size_t)e * d.H + h) * d.P + prow0;
  const float dt = Io<T>::ld((const T *)a.dt + (size_t)e * d.H + h);
  const float dA = expf(dt * a.A[h]);
  const float Dh = a.D[h];
  float4 Bv = zero4(), Cv = zero4();
  if (colok) {
    Bv = Io<T>::ld4((const T *)a.B + ((size_t)e * d.G + g) * d.N + 4 * tl.c);
    Cv = Io<T>::ld4((const T *)a.C + ((size_t)e * d.G + g) * d.N + 4 * tl.c);
  }
  float part[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const bool rowok = prow0 + tl.row(i) < d.P;
    const float u = rowok ? dt * Io<T>::ld(x + tl.row(i)) : 0.f;
    hv[i] = fma4(dA, hv[i], u, Bv);
    if (rowok && colok) nt_store4(st + (size_t)tl.row(i) * d.N, hv[i]);
    part[i] = dot4(hv[i], Cv);
  }
  const float yv = reduce_rows<R>(part, tl.lane);
  const int r = tl.reduced_row();
  if (tl.reduced_writer() && prow0 + r < d.P)
    Io<T>::st((T *)a.y + ((size_t)e * d.H + h) * d.P + prow0 + r, yv + Dh * Io<T>::ld(x + r));
}

hipError_t launch_decode(int io, const DecodeArgs &a, const DecodeMeta &m, hipStream_t s) {
  constexpr int kTileRows = 8 * kDecodeR;
  const int tiles = a.d.H * ((a.d.P + kTileRows - 1) / kTileRows);
  dim3 grid(a.n * ((tiles + kDecodeTiles - 1) / kDecodeTiles)), block(kThreads * kDecodeTiles);
  if (io == kBF16)
    hipLaunchKernelGGL((decode_kernel<bf16_t, kDecodeR, kDecodeTiles>), grid, block, 0, s, a, m);
  else
    hipLaunchKernelGGL((decode_kernel<float, kDecodeR, kDecodeTiles>), grid, block, 0, s, a, m);
  return hipGetLastError();
}

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
    const float yv = reduce_rows<R>(part, tl.lane);
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
LogLayout log_layout(int io, const Dims &d, int S, int W) {
  const size_t es = io == kBF16 ? 2 : 4;
  const size_t ent = (size_t)S * 2 * W;
  LogLayout L;
  L.dt_off = 0;
  L.x_off = (L.dt_off + ent * d.H * es + 255) & ~(size_t)255;
  L.B_off = (L.x_off + ent * d.H * d.P * es + 255) & ~(size_t)255;
  L.bc_off = (L.B_off + ent * d.G * d.N * es + 255) & ~(size_t)255;
  // B.C scratch: [kBatchPerLaunch][G][W][kMaxInFlight] fp32
  L.total = L.bc_off + (size_t)kBatchPerLaunch * d.G * W * kMaxInFlight * 4;
  return L;
}

// Offsets of entry j of half `half` of slot `slot` (element units).
struct LogIdx {
  int W;
  __device__ __forceinline__ size_t ent(int slot, int half, int j) const {
    return ((size_t)slot * 2 + half) * W + j;
  }
};

// Pass 1: B_j . C_k for every combined entry j (committed log, then in-flight)
// and in-flight token k, per (entry, group); these are shared by all heads of
// a group.  Also appends the in-flight B rows to the live log half.
template <typename T>
__global__ __launch_bounds__(kThreads) void replay_bc_kernel(ReplayArgs a, ReplayMeta m,
                                                             LogLayout lay) {
  const Dims d = a.d;
  const int e = blockIdx.x / d.G, g = blockIdx.x % d.G;
  const int slot = m.slot[e];
  const int base = m.base_len[e];
  const int wh = (m.halves[e] >> 1) & 1;
  const int J = base + a.n_in;
  const LogIdx li{a.W};
  T *logB = (T *)((char *)a.log + lay.B_off);
  const T *inB = (const T *)a.B, *inC = (const T *)a.C;
  // append in-flight B rows
  for (int i = threadIdx.x; i < a.n_in * d.N; i += kThreads) {
    const int k = i / d.N, n = i % d.N;
    const size_t ek = (size_t)e * a.n_in + k;
    logB[(li.ent(slot, wh, base + k) * d.G + g) * d.N + n] = inB[(ek * d.G + g) * d.N + n];
  }
  // dot products: one wave per (j, k) pair, lanes over n
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float *bc = a.bc + ((size_t)e * d.G + g) * a.W * kMaxInFlight;
  for (int pr = wave; pr < J * a.n_in; pr += kThreads / 64) {
    const int j = pr / a.n_in, k = pr % a.n_in;
    const T *Bj = j < base ? logB + (li.ent(slot, wh, j) * d.G + g) * d.N
                           : inB + (((size_t)e * a.n_in + (j - base)) * d.G + g) * d.N;
    const T *Ck = inC + (((size_t)e * a.n_in + k) * d.G + g) * d.N;
    float acc = 0.f;
    for (int n = lane; n < d.N; n += 64) acc += Io<T>::ld(Bj + n) * Io<T>::ld(Ck + n);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) bc[j * kMaxInFlight + k] = acc;
  }
}

// Pass 2, per (entry, head, 64-row tile): read the checkpoint once; if the log
// is full, fold it in (ckpt <- Lambda ckpt + sum_j w_j x_j B_j^T) and write the
// checkpoint back -- the only state write; then emit every in-flight token's
// output from the checkpoint and the combined log:
//   y_k = Lambda_m (ckpt . C_k) + sum_{j<=m} w_{j,m} x_j (B_j . C_k) + D x_k,
// m = base + k, Lambda_m = exp(A sum_{i<=m} dt_i),
// w_{j,m} = exp(A sum_{j<i<=m} dt_i) dt_j  (direct suffix sums, at most W terms).
constexpr int kReplayR = 8;  // 32 KiB tiles: its per-workgroup setup (log staging, decay
                             // weights) costs more than 16 KiB tiles gain

template <typename T, int R>
__global__ __launch_bounds__(kThreads) void replay_kernel(ReplayArgs a, ReplayMeta m,
                                                          LogLayout lay) {
  extern __shared__ float smem[];
  const TileR<R> tl;
  constexpr int kRows = 8 * R;  // state rows of this workgroup's tile
  const Dims d = a.d;
  const int W = a.W, n_in = a.n_in;
  const int pt_n = (d.P + kRows - 1) / kRows;
  int bid = blockIdx.x;
  const int pt = bid % pt_n;
  bid /= pt_n;
  const int h = bid % d.H;
  const int e = bid / d.H;
  const int slot = m.slot[e];
  const int F = m.fold_len[e];
  const int base = m.base_len[e];
  const int rh = m.halves[e] & 1, wh = (m.halves[e] >> 1) & 1;
  const int J = base + n_in;
  const int g = h / (d.H / d.G);
  const int prow0 = pt * kRows;
  const bool colok = 4 * tl.c < d.N;
  const size_t PN = (size_t)d.P * d.N;
  const float Ah = a.A[h], Dh = a.D[h];
  const LogIdx li{W};
  T *logdt = (T *)((char *)a.log + lay.dt_off);
  T *logx = (T *)((char *)a.log + lay.x_off);
  const T *logB = (const T *)((const char *)a.log + lay.B_off);
  const T *inx = (const T *)a.x, *indt = (const T *)a.dt, *inC = (const T *)a.C;

  // checkpoint tile first
  float *st = a.state + ((size_t)slot * d.H + h) * PN + (size_t)prow0 * d.N + 4 * tl.c;
  float4 hv[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const bool ok = colok && (prow0 + tl.row(i) < d.P);
    hv[i] = ok ? nt_load4(st + (size_t)tl.row(i) * d.N) : zero4();
  }

  // LDS carve-up (sizes from the host): fold x [W][64], fold dt/w [W],
  // combined dt [W], combined x [W][64], coef [W][kMaxInFlight],
  // lambda [kMaxInFlight], dot [kMaxInFlight][64], fold lambda [1]
  float *s_fx = smem;
  float *s_fdt = s_fx + W * kRows;
  float *s_fw = s_fdt + W;
  float *s_dt = s_fw + W;
  float *s_x = s_dt + W;
  float *s_coef = s_x + W * kRows;
  float *s_lam = s_coef + W * kMaxInFlight;
  float *s_dot = s_lam + kMaxInFlight;
  float *s_flam = s_dot + kMaxInFlight * kRows;

  // stage fold entries (read half), combined entries, and append in-flight x/dt
  for (int i = threadIdx.x; i < F * kRows; i += kThreads) {
    const int j = i / kRows, r = i % kRows;
    s_fx[i] = prow0 + r < d.P
                  ? Io<T>::ld(logx + (li.ent(slot, rh, j) * d.H + h) * d.P + prow0 + r)
                  : 0.f;
  }
  for (int j = threadIdx.x; j < F; j += kThreads)
    s_fdt[j] = Io<T>::ld(logdt + li.ent(slot, rh, j) * d.H + h);
  for (int i = threadIdx.x; i < J * kRows; i += kThreads) {
    const int j = i / kRows, r = i % kRows;
    float v = 0.f;
    if (prow0 + r < d.P) {
      if (j < base) {
        v = Io<T>::ld(logx + (li.ent(slot, wh, j) * d.H + h) * d.P + prow0 + r);
      } else {
        const T *src = inx + (((size_t)e * n_in + (j - base)) * d.H + h) * d.P + prow0 + r;
        const T raw = *src;
        v = Io<T>::ld(src);
        logx[(li.ent(slot, wh, j) * d.H + h) * d.P + prow0 + r] = raw;
      }
    }
    s_x[i] = v;
  }
  for (int j = threadIdx.x; j < J; j += kThreads) {
    float v;
    if (j < base) {
      v = Io<T>::ld(logdt + li.ent(slot, wh, j) * d.H + h);
    } else {
      const T *src = indt + ((size_t)e * n_in + (j - base)) * d.H + h;
      v = Io<T>::ld(src);
      if (pt == 0) logdt[li.ent(slot, wh, j) * d.H + h] = *src;
    }
    s_dt[j] = v;
  }
  __syncthreads();

  // scalar weights
  for (int j = threadIdx.x; j < F; j += kThreads) {
    float suf = 0.f;
    for (int i = j + 1; i < F; ++i) suf += s_fdt[i];
    s_fw[j] = expf(Ah * suf) * s_fdt[j];
  }
  if (threadIdx.x == kThreads - 1) {
    float tot = 0.f;
    for (int i = 0; i < F; ++i) tot += s_fdt[i];
    s_flam[0] = expf(Ah * tot);
  }
  const float *bc = a.bc + ((size_t)e * d.G + g) * W * kMaxInFlight;
  for (int t = threadIdx.x; t < J * n_in; t += kThreads) {
    const int j = t / n_in, k = t % n_in, mm = base + k;
    float cf = 0.f;
    if (j <= mm) {
      float suf = 0.f;
      for (int i = j + 1; i <= mm; ++i) suf += s_dt[i];
      cf = expf(Ah * suf) * s_dt[j] * bc[j * kMaxInFlight + k];
    }
    s_coef[j * kMaxInFlight + k] = cf;
  }
  for (int k = threadIdx.x; k < n_in; k += kThreads) {
    float tot = 0.f;
    for (int i = 0; i <= base + k; ++i) tot += s_dt[i];
    s_lam[k] = expf(Ah * tot);
  }
  __syncthreads();

  // fold the full log into the checkpoint and write it back
  if (F > 0) {
    const float lam = s_flam[0];
#pragma unroll
    for (int i = 0; i < R; ++i)
      hv[i] = make_float4(lam * hv[i].x, lam * hv[i].y, lam * hv[i].z, lam * hv[i].w);
    for (int j = 0; j < F; ++j) {
      float4 Bv = zero4();
      if (colok) Bv = Io<T>::ld4(logB + (li.ent(slot, rh, j) * d.G + g) * d.N + 4 * tl.c);
      const float w = s_fw[j];
#pragma unroll
      for (int i = 0; i < R; ++i) hv[i] = fma4(1.f, hv[i], w * s_fx[j * kRows + tl.row(i)], Bv);
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (colok && prow0 + tl.row(i) < d.P) nt_store4(st + (size_t)tl.row(i) * d.N, hv[i]);
  }

  // ckpt . C_k for every in-flight token
  for (int k = 0; k < n_in; ++k) {
    float4 Cv = zero4();
    if (colok) Cv = Io<T>::ld4(inC + (((size_t)e * n_in + k) * d.G + g) * d.N + 4 * tl.c);
    float part[R];
#pragma unroll
    for (int i = 0; i < R; ++i) part[i] = dot4(hv[i], Cv);
    const float v = reduce_rows<R>(part, tl.lane);
    if (tl.reduced_writer()) s_dot[k * kRows + tl.reduced_row()] = v;
  }
  __syncthreads();

  // outputs
  for (int i = threadIdx.x; i < n_in * kRows; i += kThreads) {
    const int k = i / kRows, r = i % kRows;
    if (prow0 + r >= d.P) continue;
    const int mm = base + k;
    float acc = s_lam[k] * s_dot[k * kRows + r];
    for (int j = 0; j <= mm; ++j) acc += s_coef[j * kMaxInFlight + k] * s_x[j * kRows + r];
    acc += Dh * s_x[mm * kRows + r];
    Io<T>::st((T *)a.y + (((size_t)e * n_in + k) * d.H + h) * d.P + prow0 + r, acc);
  }
}

static size_t replay_smem_bytes(int W) {
  constexpr int kRows = 8 * kReplayR;
  return sizeof(float) *
         ((size_t)W * kRows + W + W + W + (size_t)W * kRows + (size_t)W * kMaxInFlight +
          kMaxInFlight + (size_t)kMaxInFlight * kRows + 1);
}

hipError_t launch_replay(int io, const ReplayArgs &a, const ReplayMeta &m, const LogLayout &lay,
                         hipStream_t s) {
  if (a.n_in > 0) {
    dim3 g1(a.n * a.d.G), b1(kThreads);
    if (io == kBF16)
      hipLaunchKernelGGL(replay_bc_kernel<bf16_t>, g1, b1, 0, s, a, m, lay);
    else
      hipLaunchKernelGGL(replay_bc_kernel<float>, g1, b1, 0, s, a, m, lay);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int pt_n = (a.d.P + 8 * kReplayR - 1) / (8 * kReplayR);
  dim3 grid(a.n * a.d.H * pt_n), block(kThreads);
  const size_t sm = replay_smem_bytes(a.W);
  if (io == kBF16)
    hipLaunchKernelGGL((replay_kernel<bf16_t, kReplayR>), grid, block, sm, s, a, m, lay);
  else
    hipLaunchKernelGGL((replay_kernel<float, kReplayR>), grid, block, sm, s, a, m, lay);
  return hipGetLastError();
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
