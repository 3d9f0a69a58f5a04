// ssm_chunk.hip -- chunk scan, tile-parallel form on fp32 MFMA.
//
// The recurrent form walks a segment token by token, so a long chunk of a
// few-head layer leaves most of the chip idle.  Here the chunk is cut into
// tiles of 64 tokens and the same algebra is split into three passes
// ("Separate Mamba-2 algebra from kernel behavior": within a tile the
// recurrence is a masked matrix product, across tiles it is a short affine
// chain):
//   1. chunk_state_kernel   (tile, head):  S_c = sum_s w_s x_s B_s^T  and the
//                           tile decay lam_c, from a zero state
//   2. chunk_carry_kernel   (head, slice): h_in(c) for every tile by the chain
//                           h <- lam_c h + S_c, starting from the slot state;
//                           the last value is the carry-out
//   3. chunk_output_kernel  (tile, head):  y_t = sum_{s<=t} M[t,s] x_s
//                           + exp(cs_t) C_t h_in(c) (+ D x_t on M's diagonal),
//                           and any checkpoint inside the tile
// With cs_t the inclusive running sum of dt*A inside the tile:
//   M[t,s] = (C_t . B_s) exp(cs_t - cs_s) dt_s   for s <= t in the same segment
//   w_s    = exp(cs_end - cs_s) dt_s              for s in the tile's last segment
//   lam_c  = exp(cs_end), or 0 if a reset falls inside the tile
// A reset before token t of the tile starts a new segment: pairs across it are
// masked out and the carried-in state does not reach t or later.
//
// The running sums are kept in fp64: every difference cs_t - cs_s is then
// exact to far below fp32 rounding before it is rounded once for exp, so the
// decay factors carry no cancellation error however fast the head decays.
//
// MFMA: v_mfma_f32_32x32x2f32.  Lane l supplies A[l%32][k_l] and B[k_l][l%32],
// where the two half-waves take contraction indices 32 apart (k and k + 32 of
// each 64-wide K block); accumulator register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32.  Operands are read from LDS one float
// per lane.  4-byte LDS reads are served 32 lanes per cycle from 32 banks;
// every operand array has an odd row pitch, so the 32 rows one half-wave reads
// along K (stride = pitch) fall on 32 distinct banks.
//
// exp is taken as exp2 of an fp32 argument scaled by log2(e) in fp64: the
// argument is rounded to fp32 once, as it would be for expf.
#include <algorithm>

#include "ssm_device.h"

namespace ssm {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int QT = kChunkTile;  // tokens per tile (64)
constexpr int kMaxP = 64;
constexpr int NP = kMaxN + 1;   // odd pitches (see above)
constexpr int PP = kMaxP + 1;
constexpr int MP = QT + 1;

__device__ __forceinline__ f32x16_t mfma(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
// acc += A[:, 0:K] B[0:K, :] for one 32x32 block, K a multiple of 64; fa(k) and
// fb(k) read this lane's A and B operands for contraction index k.  Eight
// MFMAs' operands are read before the first of them issues.
template <typename FA, typename FB>
__device__ __forceinline__ f32x16_t mma(f32x16_t acc, int K, FA fa, FB fb) {
  const int hk = 32 * ((threadIdx.x >> 5) & 1);
  for (int kb = 0; kb < K; kb += 64) {
#pragma unroll
    for (int ub = 0; ub < 32; ub += 8) {
      float av[8], bv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = kb + hk + ub + u;
        av[u] = fa(k);
        bv[u] = fb(k);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = mfma(av[u], bv[u], acc);
    }
  }
  return acc;
}
__device__ __forceinline__ float exp_d(double x) {
  return __builtin_amdgcn_exp2f((float)(x * 1.4426950408889634));
}

// Per-tile scalars: dt, the fp64 running sum of dt*A, and the segment index
// (resets at or before each token within the tile).
struct TileScalars {
  float dt[QT];
  double cs[QT];
  int seg[QT];
};

__device__ __forceinline__ int seg_upto(uint64_t rmask, int j) {
  return __popcll(rmask & (j == 63 ? ~0ull : ((2ull << j) - 1)));
}

// dt of token j of the tile (row clamped so the load is always in bounds).
template <typename T>
__device__ __forceinline__ float load_dt(const T *dt, int tbase, int n, int H, int h, int j) {
  return Io<T>::ld(dt + (size_t)(tbase + min(j, n - 1)) * H + h);
}

// Wave 0 (lane j = token j): inclusive running sum of dt*A in fp64 (each term
// is the exact product of two fp32 values; Hillis-Steele scan).
__device__ __forceinline__ double tile_cumsum(float d, float Ah) {
  const int j = threadIdx.x;
  double v = (double)d * (double)Ah;
#pragma unroll
  for (int o = 1; o < QT; o <<= 1) {
    const double u = __shfl_up(v, o, QT);
    if (j >= o) v += u;
  }
  return v;
}

// A [64 rows][cols] slab of the io dtype read as float4 chunks: thread t takes
// chunks t, t + 256, ...  Every load is issued before any is used, with the
// row and chunk clamped into range, so the loads overlap one another.
template <typename T, int kCols>
struct RowTile {
  static constexpr int kC4 = kCols / 4;
  static constexpr int kPer = QT * kC4 / kThreads;
  float4 v[kPer];
  __device__ __forceinline__ void load(const T *base, size_t row_stride, int rows, int cols4) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = threadIdx.x + kThreads * k;
      const int r = min(q / kC4, rows - 1), c4 = min(q % kC4, cols4 - 1);
      v[k] = Io<T>::ld4(base + (size_t)r * row_stride + 4 * c4);
    }
  }
  // dst[r * pitch + col] = value * scale(r) for rows r < rows_max; rows past
  // rows_valid and columns past 4 * cols4 (up to kCols) are written as zero,
  // so contractions may run over the padded width.
  template <int kPitch, typename F>
  __device__ __forceinline__ void store(float *dst, int rows_valid, int rows_max, int cols4,
                                        F scale) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = threadIdx.x + kThreads * k;
      const int r = q / kC4, c4 = q % kC4;
      if (r >= rows_max) continue;
      const bool ok = r < rows_valid && c4 < cols4;
      const float f = ok ? scale(r) : 0.f;
      float *o = dst + r * kPitch + 4 * c4;
      o[0] = ok ? v[k].x * f : 0.f;
      o[1] = ok ? v[k].y * f : 0.f;
      o[2] = ok ? v[k].z * f : 0.f;
      o[3] = ok ? v[k].w * f : 0.f;
    }
  }
};
struct One {
  __device__ __forceinline__ float operator()(int) const { return 1.f; }
};

// ------------------------------------------------------------- pass 1: S_c
struct StateSmem {
  float B[QT][NP];   // B[s][n]
  float X[QT][PP];   // w_s x[s][p]
  float w[QT];
};

template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(ChunkArgs a, ChunkMeta m) {
  __shared__ StateSmem sm;
  const Dims d = a.d;
  const int c = blockIdx.x / d.H, h = blockIdx.x % d.H;
  const int g = h / (d.H / d.G);
  const int tbase = a.t0 + c * QT;
  const int n = min(QT, a.t0 + a.len - tbase);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N4 = d.N >> 2, P4 = d.P >> 2;

  float dtv = 0.f;
  if (tid < QT) dtv = load_dt((const T *)a.dt, tbase, n, d.H, h, tid);
  RowTile<T, kMaxN> bt;
  bt.load((const T *)a.B + ((size_t)tbase * d.G + g) * d.N, (size_t)d.G * d.N, n, N4);
  RowTile<T, kMaxP> xt;
  xt.load((const T *)a.x + ((size_t)tbase * d.H + h) * d.P, (size_t)d.H * d.P, n, P4);

  if (tid < QT) {  // wave 0: weights w_s and the tile decay
    const double cs = tile_cumsum(tid < n ? dtv : 0.f, a.A[h]);
    const double cse = __shfl(cs, n - 1, QT);
    const uint64_t rm = m.rmask[c];
    const int sege = seg_upto(rm, n - 1);
    sm.w[tid] = (tid < n && seg_upto(rm, tid) == sege) ? exp_d(cse - cs) * dtv : 0.f;
    if (tid == 0) a.lam[(size_t)c * d.H + h] = sege == 0 ? exp_d(cse) : 0.f;
  }
  __syncthreads();
  bt.template store<NP>(&sm.B[0][0], n, QT, N4, One());
  xt.template store<PP>(&sm.X[0][0], n, QT, P4, [&](int r) { return sm.w[r]; });
  __syncthreads();

  const int kend = QT;  // rows past the tile's end are zero
  const int tp = d.P >> 5, tn = d.N >> 5;
  float *dst = a.ws + ((size_t)c * d.H + h) * d.P * d.N;
  for (int i = wave; i < tp * tn; i += 4) {
    const int pi = i / tn, ni = i - pi * tn;
    const int pc = 32 * pi + (lane & 31), nc = 32 * ni + (lane & 31);
    const f32x16_t acc = mma(f32x16_t{}, kend, [&](int k) { return sm.X[k][pc]; },
                             [&](int k) { return sm.B[k][nc]; });
#pragma unroll
    for (int r = 0; r < 16; ++r)
      dst[(size_t)(32 * pi + acc_row(r, lane)) * d.N + nc] = acc[r];
  }
}

// ------------------------------------------------------------ pass 2: chain
// One thread owns 4 consecutive floats of one head's state.  The loads of the
// next tiles' S_c do not depend on the chain and are issued kAhead tiles early.
constexpr int kCarrySpan = 4 * kThreads;  // floats per workgroup

__global__ __launch_bounds__(kThreads) void chunk_carry_kernel(ChunkArgs a) {
  const Dims d = a.d;
  const size_t PN = (size_t)d.P * d.N;
  const int per_head = (int)((PN + kCarrySpan - 1) / kCarrySpan);
  const int h = blockIdx.x / per_head, part = blockIdx.x % per_head;
  const size_t off = (size_t)part * kCarrySpan + 4 * threadIdx.x;
  if (off >= PN) return;  // PN % 4 == 0
  float *st = a.state + (size_t)h * PN + off;
  float4 hv = *reinterpret_cast<const float4 *>(st);
  const size_t stride = (size_t)d.H * PN;
  float *ws = a.ws + (size_t)h * PN + off;
  constexpr int kAhead = 8;
  float4 sv[kAhead];
  float lam[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    const int c = min(i, a.n_tiles - 1);
    sv[i] = *reinterpret_cast<const float4 *>(ws + c * stride);
    lam[i] = a.lam[(size_t)c * d.H + h];
  }
  for (int c0 = 0; c0 < a.n_tiles; c0 += kAhead) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int c = c0 + i;
      if (c < a.n_tiles) {
        *reinterpret_cast<float4 *>(ws + (size_t)c * stride) = hv;  // h_in(c)
        const float l = lam[i];
        const float4 sc = sv[i];
        // a reset inside the tile drops the old state (no 0 * inf)
        hv = l == 0.f ? sc
                      : make_float4(fmaf(l, hv.x, sc.x), fmaf(l, hv.y, sc.y),
                                    fmaf(l, hv.z, sc.z), fmaf(l, hv.w, sc.w));
        const int cn = min(c + kAhead, a.n_tiles - 1);
        sv[i] = *reinterpret_cast<const float4 *>(ws + (size_t)cn * stride);
        lam[i] = a.lam[(size_t)cn * d.H + h];
      }
    }
  }
  *reinterpret_cast<float4 *>(st) = hv;
}

// ----------------------------------------------------------- pass 3: y, ckpt
struct OutSmem {
  float C[QT][NP];     // C[t][n]
  float B[QT][NP];     // B[s][n]
  float Hs[kMaxP][NP]; // h_in[p][n]
  float X[QT][PP];     // x[s][p]
  float M[QT][MP];     // masked C.B (zero above the diagonal)
  float ecs[QT];       // exp(cs_t), the carried-in state's weight
  float w[QT];
  TileScalars ts;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_output_kernel(ChunkArgs a, ChunkMeta m) {
  __shared__ OutSmem sm;
  const Dims d = a.d;
  const int c = blockIdx.x / d.H, h = blockIdx.x % d.H;
  const int g = h / (d.H / d.G);
  const int tbase = a.t0 + c * QT;
  const int n = min(QT, a.t0 + a.len - tbase);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31;
  const float Dh = a.D[h];
  const int N4 = d.N >> 2, P4 = d.P >> 2;

  float dtv = 0.f;
  if (tid < QT) dtv = load_dt((const T *)a.dt, tbase, n, d.H, h, tid);
  {
    RowTile<T, kMaxN> ct, bt;
    const size_t bc0 = ((size_t)tbase * d.G + g) * d.N;
    ct.load((const T *)a.C + bc0, (size_t)d.G * d.N, n, N4);
    bt.load((const T *)a.B + bc0, (size_t)d.G * d.N, n, N4);
    RowTile<T, kMaxP> xt;
    xt.load((const T *)a.x + ((size_t)tbase * d.H + h) * d.P, (size_t)d.H * d.P, n, P4);
    RowTile<float, kMaxN> ht;  // h_in[p][n]: 64 rows of which P are real
    ht.load(a.ws + ((size_t)c * d.H + h) * d.P * d.N, d.N, d.P, N4);
    if (tid < QT) {
      const double cs = tile_cumsum(tid < n ? dtv : 0.f, a.A[h]);
      sm.ts.dt[tid] = tid < n ? dtv : 0.f;
      sm.ts.cs[tid] = cs;
      sm.ts.seg[tid] = seg_upto(m.rmask[c], tid);
      sm.ecs[tid] = exp_d(cs);
    }
    ct.template store<NP>(&sm.C[0][0], n, QT, N4, One());
    bt.template store<NP>(&sm.B[0][0], n, QT, N4, One());
    xt.template store<PP>(&sm.X[0][0], n, QT, P4, One());
    ht.template store<NP>(&sm.Hs[0][0], d.P, d.P, N4, One());
  }
  __syncthreads();

  const int KN = (d.N + 63) & ~63;  // columns past N are zero
  // masked C.B for the three 32x32 blocks on or below the diagonal; the block
  // above it is zero
  if (wave == 3) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.M[acc_row(r, lane)][32 + l32] = 0.f;
  } else {
    const int ta = wave == 0 ? 0 : 1, sb = wave == 2 ? 1 : 0;
    const int tr = 32 * ta + l32, sr = 32 * sb + l32;
    const f32x16_t acc = mma(f32x16_t{}, KN, [&](int k) { return sm.C[tr][k]; },
                             [&](int k) { return sm.B[sr][k]; });
    const int s = sr;
    const double css = sm.ts.cs[s];
    const float dts = sm.ts.dt[s];
    const int segs = sm.ts.seg[s];
    double cst[16];
    int segt[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * ta + acc_row(r, lane);
      cst[r] = sm.ts.cs[t];
      segt[r] = sm.ts.seg[t];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * ta + acc_row(r, lane);
      // above the diagonal the exponent may overflow: selected away below
      float v = acc[r] * exp_d(cst[r] - css) * dts;
      if (s == t) v += Dh;
      sm.M[t][s] = (s <= t && segt[r] == segs) ? v : 0.f;
    }
  }
  __syncthreads();

  const int tp = d.P >> 5;
  if (wave < 2 * tp) {
    const int ta = wave / tp, pb = wave - ta * tp;
    const int tr = 32 * ta + l32, pc = 32 * pb + l32;
    const f32x16_t yd = mma(f32x16_t{}, QT, [&](int k) { return sm.M[tr][k]; },
                            [&](int k) { return sm.X[k][pc]; });
    const f32x16_t yo = mma(f32x16_t{}, KN, [&](int k) { return sm.C[tr][k]; },
                            [&](int k) { return sm.Hs[pc][k]; });
    T *y = (T *)a.y;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * ta + acc_row(r, lane);
      const float v = sm.ts.seg[t] == 0 ? fmaf(sm.ecs[t], yo[r], yd[r]) : yd[r];
      if (t < n) Io<T>::st(y + ((size_t)(tbase + t) * d.H + h) * d.P + pc, v);
    }
  }

  // checkpoints inside this tile: the state right after token te
  for (int i = 0; i < a.n_ck; ++i) {
    const int te = m.ck_t[i] - tbase;
    if (te < 0 || te >= n) continue;
    __syncthreads();  // previous users of w are done
    const double cse = sm.ts.cs[te];
    const int sege = sm.ts.seg[te];
    if (tid < QT)
      sm.w[tid] = (tid <= te && sm.ts.seg[tid] == sege)
                      ? exp_d(cse - sm.ts.cs[tid]) * sm.ts.dt[tid]
                      : 0.f;
    __syncthreads();
    const float carry = sege == 0 ? sm.ecs[te] : 0.f;
    const int kend = QT;  // w is zero past te
    const int tn = d.N >> 5;
    float *dst = a.ckpt_out + ((size_t)m.ck_idx[i] * d.H + h) * d.P * d.N;
    for (int q = wave; q < tp * tn; q += 4) {
      const int pi = q / tn, ni = q - pi * tn;
      const int pc = 32 * pi + l32, nc = 32 * ni + l32;
      const f32x16_t acc = mma(f32x16_t{}, kend, [&](int k) { return sm.X[k][pc] * sm.w[k]; },
                               [&](int k) { return sm.B[k][nc]; });
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = 32 * pi + acc_row(r, lane);
        float v = acc[r];
        if (sege == 0) v = fmaf(carry, sm.Hs[p][nc], v);
        dst[(size_t)p * d.N + nc] = v;
      }
    }
  }
}

}  // namespace

bool chunk_supported(int io, const Dims &d) {
  (void)io;
  return d.P % 32 == 0 && d.P <= kMaxP && d.N % 32 == 0 && d.N <= kMaxN;
}

size_t chunk_ws_floats(const Dims &d, int64_t L) {
  const int64_t tiles = std::min<int64_t>((L + QT - 1) / QT, kChunkTilesPerLaunch);
  return (size_t)tiles * d.H * d.P * d.N + (size_t)kChunkTilesPerLaunch * d.H;
}

hipError_t launch_chunk(int io, const ChunkArgs &a, const ChunkMeta &m, hipStream_t s) {
  const Dims &d = a.d;
  dim3 block(kThreads);
  dim3 tiles(a.n_tiles * d.H);
  const size_t PN = (size_t)d.P * d.N;
  dim3 carry((unsigned)(d.H * ((PN + kCarrySpan - 1) / kCarrySpan)));
  if (io == kBF16) {
    hipLaunchKernelGGL((chunk_state_kernel<bf16_t>), tiles, block, 0, s, a, m);
    hipLaunchKernelGGL(chunk_carry_kernel, carry, block, 0, s, a);
    hipLaunchKernelGGL((chunk_output_kernel<bf16_t>), tiles, block, 0, s, a, m);
  } else {
    hipLaunchKernelGGL((chunk_state_kernel<float>), tiles, block, 0, s, a, m);
    hipLaunchKernelGGL(chunk_carry_kernel, carry, block, 0, s, a);
    hipLaunchKernelGGL((chunk_output_kernel<float>), tiles, block, 0, s, a, m);
  }
  return hipGetLastError();
}

}  // namespace ssm
