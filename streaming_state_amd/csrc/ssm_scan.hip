// ssm_scan.hip -- chunk scan, recurrent form: one workgroup per (segment,
// head, row tile) carries the fp32 state in registers through the segment's
// tokens in order.  A segment is a run of tokens between resets, so segments
// are independent and run in parallel; the state carried into the chunk feeds
// only the first segment.  This form serves fp32 inputs and shapes the MFMA
// form does not cover; it performs the recurrence in the order the oracle does.
//
// Tokens are staged through LDS in tiles of kTT (x rows, dt, the decay
// exp(dt A), B and C converted to fp32); outputs are collected in LDS and
// written back as coalesced rows.  Checkpoints (the state right after a given
// token) are written from registers as the loop passes them.  The row tile
// (8R rows of the head) is picked by the host so that short, few-head chunks
// still occupy many workgroups.
#include "ssm_device.h"

namespace ssm {

namespace {
constexpr int kTT = 32;

__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

template <typename T, int R>
__global__ __launch_bounds__(kThreads) void scan_rec_kernel(ScanArgs a, ScanMeta m) {
  constexpr int kTileRows = 8 * R;
  __shared__ __align__(16) float s_x[kTT][kTileRows];
  __shared__ __align__(16) float s_B[kTT][kMaxN];
  __shared__ __align__(16) float s_C[kTT][kMaxN];
  __shared__ __align__(16) float s_y[kTT][kTileRows];
  __shared__ float s_dt[kTT], s_dA[kTT];
  const TileR<R> tl;
  const Dims d = a.d;
  const int pt_n = (d.P + kTileRows - 1) / kTileRows;
  int bid = blockIdx.x;
  const int pt = bid % pt_n;
  bid /= pt_n;
  const int h = bid % d.H;
  const int sidx = bid / d.H;
  const ScanSeg sg = m.seg[sidx];
  const int g = h / (d.H / d.G);
  const int prow0 = pt * kTileRows;
  const bool colok = 4 * tl.c < d.N;
  const size_t PN = (size_t)d.P * d.N;
  const size_t tile_off = (size_t)prow0 * d.N + 4 * tl.c;
  const float Ah = a.A[h], Dh = a.D[h];
  const T *x = (const T *)a.x, *dt = (const T *)a.dt, *Bp = (const T *)a.B, *Cp = (const T *)a.C;

  float *seg_state = a.state + (size_t)sg.slot * d.H * PN;
  float4 hv[R];
  {
    const float *st = seg_state + (size_t)h * PN + tile_off;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const bool ok = sg.init && colok && (prow0 + tl.row(i) < d.P);
      hv[i] = ok ? *reinterpret_cast<const float4 *>(st + (size_t)tl.row(i) * d.N) : zero4();
    }
  }
  // next checkpoint at or after the segment start, kept in a register
  int ck = 0;
  while (ck < a.n_ck && m.ck_t[ck] < sg.t0) ++ck;
  int ck_t = ck < a.n_ck ? m.ck_t[ck] : 0x7fffffff;

  // Staging: the next tile's inputs are loaded into registers while the
  // current tile's tokens run, then written to LDS.  B and C rows are read four
  // elements at a time (N % 4 == 0 and their alignment are checked on the
  // host); x rows element-wise (any P).
  constexpr int kBC = kTT * kMaxN / 4 / kThreads;     // float4 chunks per thread (4)
  constexpr int kX = kTT * kTileRows / kThreads;       // x elements per thread (R)
  const int N4 = d.N >> 2;
  float4 pb[kBC], pc[kBC];
  float px[kX > 0 ? kX : 1];
  float pdt = 0.f;
  auto load_tile = [&](int tb, int nt) {
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
      const int q = threadIdx.x + kThreads * k;
      pb[k] = pc[k] = zero4();
      if (q < nt * N4) {
        const int j = q / N4, c4 = q - j * N4;
        const size_t off = ((size_t)(tb + j) * d.G + g) * d.N + 4 * c4;
        pb[k] = Io<T>::ld4(Bp + off);
        pc[k] = Io<T>::ld4(Cp + off);
      }
    }
#pragma unroll
    for (int k = 0; k < kX; ++k) {
      const int q = threadIdx.x + kThreads * k;
      const int j = q / kTileRows, r = q % kTileRows;
      px[k] = (j < nt && prow0 + r < d.P)
                  ? Io<T>::ld(x + ((size_t)(tb + j) * d.H + h) * d.P + prow0 + r)
                  : 0.f;
    }
    if (threadIdx.x < nt) pdt = Io<T>::ld(dt + (size_t)(tb + threadIdx.x) * d.H + h);
  };
  auto store_tile = [&](int nt) {
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
      const int q = threadIdx.x + kThreads * k;
      if (q < nt * N4) {
        const int j = q / N4, c4 = q - j * N4;
        *reinterpret_cast<float4 *>(&s_B[j][4 * c4]) = pb[k];
        *reinterpret_cast<float4 *>(&s_C[j][4 * c4]) = pc[k];
      }
    }
#pragma unroll
    for (int k = 0; k < kX; ++k) {
      const int q = threadIdx.x + kThreads * k;
      s_x[q / kTileRows][q % kTileRows] = px[k];
    }
    if (threadIdx.x < nt) {
      s_dt[threadIdx.x] = pdt;
      s_dA[threadIdx.x] = expf(pdt * Ah);
    }
  };

  if (sg.t0 < sg.t1) load_tile(sg.t0, min(kTT, sg.t1 - sg.t0));
  for (int tb = sg.t0; tb < sg.t1; tb += kTT) {
    const int nt = min(kTT, sg.t1 - tb);
    __syncthreads();  // the previous tile's readers are done
    store_tile(nt);
    __syncthreads();
    if (tb + kTT < sg.t1) load_tile(tb + kTT, min(kTT, sg.t1 - tb - kTT));  // in flight

    for (int j = 0; j < nt; ++j) {
      const float dtj = s_dt[j];
      const float dA = s_dA[j];
      const float4 Bv = colok ? *reinterpret_cast<const float4 *>(&s_B[j][4 * tl.c]) : zero4();
      const float4 Cv = colok ? *reinterpret_cast<const float4 *>(&s_C[j][4 * tl.c]) : zero4();
      float part[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        hv[i] = fma4(dA, hv[i], dtj * s_x[j][tl.row(i)], Bv);
        part[i] = sum32_dpp(dot4(hv[i], Cv));
      }
      if ((tl.lane & 31) == 31) {  // holds the totals of this lane's rows
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int r = tl.row(i);
          s_y[j][r] = part[i] + Dh * s_x[j][r];
        }
      }
      const int t = tb + j;
      while (t == ck_t) {
        float *dst = a.ckpt_out + ((size_t)m.ck_idx[ck] * d.H + h) * PN + tile_off;
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (colok && prow0 + tl.row(i) < d.P)
            *reinterpret_cast<float4 *>(dst + (size_t)tl.row(i) * d.N) = hv[i];
        ++ck;
        ck_t = ck < a.n_ck ? m.ck_t[ck] : 0x7fffffff;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt * kTileRows; i += kThreads) {
      const int j = i / kTileRows, r = i % kTileRows;
      if (prow0 + r < d.P)
        Io<T>::st((T *)a.y + ((size_t)(tb + j) * d.H + h) * d.P + prow0 + r, s_y[j][r]);
    }
  }

  if (sg.final) {
    float *dst = (sg.final == 1 ? seg_state : a.workspace) + (size_t)h * PN + tile_off;
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (colok && prow0 + tl.row(i) < d.P)
        *reinterpret_cast<float4 *>(dst + (size_t)tl.row(i) * d.N) = hv[i];
  }
}

template <int R>
hipError_t launch_rec(int io, const ScanArgs &a, const ScanMeta &m, hipStream_t s) {
  const int pt_n = (a.d.P + 8 * R - 1) / (8 * R);
  dim3 grid(a.n_seg * a.d.H * pt_n), block(kThreads);
  if (io == kBF16)
    hipLaunchKernelGGL((scan_rec_kernel<bf16_t, R>), grid, block, 0, s, a, m);
  else
    hipLaunchKernelGGL((scan_rec_kernel<float, R>), grid, block, 0, s, a, m);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_scan(int io, const ScanArgs &a, const ScanMeta &m, hipStream_t s) {
  // widest row tile that still gives every CU a couple of workgroups
  const int units = a.n_seg * a.d.H;
  if (units * ((a.d.P + 63) / 64) >= 512) return launch_rec<8>(io, a, m, s);
  if (units * ((a.d.P + 31) / 32) >= 512) return launch_rec<4>(io, a, m, s);
  return launch_rec<2>(io, a, m, s);
}

}  // namespace ssm
