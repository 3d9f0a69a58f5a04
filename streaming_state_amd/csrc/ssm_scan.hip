// ssm_scan.hip -- chunk scan, recurrent form: one workgroup per (segment,
// head, 64-row tile) carries the fp32 state in registers through the
// segment's tokens in order.  A segment is a run of tokens between resets, so
// segments are independent and run in parallel; the state carried into the
// chunk feeds only the first segment.
//
// Tokens are staged through LDS in tiles of kTT (x rows, dt, B, C converted to
// fp32), outputs are collected in LDS and written back as coalesced rows.
// Checkpoints (the state right after a given token) are written from
// registers as the loop passes them.
#include "ssm_device.h"

namespace ssm {

namespace {
constexpr int kTT = 32;

__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

template <typename T>
__global__ __launch_bounds__(kThreads) void scan_rec_kernel(ScanArgs a, ScanMeta m) {
  __shared__ __align__(16) float s_x[kTT][kRows];
  __shared__ __align__(16) float s_B[kTT][kMaxN];
  __shared__ __align__(16) float s_C[kTT][kMaxN];
  __shared__ __align__(16) float s_y[kTT][kRows];
  __shared__ float s_dt[kTT];
  const Tile tl;
  const Dims d = a.d;
  int bid = blockIdx.x;
  const int pt = bid % d.PT;
  bid /= d.PT;
  const int h = bid % d.H;
  const int sidx = bid / d.H;
  const ScanSeg sg = m.seg[sidx];
  const int g = h / (d.H / d.G);
  const int prow0 = pt * kRows;
  const bool colok = 4 * tl.c < d.N;
  const size_t PN = (size_t)d.P * d.N;
  const size_t tile_off = (size_t)prow0 * d.N + 4 * tl.c;
  const float Ah = a.A[h], Dh = a.D[h];
  const T *x = (const T *)a.x, *dt = (const T *)a.dt, *Bp = (const T *)a.B, *Cp = (const T *)a.C;

  float4 hv[8];
  {
    const float *st = a.state + (size_t)h * PN + tile_off;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = sg.init && colok && (prow0 + tl.row(i) < d.P);
      hv[i] = ok ? *reinterpret_cast<const float4 *>(st + (size_t)tl.row(i) * d.N) : zero4();
    }
  }
  int ck = 0;
  while (ck < a.n_ck && m.ck_t[ck] < sg.t0) ++ck;

  for (int tb = sg.t0; tb < sg.t1; tb += kTT) {
    const int nt = min(kTT, sg.t1 - tb);
    __syncthreads();
    for (int i = threadIdx.x; i < nt * kRows; i += kThreads) {
      const int j = i / kRows, r = i % kRows;
      s_x[j][r] = prow0 + r < d.P ? Io<T>::ld(x + ((size_t)(tb + j) * d.H + h) * d.P + prow0 + r)
                                  : 0.f;
    }
    for (int i = threadIdx.x; i < nt * d.N; i += kThreads) {
      const int j = i / d.N, n = i % d.N;
      const size_t off = ((size_t)(tb + j) * d.G + g) * d.N + n;
      s_B[j][n] = Io<T>::ld(Bp + off);
      s_C[j][n] = Io<T>::ld(Cp + off);
    }
    for (int j = threadIdx.x; j < nt; j += kThreads)
      s_dt[j] = Io<T>::ld(dt + (size_t)(tb + j) * d.H + h);
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
      const float dtj = s_dt[j];
      const float dA = expf(dtj * Ah);
      const float4 Bv = colok ? *reinterpret_cast<const float4 *>(&s_B[j][4 * tl.c]) : zero4();
      const float4 Cv = colok ? *reinterpret_cast<const float4 *>(&s_C[j][4 * tl.c]) : zero4();
      float part[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hv[i] = fma4(dA, hv[i], dtj * s_x[j][tl.row(i)], Bv);
        part[i] = dot4(hv[i], Cv);
      }
      const float yv = reduce8(part, tl.lane);
      if (tl.reduced_writer()) {
        const int r = tl.reduced_row();
        s_y[j][r] = yv + Dh * s_x[j][r];
      }
      const int t = tb + j;
      while (ck < a.n_ck && m.ck_t[ck] == t) {
        float *dst = a.ckpt_out + ((size_t)m.ck_idx[ck] * d.H + h) * PN + tile_off;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (colok && prow0 + tl.row(i) < d.P)
            *reinterpret_cast<float4 *>(dst + (size_t)tl.row(i) * d.N) = hv[i];
        ++ck;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt * kRows; i += kThreads) {
      const int j = i / kRows, r = i % kRows;
      if (prow0 + r < d.P)
        Io<T>::st((T *)a.y + ((size_t)(tb + j) * d.H + h) * d.P + prow0 + r, s_y[j][r]);
    }
  }

  if (sg.final) {
    float *dst = (sg.final == 1 ? a.state : a.workspace) + (size_t)h * PN + tile_off;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (colok && prow0 + tl.row(i) < d.P)
        *reinterpret_cast<float4 *>(dst + (size_t)tl.row(i) * d.N) = hv[i];
  }
}
}  // namespace

hipError_t launch_scan(int io, const ScanArgs &a, const ScanMeta &m, hipStream_t s) {
  dim3 grid(a.n_seg * a.d.H * a.d.PT), block(kThreads);
  if (io == kBF16)
    hipLaunchKernelGGL(scan_rec_kernel<bf16_t>, grid, block, 0, s, a, m);
  else
    hipLaunchKernelGGL(scan_rec_kernel<float>, grid, block, 0, s, a, m);
  return hipGetLastError();
}

}  // namespace ssm
