// ssm_decode.hip -- gfx950 batched decode: one token for each of a batch of
// slots, the fp32 state updated in place.
//
// A workgroup of kDecodeTiles x 256 threads owns kDecodeTiles (batch entry,
// head, 8R-row) tiles of the state, held in registers as R float4 per thread
// (TileR in ssm_device.h): one pass of 128-bit nontemporal loads, the update,
// one pass of 128-bit nontemporal stores, and the output row totals.
#include "ssm_device.h"

namespace ssm {

static __device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// ===========================================================================
// decode: h <- exp(dt A) h + dt x B^T ; y = h C + D x, one token per slot
// ===========================================================================
// Decode tiles: R float4 rows per thread (a 256-thread tile covers 8R state
// rows of one head) and kDecodeTiles consecutive tiles of one head per
// workgroup.  Measured on MI355X at P = 64, N = 128 with every load issued
// before the first store: 2 rows x 4 tiles (1024 threads, one head per
// workgroup) 6.36 TB/s; 4 x 2, 8 x 1, 4 x 1 and 2 x 2 within 1-2% below.
constexpr int kDecodeR = 2;
constexpr int kDecodeTiles = 4;

// Grid (tile groups, H, entries): workgroup (x, h, k) owns tiles
// pt = TW x + 0..TW-1 of head h of entry k.  kFull: P is a multiple of the
// tile height and N = 128, so every lane owns rows and columns and no access
// needs a per-lane predicate (a separate instantiation).
template <typename T, int R, int TW, bool kFull>
__global__ __launch_bounds__(kThreads *TW) void decode_kernel(DecodeArgs a, DecodeMeta m) {
  const TileR<R> tl;
  const Dims d = a.d;
  constexpr int kTileRows = 8 * R;
  const int pt_n = (d.P + kTileRows - 1) / kTileRows;
  const int pt = blockIdx.x * TW + __builtin_amdgcn_readfirstlane((int)threadIdx.x / kThreads);
  if (pt >= pt_n) return;  // whole waves; no barriers below: tiles are independent
  const int h = blockIdx.y, e = blockIdx.z;
  const uint32_t sr = m.slot_rst[e];
  const int slot = (int)(sr & ~kDecodeReset);
  const bool rst = (sr & kDecodeReset) != 0;
  const int g = d.G == 1 ? 0 : h / (d.H / d.G);
  const int N = kFull ? 4 * 32 : d.N;
  const int prow0 = pt * kTileRows;
  const bool colok = kFull || 4 * tl.c < N;

  float *st = a.state + (((size_t)slot * d.H + h) * d.P + prow0) * N + 4 * tl.c;
  // state first: the only large read, issued before anything else (a reset
  // slot is not read: the branch is uniform over the workgroup)
  float4 hv[R];
  if (kFull) {
    if (!rst) {
#pragma unroll
      for (int i = 0; i < R; ++i) hv[i] = nt_load4(st + (size_t)tl.row(i) * N);
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) hv[i] = zero4();
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const bool ok = colok && (prow0 + tl.row(i) < d.P) && !rst;
      hv[i] = ok ? nt_load4(st + (size_t)tl.row(i) * N) : zero4();
    }
  }
  // then every input, all before the first store: on gfx9 a wait for a load
  // also waits for the stores issued before it
  const T *x = (const T *)a.x + ((size_t)e * d.H + h) * d.P + prow0;
  const int r = tl.reduced_row();
  const bool rok = kFull || prow0 + r < d.P;
  float xr[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    xr[i] = (kFull || prow0 + tl.row(i) < d.P) ? Io<T>::ld(x + tl.row(i)) : 0.f;
  const float xo = rok ? Io<T>::ld(x + r) : 0.f;
  const float dt = Io<T>::ld((const T *)a.dt + (size_t)e * d.H + h);
  const float dA = expf(dt * a.A[h]);
  const float Dh = a.D[h];
  float4 Bv = zero4(), Cv = zero4();
  if (colok) {
    Bv = Io<T>::ld4((const T *)a.B + ((size_t)e * d.G + g) * N + 4 * tl.c);
    Cv = Io<T>::ld4((const T *)a.C + ((size_t)e * d.G + g) * N + 4 * tl.c);
  }
  float part[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const bool rowok = kFull || prow0 + tl.row(i) < d.P;
    hv[i] = fma4(dA, hv[i], dt * xr[i], Bv);
    if (rowok && colok) nt_store4(st + (size_t)tl.row(i) * N, hv[i]);
    part[i] = dot4(hv[i], Cv);
  }
  const float yv = row_totals<R>(part, tl.lane);
  if (tl.reduced_writer() && rok)
    Io<T>::st((T *)a.y + ((size_t)e * d.H + h) * d.P + prow0 + r, yv + Dh * xo);
}

hipError_t launch_decode(int io, const DecodeArgs &a, const DecodeMeta &m, hipStream_t s) {
  constexpr int kTileRows = 8 * kDecodeR;
  const int pt_n = (a.d.P + kTileRows - 1) / kTileRows;
  dim3 grid((pt_n + kDecodeTiles - 1) / kDecodeTiles, a.d.H, a.n), block(kThreads * kDecodeTiles);
  const bool full = a.d.P % kTileRows == 0 && a.d.N == 4 * 32;
  if (io == kBF16) {
    if (full)
      hipLaunchKernelGGL((decode_kernel<bf16_t, kDecodeR, kDecodeTiles, true>), grid, block, 0, s, a, m);
    else
      hipLaunchKernelGGL((decode_kernel<bf16_t, kDecodeR, kDecodeTiles, false>), grid, block, 0, s, a, m);
  } else {
    if (full)
      hipLaunchKernelGGL((decode_kernel<float, kDecodeR, kDecodeTiles, true>), grid, block, 0, s, a, m);
    else
      hipLaunchKernelGGL((decode_kernel<float, kDecodeR, kDecodeTiles, false>), grid, block, 0, s, a, m);
  }
  return hipGetLastError();
}

}  // namespace ssm
