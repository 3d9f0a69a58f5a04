// ssm_ssd.hip -- chunk scan, SSD (matrix) form on MFMA, for bf16 inputs with
// head dim P = 64 and state size N = 128.
//
// Within a block of Q = 64 tokens the recurrence is a pair of dense
// contractions ("Separate Mamba-2 algebra from kernel behavior": the matrix
// view for prefill, the recurrent view for decode).  With cs_t the running sum
// of dt*A inside the block:
//   Y_diag[t,p] = sum_{s<=t} (C_t.B_s) exp(cs_t - cs_s) dt_s x[s,p]      (G1, G2)
//   Y_off [t,p] = exp(cs_t) sum_n C[t,n] h_prev[p,n]                     (G4)
//   h_new[p,n]  = exp(cs_end) h_prev[p,n]
//               + sum_s exp(cs_end - cs_s) dt_s x[s,p] B[s,n]            (G3)
//   y = Y_diag + Y_off + D x
// One workgroup (8 waves) owns one (segment, head): a segment is a run of
// tokens between resets, so it starts from the carried-in state or from zero
// and no reset falls inside it.  Roles, in the two compute phases of a block:
//   waves 0-3  own the four 32 x 32 tiles of y: G4, then G2 and the epilogue;
//   waves 4-7  own the fp32 state h^T[n,p] in MFMA accumulators for the whole
//              segment (wave 4+i: n in [32i, +32), both p tiles); waves 4-6
//              first compute the three tiles of C.B on or below the diagonal
//              (G1) and mask them into M, then all four run G3 (beside G2),
//              the checkpoints and the bf16 copy of h that feeds G4.
// All eight stage the next block's inputs.  Two workgroups share a CU, so each
// SIMD holds four waves.  Blocks end early at checkpoint tokens so the
// post-token state can be written from the accumulators.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Operand lane layout (A: 32 x 16, B: 16 x 32):
// lane l supplies row/column l%32 and K indices 8*(l/32) .. +7; accumulator
// register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// Operands whose K runs along an LDS row are read as 16-byte segments; those
// whose K runs down the rows of a row-major tile (B^T for G3, x for G2 and
// G3) are read with the LDS transposing load ds_read_b64_tr_b16, so every
// input is staged once, row-major, straight from coalesced global loads.
#include "ssm_device.h"

namespace ssm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kSsdThreads = 512;  // 8 waves
constexpr int Q = 64;    // tokens per block
constexpr int SP = 64;   // head dim
constexpr int SN = 128;  // state size

// LDS layouts.  Rows are unpadded; 16-byte chunks are XOR-swizzled by row so
// that both access patterns of a tile are free of bank conflicts.  The LDS
// serves 256 bytes per cycle to 8- and 16-byte accesses: a 16-byte access is
// conflict-free when each group of 16 lanes touches 16 distinct 16-byte slots
// modulo 256 bytes, an 8-byte access (also the transposing read) when each
// group of 32 lanes touches 32 distinct 8-byte slots (measured on gfx950):
//  - 256-byte rows (C, B, h: 128 bf16): chunk ^ f(row), f(r) = (r%4)*4 + (r/4)%4.
//    A 16-row read of one chunk hits 16 distinct chunks (f is a bijection of
//    0..15); a transposing read covers rows r..r+3 (r % 4 == 0) x 4 chunks of
//    an aligned quad, and f moves each row's quad to a different quad.
//  - 128-byte rows (x, w*x: 64 bf16) are only read transposed: chunk ^ 4 on
//    rows with bit 1 set separates rows r and r+2, which share banks.
//  - 128-byte rows of M^T (read as 16-row segments): chunk ^ ((row / 2) % 8).
__device__ __forceinline__ int sw_n(int row, int col) {  // element index, 128-wide rows
  const int f = ((row & 3) << 2) | ((row >> 2) & 3);
  return row * SN + ((((col >> 3) ^ f)) << 3) + (col & 7);
}
__device__ __forceinline__ int sw_x(int row, int col) {  // 64-wide rows, transposed reads
  return row * SP + ((((col >> 3) ^ ((row & 2) << 1))) << 3) + (col & 7);
}
__device__ __forceinline__ int sw_m(int row, int col) {  // 64-wide rows, row reads
  return row * Q + ((((col >> 3) ^ ((row >> 1) & 7))) << 3) + (col & 7);
}

// 72 KiB: two workgroups per CU.
struct Smem {
  alignas(16) bf16_t C[Q * SN];   // C[t][n]
  alignas(16) bf16_t B[Q * SN];   // B[s][n]
  alignas(16) bf16_t HT[SP * SN]; // bf16 copy of h_prev[p][n]
  alignas(16) bf16_t X[Q * SP];   // x[s][p]
  alignas(16) bf16_t XW[Q * SP];  // w_s x[s][p]
  alignas(16) bf16_t MT[Q * Q];   // M[t][s] (masked C.B with D on the diagonal)
  float csl[Q], ecs[Q], dt[Q];  // running sum of dt*A times log2(e); exp of it; dt
  float lam;
};
static_assert(2 * sizeof(Smem) <= 160 * 1024, "two workgroups per CU");

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// LDS vector accesses with their alignment stated: without it the compiler
// splits a 16-byte store into 4-byte pairs, which conflict on the banks where
// one 16-byte store would not.
__device__ __forceinline__ bf16x8_t lds8(const bf16_t *p) {
  return *static_cast<const bf16x8_t *>(__builtin_assume_aligned(p, 16));
}
__device__ __forceinline__ uint4 lds_ld16(const bf16_t *p) {
  return *static_cast<const uint4 *>(__builtin_assume_aligned(p, 16));
}
__device__ __forceinline__ void lds_st16(bf16_t *p, uint4 v) {
  *static_cast<uint4 *>(__builtin_assume_aligned(p, 16)) = v;
}
__device__ __forceinline__ void lds_st8(bf16_t *p, uint2 v) {
  *static_cast<uint2 *>(__builtin_assume_aligned(p, 8)) = v;
}
__device__ __forceinline__ void lds_st4(bf16_t *p, uint32_t v) {
  *static_cast<uint32_t *>(__builtin_assume_aligned(p, 4)) = v;
}
__device__ __forceinline__ s16x4_t ldtr4(const bf16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t *)(p));
}
// An MFMA operand whose 8 K values run down rows k0..k0+7 of a row-major tile,
// at column col0 + l%16 of the lane's 16-lane group (col0 is the group's first
// column): two transposing reads of 4 rows each.  Lane l of a 16-lane group
// supplies row k0 + 4r + (l%16)/4, columns col0 + 4(l%4) .. +3; the hardware
// hands lane j element j%4 of the segments of lanes j/4, 4 + j/4, 8 + j/4 and
// 12 + j/4, i.e. column col0 + j of rows k0 + 4r .. +3.
// For K rows k0 = 16k + 8(l/32), the swizzles below do not depend on k, so a
// lane's two addresses are fixed offsets (computed once, by tr_off) plus
// 16k whole rows.
struct TrOff {
  int o0, o1;
};
template <typename SW>
__device__ __forceinline__ TrOff tr_off(int col0, int lane, SW sw) {
  const int rr = (lane & 15) >> 2, cc = col0 + 4 * (lane & 3), hk = 8 * (lane >> 5);
  return TrOff{sw(hk + rr, cc), sw(hk + 4 + rr, cc)};
}
__device__ __forceinline__ bf16x8_t ldtr8(const bf16_t *tile, TrOff o) {
  const s16x4_t lo = ldtr4(tile + o.o0);
  const s16x4_t hi = ldtr4(tile + o.o1);
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}
struct SwN {
  __device__ __forceinline__ int operator()(int r, int c) const { return sw_n(r, c); }
};
struct SwX {
  __device__ __forceinline__ int operator()(int r, int c) const { return sw_x(r, c); }
};

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes a wave with pending global stores (y, checkpoints) wait
// for all its outstanding loads too -- including the next block's prefetch.
// No wave reads another wave's global writes inside this kernel.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
// row of accumulator register r for lane half hi (within a 32 x 32 tile)
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  uint2 v;
  v.x = pack2_bf16(a, b);
  v.y = pack2_bf16(c, d);
  return v;
}

// h^T accumulator tiles (n in [32 nt, +32), p tile j = 0, 1) <-> a [P][N] fp32
// state.  Register r of lane l of tile j is h[p = 32j + l%32][n = 32nt +
// acc_row(r)], so four consecutive registers are four consecutive n.
__device__ __forceinline__ void state_load(f32x16_t hacc[2], const float *src, int nt, int l32,
                                           int hi) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 32 * j + l32, n = 32 * nt + 8 * q + 4 * hi;
      const float4 v = *reinterpret_cast<const float4 *>(src + (size_t)p * SN + n);
      hacc[j][4 * q + 0] = v.x;
      hacc[j][4 * q + 1] = v.y;
      hacc[j][4 * q + 2] = v.z;
      hacc[j][4 * q + 3] = v.w;
    }
}
__device__ __forceinline__ void state_store(const f32x16_t hacc[2], float *dst, int nt, int l32,
                                            int hi) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 32 * j + l32, n = 32 * nt + 8 * q + 4 * hi;
      *reinterpret_cast<float4 *>(dst + (size_t)p * SN + n) =
          make_float4(hacc[j][4 * q], hacc[j][4 * q + 1], hacc[j][4 * q + 2], hacc[j][4 * q + 3]);
    }
}
__device__ __forceinline__ void state_to_lds(const f32x16_t hacc[2], bf16_t *HT, int nt, int l32,
                                             int hi) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 32 * j + l32, n = 32 * nt + 8 * q + 4 * hi;
      lds_st8(HT + sw_n(p, n),
              pack4(hacc[j][4 * q], hacc[j][4 * q + 1], hacc[j][4 * q + 2], hacc[j][4 * q + 3]));
    }
}

// One block's global inputs, held in registers between the load and the LDS
// write so the loads overlap the previous block's compute.  Thread q takes
// 16-byte chunks q and q + 512 of the C and B tiles (16 chunks per row) and
// chunk q of the x tile (8 per row): every wave reads whole rows, so the loads
// are coalesced.  Every lane of every wave also reads the dt of token `lane`
// (the running sums are computed in each wave).  Loads are unconditional (rows
// past the block end re-read its last row) so nothing waits until the values
// are written to LDS; stage_store zeroes those rows.
struct Staged {
  uint4 c[2], b[2], x;
  uint32_t dt;  // raw bf16 bits
};

__device__ __forceinline__ void stage_load(Staged &st, const ScanArgs &a, int t0, int len, int h,
                                           int g, int tid, int lane) {
  const Dims &d = a.d;
  const bf16_t *Cg = (const bf16_t *)a.C, *Bg = (const bf16_t *)a.B;
  const bf16_t *xg = (const bf16_t *)a.x, *dtg = (const bf16_t *)a.dt;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + kSsdThreads * k;
    const int row = t0 + min(q >> 4, len - 1);
    const size_t off = ((size_t)row * d.G + g) * SN + (q & 15) * 8;
    st.c[k] = *reinterpret_cast<const uint4 *>(Cg + off);
    st.b[k] = *reinterpret_cast<const uint4 *>(Bg + off);
  }
  {
    const int row = t0 + min(tid >> 3, len - 1);
    st.x = *reinterpret_cast<const uint4 *>(xg + ((size_t)row * d.H + h) * SP + (tid & 7) * 8);
  }
  st.dt = dtg[(size_t)(t0 + min(lane, len - 1)) * d.H + h];
}

__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
  return ok ? v : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ uint32_t scale2(uint32_t v, float w) {
  return pack2_bf16(__uint_as_float(v << 16) * w, __uint_as_float(v & 0xffff0000u) * w);
}

// Write a staged block to LDS, with its running sums: cs (inclusive sum of
// dt*A), exp(cs), the G3 weights w_s = exp(cs_end - cs_s) dt_s (applied to x
// rows here) and lam = exp(cs_end).  Every wave computes the sums (one token
// per lane); wave 0 publishes them.
__device__ __forceinline__ void stage_store(const Staged &st, Smem &sm, int len, int tid,
                                            int lane, int wave, float Ah) {
  const float dtv = lane < len ? __uint_as_float(st.dt << 16) : 0.f;
  const float v = scan64(dtv * Ah);
  // rows past len add nothing, so lane 63 holds the block's total
  const float end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  const float w = __expf(end - v) * dtv;
  if (wave == 0) {
    sm.csl[lane] = v * 1.4426950408889634f;
    sm.ecs[lane] = __expf(v);
    sm.dt[lane] = dtv;
    if (lane == 0) sm.lam = __expf(end);
  }
  const bool full = len == Q;  // otherwise rows past len are zeroed
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + kSsdThreads * k;
    const int row = q >> 4, col = (q & 15) * 8;
    const bool ok = full || row < len;
    lds_st16(sm.C + sw_n(row, col), full ? st.c[k] : keep_if(ok, st.c[k]));
    lds_st16(sm.B + sw_n(row, col), full ? st.b[k] : keep_if(ok, st.b[k]));
  }
  {
    const int row = tid >> 3, col = (tid & 7) * 8;
    const uint4 xv = full ? st.x : keep_if(row < len, st.x);
    const float wr = __shfl(w, row);  // zero past len
    lds_st16(sm.X + sw_x(row, col), xv);
    lds_st16(sm.XW + sw_x(row, col),
             make_uint4(scale2(xv.x, wr), scale2(xv.y, wr), scale2(xv.z, wr), scale2(xv.w, wr)));
  }
}

// end (exclusive) of the block starting at t0: Q tokens, the segment end, or
// just past the next checkpoint token
__device__ __forceinline__ int block_end(const ScanArgs &a, const ScanMeta &m, int t0, int seg_end,
                                         int ck) {
  int t1 = min(t0 + Q, seg_end);
  if (ck < a.n_ck && m.ck_t[ck] < t1) t1 = m.ck_t[ck] + 1;
  return t1;
}

__global__ __launch_bounds__(kSsdThreads, 4) void scan_ssd_kernel(ScanArgs a, ScanMeta m) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const Dims d = a.d;
  const int h = blockIdx.x % d.H;
  const int sidx = blockIdx.x / d.H;
  const ScanSeg sg = m.seg[sidx];
  const int g = h / (d.H / d.G);
  const float Ah = a.A[h], Dh = a.D[h];
  bf16_t *yg = (bf16_t *)a.y;
  const size_t PN = (size_t)SP * SN;

  // Accumulators by role: waves 4-7 keep their state tiles (n in [32 nt, +32),
  // both p tiles) in acc[0..1] for the whole segment, and waves 4-6 build a
  // masked (C.B)^T tile in acc[2]; waves 0-3 build their y tile in acc[0].
  const bool swave = wave >= 4;
  const int nt = wave & 3;
  f32x16_t acc[3];
  f32x16_t *hacc = acc;
  f32x16_t &tile = acc[0], &mt = acc[2];
  float *seg_state = a.state + (size_t)sg.slot * d.H * PN;
  bool have_h = sg.init != 0;
  acc[0] = zero16();
  acc[1] = zero16();
  if (have_h && swave) {
    state_load(hacc, seg_state + (size_t)h * PN, nt, l32, hi);
    state_to_lds(hacc, sm.HT, nt, l32, hi);
  }
  int ck = 0;
  while (ck < a.n_ck && m.ck_t[ck] < sg.t0) ++ck;

  // waves 0-3: y tile rows t in [32 ta, +32), columns p in [32 pb, +32);
  // waves 4-6: (C.B)^T tile with s in [32 si, +32), t in [32 gt, +32), s <= t
  const int ta = (wave >> 1) & 1, pb = wave & 1;
  const bool g1 = wave >= 4 && wave < 7;
  const int si = wave == 6 ? 1 : 0, gt = wave == 4 ? 0 : 1;

  Staged st;
  int t0 = sg.t0;
  int t1 = block_end(a, m, t0, sg.t1, ck);
  stage_load(st, a, t0, t1 - t0, h, g, tid, lane);
  stage_store(st, sm, t1 - t0, tid, lane, wave, Ah);

  while (true) {
    // The lane indices are re-derived each block through an opaque zero:
    // otherwise the compiler hoists every swizzled LDS address out of the loop
    // and keeps dozens of them in registers, which spills.
    int opq = 0;
    asm volatile("" : "+v"(opq));
    const int tid = threadIdx.x + opq, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int len = t1 - t0;
    // checkpoints at t1 - 1 are consumed by this block
    int ck_next = ck;
    while (ck_next < a.n_ck && m.ck_t[ck_next] == t1 - 1) ++ck_next;
    const int n0 = t1, n1 = n0 < sg.t1 ? block_end(a, m, n0, sg.t1, ck_next) : n0;
    lds_barrier();  // [A] this block's inputs and running sums are in LDS

    if (n1 > n0) stage_load(st, a, n0, n1 - n0, h, g, tid, lane);  // next block, in flight

    if (!swave) {
      // ---- G4: C h_prev^T tile (ta, pb), rows scaled by exp(cs_t)
      tile = zero16();
      if (have_h) {
        const int tr = 32 * ta + l32, pr = 32 * pb + l32;
#pragma unroll 4
        for (int k = 0; k < SN / 16; ++k) {
          const int col = 16 * k + 8 * hi;
          tile = mfma(lds8(sm.C + sw_n(tr, col)), lds8(sm.HT + sw_n(pr, col)), tile);
        }
        const float *eb = sm.ecs + 32 * ta + 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r) tile[r] *= eb[8 * (r >> 2) + (r & 3)];
      }
    } else if (g1) {
      // ---- G1: (C.B)^T tile (si, gt), masked into M
      mt = zero16();
      const int tr = 32 * gt + l32, sr = 32 * si + l32;
#pragma unroll 4
      for (int k = 0; k < SN / 16; ++k) {
        const int col = 16 * k + 8 * hi;
        mt = mfma(lds8(sm.B + sw_n(sr, col)), lds8(sm.C + sw_n(tr, col)), mt);
      }
      const int t = tr;
      const float cst = sm.csl[t];
      const int sb = 32 * si + 4 * hi;
      const float *csb = sm.csl + sb, *dtb = sm.dt + sb;
      if (si != gt) {  // the tile below the diagonal: every s < t
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int so = 8 * (r >> 2) + (r & 3);
          mt[r] *= __builtin_amdgcn_exp2f(cst - csb[so]) * dtb[so];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int so = 8 * (r >> 2) + (r & 3), s = sb + so;
          // above the diagonal the exponent may overflow: selected away.  The
          // skip term D x[t] rides on the diagonal, so sum_s M[t,s] x[s]
          // includes it.
          const float v = mt[r] * __builtin_amdgcn_exp2f(cst - csb[so]) * dtb[so];
          mt[r] = s < t ? v : (s == t ? v + Dh : 0.f);
        }
      }
      // M is read only after the next barrier (the previous block's reads of
      // it ended before barrier A)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        lds_st8(sm.MT + sw_m(t, 32 * si + 8 * q + 4 * hi),
                pack4(mt[4 * q], mt[4 * q + 1], mt[4 * q + 2], mt[4 * q + 3]));
    }
    lds_barrier();  // [C] M is in LDS; G4 has read h_prev

    if (!swave) {
      // ---- G2: intra-block part and the skip term, M[t, s<=t] x[s, p]
      const int ksteps = ta == 0 ? 2 : 4;
      const TrOff xo = tr_off(32 * pb + 16 * ((lane >> 4) & 1), lane, SwX());
      for (int k = 0; k < ksteps; ++k) {
        const bf16x8_t av = lds8(sm.MT + sw_m(32 * ta + l32, 16 * k + 8 * hi));
        const bf16x8_t bv = ldtr8(sm.X + 16 * k * SP, xo);
        tile = mfma(av, bv, tile);
      }
    } else {
      // ---- G3: h^T <- lam h^T + B^T (w x); then the checkpoints and the bf16
      // copy of h for the next block's G4 (G4 of this block is done: barrier C)
      const float lam = sm.lam;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) hacc[j][r] *= lam;
      const int grp = 16 * ((lane >> 4) & 1);
      const TrOff bo = tr_off(32 * nt + grp, lane, SwN());
      const TrOff wo0 = tr_off(grp, lane, SwX()), wo1 = tr_off(32 + grp, lane, SwX());
#pragma unroll
      for (int k = 0; k < Q / 16; ++k) {
        const bf16x8_t av = ldtr8(sm.B + 16 * k * SN, bo);
        hacc[0] = mfma(av, ldtr8(sm.XW + 16 * k * SP, wo0), hacc[0]);
        hacc[1] = mfma(av, ldtr8(sm.XW + 16 * k * SP, wo1), hacc[1]);
      }
      for (int c = ck; c < ck_next; ++c)
        state_store(hacc, a.ckpt_out + ((size_t)m.ck_idx[c] * d.H + h) * PN, nt, l32, hi);
      state_to_lds(hacc, sm.HT, nt, l32, hi);
    }
    have_h = true;
    ck = ck_next;
    const bool more = n1 > n0;
    lds_barrier();  // [E] every read of this block's LDS is done
    // The next block's inputs go to LDS first: waiting for the prefetched
    // loads here must not also wait for this block's y stores, which are only
    // issued afterwards.
    if (more) stage_store(st, sm, n1 - n0, tid, lane, wave, Ah);
    if (!swave) {
      // ---- epilogue: the wave's 32 x 32 y tile goes through its own 2 KiB of
      // the M region (free since barrier E; M is next written after barrier A)
      // and leaves as 16-byte row segments.  Registers 2i, 2i+1 hold rows t,
      // t+1 of column p = l%32: one conversion packs both, written as two
      // 16-bit halves.
      bf16_t *yt = sm.MT + wave * (32 * 32);  // [t][p], 64 bytes per row
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t pk = pack2_bf16(tile[2 * i], tile[2 * i + 1]);
        const int t = acc_row(2 * i, hi);
        yt[t * 32 + l32] = (bf16_t)pk;
        yt[(t + 1) * 32 + l32] = (bf16_t)(pk >> 16);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int q = lane + 64 * k;  // 128 chunks of 16 bytes
        const int row = q >> 2, c = q & 3;
        const uint4 v = lds_ld16(yt + row * 32 + c * 8);
        const int t = 32 * ta + row;
        if (t < len)
          *reinterpret_cast<uint4 *>(yg + ((size_t)(t0 + t) * d.H + h) * SP + 32 * pb + c * 8) = v;
      }
    }
    if (!more) break;
    t0 = n0;
    t1 = n1;
  }

  if (sg.final && swave)
    state_store(hacc, (sg.final == 1 ? seg_state : a.workspace) + (size_t)h * PN, nt, l32, hi);
}

}  // namespace

bool ssd_supported(int io, const Dims &d) { return io == kBF16 && d.P == SP && d.N == SN; }

hipError_t launch_scan_ssd(const ScanArgs &a, const ScanMeta &m, hipStream_t s) {
  dim3 grid(a.n_seg * a.d.H), block(kSsdThreads);
  hipLaunchKernelGGL(scan_ssd_kernel, grid, block, 0, s, a, m);
  return hipGetLastError();
}

}  // namespace ssm
