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
// One workgroup (4 waves) owns one (segment, head): a segment is a run of
// tokens between resets, so it starts from the carried-in state or from zero
// and no reset falls inside it.  The fp32 state h^T[n,p] stays in MFMA
// accumulators across blocks (wave w owns n in [32w, 32w+32)); a bf16 copy in
// LDS feeds G4 of the next block.  Blocks end early at checkpoint tokens so the
// post-token state can be written from the accumulators.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Operand lane layout (A: 32 x 16, B: 16 x 32):
// lane l supplies row/column l%32 and K indices 8*(l/32) .. +7; accumulator
// register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.  Every
// operand is read from LDS as one 16-byte row segment, so each operand tile is
// staged in the orientation that puts K contiguous.
#include "ssm_device.h"

namespace ssm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int Q = 64;    // tokens per block
constexpr int SP = 64;   // head dim
constexpr int SN = 128;  // state size

// Rows of 128 bf16 (C, B, h) are unpadded with their 16-byte chunks
// XOR-swizzled by row; rows of 64 bf16 (the transposed tiles) are padded to 72
// so that the scattered 2-byte transposing writes have linear addresses.
// Either way the 32 rows one MFMA operand read touches fall on distinct banks.
constexpr int LDT = Q + 8;
__device__ __forceinline__ int sw128(int row, int col) {
  return row * 128 + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
}

// 78 KiB: two workgroups fit in one CU's 160 KiB.
struct Smem {
  bf16_t C[Q * SN];          // C[t][n]                     (swizzled)
  bf16_t R[2 * Q * LDT];     // B[s][n] (swizzled) until G1 is done, then
                             // M^T[t][s] and (w x)^T[p][s] (padded)
  bf16_t BT[SN * LDT];       // B[s][n] stored [n][s]       (padded)
  bf16_t Xt[SP * LDT];       // x[s][p] stored [p][s]       (padded)
  bf16_t HT[SP * SN];        // bf16 copy of h_prev[p][n]   (swizzled)
  float dt[Q], cs[Q], ecs[Q], w[Q];
  float lam;
};
static_assert(2 * Q * LDT >= Q * SN, "R must hold B row-major");
static_assert(2 * sizeof(Smem) <= 160 * 1024, "two workgroups per CU");

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t lds8(const bf16_t *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
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

// h^T accumulators (two 32 x 32 tiles: n in [32w, 32w+32), p-tile j) <-> a
// [P][N] fp32 state tile.  Register r of lane l is h[p = 32j + l%32][n = 32w +
// acc_row(r)], so four consecutive registers are four consecutive n.
__device__ __forceinline__ void state_load(f32x16_t hacc[2], const float *src, int wave, int l32,
                                           int hi) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 32 * j + l32, n = 32 * wave + 8 * q + 4 * hi;
      const float4 v = *reinterpret_cast<const float4 *>(src + (size_t)p * SN + n);
      hacc[j][4 * q + 0] = v.x;
      hacc[j][4 * q + 1] = v.y;
      hacc[j][4 * q + 2] = v.z;
      hacc[j][4 * q + 3] = v.w;
    }
}
__device__ __forceinline__ void state_store(const f32x16_t hacc[2], float *dst, int wave, int l32,
                                            int hi) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 32 * j + l32, n = 32 * wave + 8 * q + 4 * hi;
      *reinterpret_cast<float4 *>(dst + (size_t)p * SN + n) =
          make_float4(hacc[j][4 * q], hacc[j][4 * q + 1], hacc[j][4 * q + 2], hacc[j][4 * q + 3]);
    }
}
__device__ __forceinline__ void state_to_lds(const f32x16_t hacc[2], bf16_t *HT, int wave, int l32,
                                             int hi) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 32 * j + l32, n = 32 * wave + 8 * q + 4 * hi;
      *reinterpret_cast<uint2 *>(HT + sw128(p, n)) =
          pack4(hacc[j][4 * q], hacc[j][4 * q + 1], hacc[j][4 * q + 2], hacc[j][4 * q + 3]);
    }
}

// One block's global inputs, held in registers between the load and the LDS
// write so the loads overlap the previous block's compute.
struct Staged {
  uint4 c[4], b[4], x[2];
  uint32_t dt;  // raw bf16 bits
};

// Thread layout of the staging: in pass k, wave w handles 16-byte chunk
// c = w + 4k of every token row, one row per lane (row = lane).  Each
// transposing write then covers 64 consecutive tokens of one row of B^T / x^T,
// and lane pairs (2i, 2i+1) swap halves so that each lane writes 4-byte words
// holding two consecutive tokens: bank-conflict-free.  Loads are
// unconditional (rows past the block end re-read its last row) so no wait is
// needed until the values are written to LDS; stage_store zeroes those rows.
__device__ __forceinline__ void stage_load(Staged &st, const ScanArgs &a, int t0, int len, int h,
                                           int g, int lane, int wave) {
  const Dims &d = a.d;
  const bf16_t *Cg = (const bf16_t *)a.C, *Bg = (const bf16_t *)a.B;
  const bf16_t *xg = (const bf16_t *)a.x, *dtg = (const bf16_t *)a.dt;
  const int row = t0 + min(lane, len - 1);
  const size_t rowCB = ((size_t)row * d.G + g) * SN;
  const size_t rowX = ((size_t)row * d.H + h) * SP;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c8 = (wave + 4 * k) * 8;
    st.c[k] = *reinterpret_cast<const uint4 *>(Cg + rowCB + c8);
    st.b[k] = *reinterpret_cast<const uint4 *>(Bg + rowCB + c8);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
    st.x[k] = *reinterpret_cast<const uint4 *>(xg + rowX + (wave + 4 * k) * 8);
  st.dt = dtg[(size_t)row * d.H + h];
}

// Write 8 bf16 of token `lane` (elements col8..col8+7 of its row) transposed
// into dst[(col8 + j) * LDT + token]; the partner lane holds the other token of
// the pair.
__device__ __forceinline__ void transpose_store(bf16_t *dst, int col8, uint4 v, int lane) {
  const int odd = lane & 1;
  // v.{x,y,z,w} hold element pairs (0,1) (2,3) (4,5) (6,7).  The even lane keeps
  // the even elements of each pair and receives the partner's even elements;
  // the odd lane the odd ones.
  uint32_t mine[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t send = odd ? (mine[i] & 0xffffu) : (mine[i] >> 16);
    // swap with the adjacent lane (DPP quad_perm [1,0,3,2])
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
    // word for (token pair, element 2i + odd): low half = even token, high = odd token
    out[i] = odd ? (recv | (mine[i] & 0xffff0000u)) : ((mine[i] & 0xffffu) | (recv << 16));
  }
  const int tok0 = lane & ~1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint32_t *>(dst + (col8 + 2 * i + odd) * LDT + tok0) = out[i];
}

__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
  return ok ? v : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void stage_store(const Staged &st, Smem &sm, int len, int lane,
                                            int wave) {
  const bool ok = lane < len;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c8 = (wave + 4 * k) * 8;
    const uint4 b = keep_if(ok, st.b[k]);
    *reinterpret_cast<uint4 *>(sm.C + sw128(lane, c8)) = keep_if(ok, st.c[k]);
    *reinterpret_cast<uint4 *>(sm.R + sw128(lane, c8)) = b;
    transpose_store(sm.BT, c8, b, lane);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) transpose_store(sm.Xt, (wave + 4 * k) * 8, keep_if(ok, st.x[k]), lane);
  if (wave == 0) sm.dt[lane] = ok ? __uint_as_float(st.dt << 16) : 0.f;
}

// end (exclusive) of the block starting at t0: Q tokens, the segment end, or
// just past the next checkpoint token
__device__ __forceinline__ int block_end(const ScanArgs &a, const ScanMeta &m, int t0, int seg_end,
                                         int ck) {
  int t1 = min(t0 + Q, seg_end);
  if (ck < a.n_ck && m.ck_t[ck] < t1) t1 = m.ck_t[ck] + 1;
  return t1;
}

__global__ __launch_bounds__(kThreads, 2) void scan_ssd_kernel(ScanArgs a, ScanMeta m) {
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
  bf16_t *MT = sm.R;              // [t][s], valid after G1
  bf16_t *XwT = sm.R + Q * LDT;   // [p][s], valid after G1

  f32x16_t hacc[2];
  bool have_h = sg.init != 0;
  if (have_h) {
    state_load(hacc, a.state + (size_t)h * PN, wave, l32, hi);
    state_to_lds(hacc, sm.HT, wave, l32, hi);
  } else {
    hacc[0] = zero16();
    hacc[1] = zero16();
  }
  int ck = 0;
  while (ck < a.n_ck && m.ck_t[ck] < sg.t0) ++ck;

  // the wave's output tile of y: rows t in [32*ta, +32), columns p in [32*pb, +32)
  const int ta = wave >> 1, pb = wave & 1;

  Staged st;
  int t0 = sg.t0;
  int t1 = block_end(a, m, t0, sg.t1, ck);
  stage_load(st, a, t0, t1 - t0, h, g, lane, wave);
  stage_store(st, sm, t1 - t0, lane, wave);

  while (true) {
    const int len = t1 - t0;
    // checkpoints at t1 - 1 are consumed by this block
    int ck_next = ck;
    while (ck_next < a.n_ck && m.ck_t[ck_next] == t1 - 1) ++ck_next;
    const int n0 = t1, n1 = n0 < sg.t1 ? block_end(a, m, n0, sg.t1, ck_next) : n0;
    __syncthreads();  // [A] this block's inputs are in LDS

    if (n1 > n0) stage_load(st, a, n0, n1 - n0, h, g, lane, wave);  // next block, in flight

    // ---- running log-decay inside the block (one wave, one token per lane)
    if (wave == 0) {
      const float dtv = sm.dt[lane];
      float v = dtv * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_up(v, off);
        if (lane >= off) v += u;
      }
      const float end = __shfl(v, 63);
      sm.cs[lane] = v;
      sm.ecs[lane] = __expf(v);
      sm.w[lane] = __expf(end - v) * dtv;
      if (lane == 0) sm.lam = __expf(end);
    }
    __syncthreads();  // [B]

    // ---- G1 and G4 in one K loop.  Wave w's output tile of y has rows
    // t in [32 ta, +32) and columns p in [32 pb, +32); G1 tiles are given to
    // the waves whose y rows match their t-tile, so the C fragment (rows t, K = n)
    // is read once per K step for both contractions:
    //   G1 (waves 0, 2, 3): (C.B)^T tile (s-tile si, t-tile ta)
    //   G4 (every wave):    C h_prev^T tile (ta, pb), scaled by exp(cs_t) after
    const bool g1 = wave != 1;
    const int si = wave == 3 ? 1 : 0;
    float mv[16];
    f32x16_t yacc = zero16();
    {
      f32x16_t acc = zero16();
      const bf16_t *crow = sm.C + (32 * ta + l32) * SN;
      const bf16_t *brow = sm.R + (32 * si + l32) * SN;
      const bf16_t *hrow = sm.HT + (32 * pb + l32) * SN;
      const int xr = l32 & 15;  // swizzle of every row read here (row & 15 == l32 & 15)
#pragma unroll 4
      for (int k = 0; k < SN / 16; ++k) {
        const int off = ((2 * k + hi) ^ xr) << 3;
        const bf16x8_t cv = lds8(crow + off);
        if (g1) acc = mfma(lds8(brow + off), cv, acc);
        if (have_h) yacc = mfma(cv, lds8(hrow + off), yacc);
      }
      if (g1) {
        const int t = 32 * ta + l32;
        const float cst = sm.cs[t];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int s = 32 * si + acc_row(r, hi);
          // the skip term D x[t] rides on the diagonal: sum_s M[t,s] x[s] then includes it
          mv[r] = s <= t ? acc[r] * __expf(cst - sm.cs[s]) * sm.dt[s] + (s == t ? Dh : 0.f) : 0.f;
        }
      }
      if (have_h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) yacc[r] *= sm.ecs[32 * ta + acc_row(r, hi)];
      }
    }
    __syncthreads();  // [C] B row-major no longer needed: R becomes M^T and (w x)^T

    if (g1) {
      const int t = 32 * ta + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2 *>(MT + t * LDT + 32 * si + 8 * q + 4 * hi) =
            pack4(mv[4 * q], mv[4 * q + 1], mv[4 * q + 2], mv[4 * q + 3]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = tid + kThreads * k;  // 512 chunks of x^T
      const int p = q >> 3, s0 = (q & 7) * 8;
      const uint4 v = *reinterpret_cast<const uint4 *>(sm.Xt + p * LDT + s0);
      const bf16_t *e = reinterpret_cast<const bf16_t *>(&v);
      uint4 o;
      uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ow[j] = pack2_bf16(bf16_to_f(e[2 * j]) * sm.w[s0 + 2 * j],
                           bf16_to_f(e[2 * j + 1]) * sm.w[s0 + 2 * j + 1]);
      *reinterpret_cast<uint4 *>(XwT + p * LDT + s0) = o;
    }
    __syncthreads();  // [D]

    // ---- G2: intra-block part (and the skip term), (M^T)[t, s<=t] x[s, p]
    const int ksteps = ta == 0 ? 2 : 4;
    for (int k = 0; k < ksteps; ++k) {
      const bf16x8_t av = lds8(MT + (32 * ta + l32) * LDT + 16 * k + 8 * hi);
      const bf16x8_t bv = lds8(sm.Xt + (32 * pb + l32) * LDT + 16 * k + 8 * hi);
      yacc = mfma(av, bv, yacc);
    }
    // ---- G3: h^T <- lam h^T + B^T (w x)  (this wave's n-tile, both p-tiles)
    const float lam = sm.lam;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) hacc[j][r] *= lam;
#pragma unroll 2
      for (int k = 0; k < Q / 16; ++k) {
        const bf16x8_t av = lds8(sm.BT + (32 * wave + l32) * LDT + 16 * k + 8 * hi);
        const bf16x8_t bv = lds8(XwT + (32 * j + l32) * LDT + 16 * k + 8 * hi);
        hacc[j] = mfma(av, bv, hacc[j]);
      }
    }
    // ---- epilogue: the wave's 32 x 32 y tile goes through its own 2 KiB of the
    // C region (free since barrier C) and leaves as 16-byte row segments.
    {
      bf16_t *yt = sm.C + wave * (32 * 32);  // [t][p], 64 bytes per row
      const int odd = lane & 1;
      const uint32_t sel = 0u - (uint32_t)odd;  // all ones on odd lanes
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // registers 2i, 2i+1 are rows t, t+1; adjacent lanes are columns p, p+1.
        // The even lane keeps row t and the odd lane row t+1; each sends the
        // other row to its partner.  (Bit blends rather than ?: on vector
        // elements, which the compiler would turn into a variable-index extract.)
        const uint32_t a = __float_as_uint(yacc[2 * i]), b = __float_as_uint(yacc[2 * i + 1]);
        const uint32_t keep = (a & ~sel) | (b & sel);
        const uint32_t send = (b & ~sel) | (a & sel);
        const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
        // low half = column p (even lane's value), high half = column p+1
        const uint32_t lo = (keep & ~sel) | (recv & sel), hiw = (recv & ~sel) | (keep & sel);
        const int t = acc_row(2 * i, hi) + odd;  // even lane: row t, odd lane: row t+1
        *reinterpret_cast<uint32_t *>(yt + t * 32 + (l32 & ~1)) =
            pack2_bf16(__uint_as_float(lo), __uint_as_float(hiw));
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int q = lane + 64 * k;  // 128 chunks of 16 bytes
        const int row = q >> 2, c = q & 3;
        const uint4 v = *reinterpret_cast<const uint4 *>(yt + row * 32 + c * 8);
        const int t = 32 * ta + row;
        if (t < len)
          *reinterpret_cast<uint4 *>(yg + ((size_t)(t0 + t) * d.H + h) * SP + 32 * pb + c * 8) = v;
      }
    }
    have_h = true;
    for (; ck < ck_next; ++ck)
      state_store(hacc, a.ckpt_out + ((size_t)m.ck_idx[ck] * d.H + h) * PN, wave, l32, hi);
    if (n1 <= n0) break;
    __syncthreads();  // [E] every read of this block's LDS is done
    state_to_lds(hacc, sm.HT, wave, l32, hi);
    stage_store(st, sm, n1 - n0, lane, wave);
    t0 = n0;
    t1 = n1;
  }

  if (sg.final)
    state_store(hacc, (sg.final == 1 ? a.state : a.workspace) + (size_t)h * PN, wave, l32, hi);
}

}  // namespace

bool ssd_supported(int io, const Dims &d) { return io == kBF16 && d.P == SP && d.N == SN; }

hipError_t launch_scan_ssd(const ScanArgs &a, const ScanMeta &m, hipStream_t s) {
  dim3 grid(a.n_seg * a.d.H), block(kThreads);
  hipLaunchKernelGGL(scan_ssd_kernel, grid, block, 0, s, a, m);
  return hipGetLastError();
}

}  // namespace ssm
