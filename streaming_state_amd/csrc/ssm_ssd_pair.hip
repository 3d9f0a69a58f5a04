// ssm_ssd_pair.hip -- chunk scan, SSD (matrix) form on MFMA, for bf16 inputs
// with head dim P = 64 and state size N = 128, two heads of one B/C group per
// workgroup.
//
// The block algebra is the one of the single-head form ("Separate Mamba-2
// algebra from kernel behavior": the matrix view for prefill).  With cs_t the
// running sum of dt*A inside a block of Q = 64 tokens:
//   G1  M[t,s]   = (C_t.B_s) exp(cs_t - cs_s) dt_s  for s <= t, plus D on s = t
//   G4  y[t,p]   = exp(cs_t) sum_n C[t,n] h_prev[p,n]
//   G2  y[t,p]  += sum_{s<=t} M[t,s] x[s,p]
//   G3  h[p,n]   = exp(cs_end) h_prev[p,n] + sum_s exp(cs_end - cs_s) dt_s x[s,p] B[s,n]
// Split of the work: one workgroup (8 waves) owns one (segment, head pair);
// a segment is a run of tokens between resets.  Wave w works on head
// h0 + w/4 and the 16 head-dim rows p in [16 (w%4), +16).  It keeps that slice
// of the fp32 state, for all 128 n, in MFMA accumulators
// (v_mfma_f32_16x16x32_bf16) for the whole segment and produces the same slice
// of y, so G4, G3 and G2 need nothing from other waves but M: G4 takes its A
// operand from the wave's own state registers (converted to bf16), and the
// products are arranged transposed (y^T[p,t], h^T[n,p]) so that every result
// lands in the layout its consumer or its store needs.  The ten 16 x 16 tiles
// of C.B^T on or below the diagonal are shared out over the eight waves, and
// each is masked once per head: the heads share B and C, so the products are
// computed once for both.
//
// Inputs reach LDS by direct global->LDS loads (no registers on the way),
// double buffered: the next block's loads are in flight while this block
// computes, issued in three parts spread over its phases.  They are issued
// from inline assembly, so the compiler, which cannot tell which LDS bytes
// such a load writes, does not make every LDS read of the current block wait
// for them; the kernel waits for them itself (an explicit vmcnt before the
// first barrier of the next block).  Two barriers per block: inputs landed; M
// written.  The next block's running sums are computed after the second, while
// M is read.  Each phase issues its reads together, ahead of the work that
// hides their latency.  ~124 KiB of LDS, one workgroup per CU, two waves per
// SIMD.
//
// MFMA 16x16x32 operand layout: lane l supplies row (A) or column (B) l%16 and
// eight K values; which K a register slot carries is the same for A and B,
// which is all a product needs, so every operand below is read so that slot j
// of lane group g = l/16 carries the same contraction index on both sides.
// Accumulator register r of lane l holds row 4(l/16) + r, column l%16.
#include "ssm_device.h"

namespace ssm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kPairThreads = 512;
constexpr int Q = 64;    // tokens per block
constexpr int SP = 64;   // head dim
constexpr int SN = 128;  // state size

// LDS map (bytes).  C, B and X (x of both heads, [t][2P]) are double-buffered
// 64-row tiles of 256-byte rows; M holds one 64 x 64 bf16 matrix per head;
// each head has an area for its running sums, written by one wave and read by
// all eight.
constexpr int kRowB = 256;
constexpr int kTileB = Q * kRowB;
constexpr int kOffC = 0;
constexpr int kOffB = 2 * kTileB;
constexpr int kOffX = 4 * kTileB;
constexpr int kOffM = 6 * kTileB;
constexpr int kMHeadB = Q * Q * 2;
constexpr int kOffSums = kOffM + 2 * kMHeadB;
// running sums of one head: rows cs, cs - log2|dt|, exp(cs), w (64 floats
// each), then exp(cs_end) and a negative-dt flag
constexpr int kSumsB = 4 * Q * 4 + 16;
constexpr int kSumLam = 4 * Q * 4, kSumNeg = kSumLam + 4;
constexpr int kOffDt = kOffSums + 2 * kSumsB;  // dt of both heads per token, per buffer
constexpr int kSmemB = kOffDt + 2 * Q * 4;
static_assert(kSmemB <= 160 * 1024, "fits the LDS of one CU");

extern __shared__ __attribute__((aligned(16))) char pair_smem[];

// 256-byte rows: 16-byte chunk c of row r sits at chunk c ^ f(r), f a linear
// bijection of r mod 16 (over GF(2)).  B and x are read two ways: by rows (a
// 16-byte read of one chunk over 16 consecutive rows) and transposed (rows
// {r..r+3, r+8..r+11}, r % 16 in {0, 4}, x one aligned chunk pair).  For the
// transposed reads f >> 1 must be distinct over those eight rows, so that the
// pairs land on distinct 32-byte slots; which f also keeps the row reads free
// of bank conflicts was measured on gfx950 (the 16-byte rule is not the plain
// "distinct 16-byte slots per 16 lanes"): this one, bits
//   f0 = r0^r2, f1 = r0^r2^r3, f2 = r1, f3 = r2^r3.
__device__ __forceinline__ int fsw(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  return (r0 ^ r2) | ((r0 ^ r2 ^ r3) << 1) | (r1 << 2) | ((r2 ^ r3) << 3);
}
__device__ __forceinline__ int tile_off(int r, int c) { return r * kRowB + ((c ^ fsw(r)) << 4); }
// C is only read by rows: the plain row XOR (chunk c of row r at c ^ (r % 16))
// is conflict-free for them (measured).
__device__ __forceinline__ int c_off(int r, int c) { return r * kRowB + ((c ^ (r & 15)) << 4); }
// M rows are 128 bytes (64 s): chunk c of row t sits at c ^ ((t >> 1) & 7).
__device__ __forceinline__ int m_off(int t, int c) { return t * 128 + ((c ^ ((t >> 1) & 7)) << 4); }

template <typename T> __device__ __forceinline__ T ld_lds(int off) {
  return *(const __attribute__((address_space(3))) T *)((const lds_char *)pair_smem + off);
}
template <typename T> __device__ __forceinline__ void st_lds(int off, T v) {
  *(__attribute__((address_space(3))) T *)((lds_char *)pair_smem + off) = v;
}
// transposing read: lane j of each 16-lane group receives column col0 + j of
// the four rows its group's lanes address (lane i of the group addresses row
// i/4, columns col0 + 4(i%4) .. +3)
__device__ __forceinline__ s16x4_t ld_tr(int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t *)((lds_char *)pair_smem + off));
}
__device__ __forceinline__ bf16x8_t cat8(s16x4_t lo, s16x4_t hi) {
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t cat8(u32x2_t lo, u32x2_t hi) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}
__device__ __forceinline__ u32x2_t pk4(f32x4_t v) {
  return u32x2_t{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
}
__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Direct global->LDS copies of 16 (4) bytes per lane: lane l's bytes at
// base + voff land at LDS byte lds + 16 l (4 l); lds is wave-uniform, passed
// in M0, which is restored afterwards.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void dma4(const void *base, uint32_t voff, uint32_t lds) {  // 4 bytes
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}

// Workgroup barrier that orders LDS only (see the single-head form).
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// end (exclusive) of the block starting at t0: Q tokens, the segment end, or
// just past the next checkpoint token
__device__ __forceinline__ int block_end(const ScanArgs &a, const ScanMeta &m, int t0, int seg_end,
                                         int ck) {
  int t1 = min(t0 + Q, seg_end);
  if (ck < a.n_ck && m.ck_t[ck] < t1) t1 = m.ck_t[ck] + 1;
  return t1;
}

// G4's A operand for K = n in [32j, 32j + 32) from the state tiles 2j and
// 2j+1 (lane group g holds n = 32j + 4g .. +3 and 32j + 16 + 4g .. +3): two
// row swaps (upper half with lower half, then odd rows with even rows) give
// lane group g n = 32j + 8g .. +7 in order, the K layout of a 16-byte read
// of C.
__device__ __forceinline__ bf16x8_t state_operand(f32x4_t lo_tile, f32x4_t hi_tile) {
  const u32x2_t a = pk4(lo_tile), b = pk4(hi_tile);
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const auto s32 = __builtin_amdgcn_permlane32_swap(a[e], b[e], false, false);
    const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
    o[e] = s16[0];      // n = 32j + 8g + 2e .. +1
    o[2 + e] = s16[1];  // n = 32j + 8g + 4 + 2e .. +1
  }
  return __builtin_bit_cast(bf16x8_t, o);
}

// Everything a wave carries from block to block.
struct Wave {
  // identity
  int lane, li, g, w, q, ps;
  // per-lane LDS byte offsets, fixed for the whole kernel (a buffer, a tile
  // row or a K step adds a constant)
  int o_c[4];    // C rows (G4, G1): n = 32k + 8g .. +7
  int o_b1[4];   // B rows (G1): the same n
  int o_x[2];    // x, transposing, rows +0 / +4
  int bt_base[2], bt_xor[2];  // B^T, transposing, rows +0 / +4: n tile i at base + (32 i ^ xor)
  int o_m[2];    // M rows for G2, per K step
  int sums;      // this wave's head's running-sum area
  // staging: per-lane source offsets of full blocks (row 8w + 4u + g)
  uint32_t v_b[2], v_x[2], v_c[2];
  // state and output accumulators
  f32x4_t h[8];  // h^T[n = 16i + 4g + r][p = 16 ps + li]
  f32x4_t y[4];  // y^T[p = 16 ps + 4g + r][t = 16 tt + li]
  bool have_h;
  bool neg;      // some dt of the current block is negative (either head)
  bool stores4;  // exactly four global stores followed the last input loads
};

struct Seg {
  int t0, t1, n0, n1;  // current block [t0, t1), next block [n0, n1)
  int seg_end, ck;
  int h0, grp;
  float al2[2], Dq[2];
};

// The next block's loads, prepared once and issued in parts spread over the
// block, so that the eight waves do not all queue their copies at once.
struct Loads {
  const char *cb, *bb, *xb, *dtb;
  uint32_t vb[2], vx[2], vc[2], vdt, lds;
};
__device__ __forceinline__ Loads prepare_loads(const ScanArgs &a, const Wave &W, const Seg &S,
                                               int buf, int t0, int len) {
  const Dims &d = a.d;
  const size_t sCB = (size_t)d.G * SN * 2, sX = (size_t)d.H * SP * 2;
  Loads L;
  L.cb = (const char *)a.C + ((size_t)t0 * d.G + S.grp) * SN * 2;
  L.bb = (const char *)a.B + ((size_t)t0 * d.G + S.grp) * SN * 2;
  L.xb = (const char *)a.x + ((size_t)t0 * d.H + S.h0) * SP * 2;
  L.dtb = (const char *)((const bf16_t *)a.dt + (size_t)t0 * d.H + S.h0);
  L.vdt = (uint32_t)(min(W.lane, len - 1) * d.H * 2);  // dt of both heads, token `lane`
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    L.vb[u] = W.v_b[u];
    L.vx[u] = W.v_x[u];
    L.vc[u] = W.v_c[u];
  }
  if (len < Q) {  // rows past the block end re-read its last row (finite, weighted by dt = 0)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rdst = 8 * W.w + 4 * u + W.g, rs = min(rdst, len - 1);
      const int lc = (W.li ^ fsw(rdst)) << 4;
      L.vb[u] = (uint32_t)(rs * sCB + lc);
      L.vx[u] = (uint32_t)(rs * sX + lc);
      L.vc[u] = (uint32_t)(rs * sCB + ((W.li ^ (rdst & 15)) << 4));
    }
  }
  L.lds = (uint32_t)(uintptr_t)(lds_char *)pair_smem + buf * kTileB + 8 * W.w * kRowB;
  return L;
}
// part 0: dt (wave 0, first: six copies follow it) and C; part 1: B; part 2: x
__device__ __forceinline__ void issue_part(const Loads &L, const Wave &W, int part, int buf) {
  if (part == 0 && W.w == 0)
    dma4(L.dtb, L.vdt, (uint32_t)(uintptr_t)(lds_char *)pair_smem + kOffDt + buf * Q * 4);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t dst = L.lds + 4 * u * kRowB;
    if (part == 0) dma16(L.cb, L.vc[u], kOffC + dst);
    if (part == 1) dma16(L.bb, L.vb[u], kOffB + dst);
    if (part == 2) dma16(L.xb, L.vx[u], kOffX + dst);
  }
}

// Makes the register value available at this point (the compiler waits for
// its load here) and keeps memory operations on their side of it: the reads
// of a phase are issued together, ahead of the work that hides their latency.
template <typename T> __device__ __forceinline__ void pin(T &v) {
  asm volatile("" : "+v"(v)::"memory");
}

// Keeps the compiler from moving memory operations across this point (it
// fixes the order in which reads are issued).
__device__ __forceinline__ void fence() { asm volatile("" ::: "memory"); }

// One 16 x 16 tile of C.B^T (s tile a, t tile b) and the running sums its mask
// needs, read ahead of its products.
struct Tile {
  int a, b;
  bf16x8_t ga[4], gb[4];
  float cst[2];
  f32x4_t cp[2];
};
__device__ __forceinline__ Tile tile_load(const Wave &W, int id, int bbuf, int cbuf) {
  Tile t;
  t.a = id < 4 ? id : id < 7 ? id - 4 : id == 7 ? 0 : id == 8 ? 1 : 0;
  t.b = id < 4 ? id : id < 7 ? id - 3 : id == 7 ? 2 : 3;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.ga[k] = ld_lds<bf16x8_t>(bbuf + t.a * 16 * kRowB + W.o_b1[k]);
    t.gb[k] = ld_lds<bf16x8_t>(cbuf + t.b * 16 * kRowB + W.o_c[k]);
  }
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    t.cst[hq] = ld_lds<float>(kOffSums + hq * kSumsB + 4 * (16 * t.b + W.li));
    t.cp[hq] = ld_lds<f32x4_t>(kOffSums + hq * kSumsB + 256 + 4 * (16 * t.a + 4 * W.g));
  }
  return t;
}
// M_q[t][s] = C_t.B_s exp2(cs_t - cs_s) dt_s for both heads, D on the diagonal.
// |dt_s| rides in the exponent; a block with a negative dt takes its sign from
// the block's dt in LDS (dtbuf).
__device__ __forceinline__ void tile_mask(const Wave &W, const Seg &S, Tile &t, int dtbuf) {
  const int li = W.li, g = W.g;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    pin(t.ga[k]);
    pin(t.gb[k]);
  }
  f32x4_t cb = zero4();
#pragma unroll
  for (int k = 0; k < 4; ++k) cb = mfma(t.ga[k], t.gb[k], cb);
  // cb[r] = C_t.B_s with t = 16 b + li, s = 16 a + 4 g + r
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    f32x4_t mv;
#pragma unroll
    for (int r = 0; r < 4; ++r) mv[r] = cb[r] * __builtin_amdgcn_exp2f(t.cst[hq] - t.cp[hq][r]);
    if (W.neg) {  // dt of both heads, tokens s = 16 a + 4 g + r
      const u32x4_t dw = ld_lds<u32x4_t>(dtbuf + 4 * (16 * t.a + 4 * g));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mv[r] = __uint_as_float(__float_as_uint(mv[r]) ^ ((hq ? dw[r] : dw[r] << 16) & 0x80000000u));
    }
    if (t.a == t.b) {
      // above the diagonal the exponent may overflow: selected away; the skip
      // term D x[t] rides on the diagonal
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 4 * g + r;
        mv[r] = s < li ? mv[r] : (s == li ? mv[r] + S.Dq[hq] : 0.f);
      }
    }
    st_lds<u32x2_t>(kOffM + hq * kMHeadB + (16 * t.b + li) * 128 +
                        (((2 * t.a + (g >> 1)) ^ ((li >> 1) & 7)) << 4) + 8 * (g & 1),
                    pk4(mv));
  }
}

// Running sums of dt*A (log2 units) of a block for head hq, one token per
// lane, into the head's area: cs, cs - log2|dt| (the mask's exp2(cs_t - this)
// carries the |dt_s| factor; dt = 0, past the block end, gives +inf and a zero
// weight), exp(cs), the G3 weights, exp(cs_end) and whether a dt of the block
// is negative.  One wave per head (on different SIMDs) computes them; the
// barrier that opens the block makes them visible to the other seven.
__device__ __forceinline__ void block_sums(const Wave &W, const Seg &S, int buf, int len, int hq) {
  const int lane = W.lane;
  const uint32_t dtw = ld_lds<uint32_t>(kOffDt + buf * Q * 4 + 4 * lane);
  const float dq = lane < len ? __uint_as_float(hq ? (dtw & 0xffff0000u) : (dtw << 16)) : 0.f;
  const float c = scan64(dq * (hq ? S.al2[1] : S.al2[0]));
  const float end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
  const int area = kOffSums + hq * kSumsB;
  const int s = area + 4 * lane;
  st_lds<float>(s + 0 * 256, c);
  st_lds<float>(s + 1 * 256, c - __builtin_amdgcn_logf(fabsf(dq)));
  st_lds<float>(s + 2 * 256, __builtin_amdgcn_exp2f(c));
  st_lds<float>(s + 3 * 256, __builtin_amdgcn_exp2f(end - c) * dq);
  const bool neg = __builtin_amdgcn_ballot_w64(dq < 0.f) != 0;
  if (lane == 0) {
    st_lds<float>(area + kSumLam, __builtin_amdgcn_exp2f(end));
    st_lds<uint32_t>(area + kSumNeg, neg ? 1u : 0u);
  }
}
// the wave that computes head hq's sums: waves 0 and 5 (SIMDs 0 and 1)
__device__ __forceinline__ bool sums_wave(const Wave &W) { return W.w == 0 || W.w == 5; }

template <int BUF>
__device__ __forceinline__ bool pair_block(const ScanArgs &a, const ScanMeta &m, Wave &W, Seg &S) {
  const Dims &d = a.d;
  const int len = S.t1 - S.t0;
  const bool full = len == Q;
  // checkpoints at t1 - 1 are consumed by this block
  int ck_next = S.ck;
  while (ck_next < a.n_ck && m.ck_t[ck_next] == S.t1 - 1) ++ck_next;
  S.n0 = S.t1;
  S.n1 = S.n0 < S.seg_end ? block_end(a, m, S.n0, S.seg_end, ck_next) : S.n0;
  const bool more = S.n1 > S.n0;

  // this block's inputs (issued one block ago) have landed in LDS
  if (W.stores4)
    __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();  // [A] inputs of this block visible; the other buffer is free
  // this block's sums were written during the previous one
  const float lam = ld_lds<float>(W.sums + kSumLam);
  W.neg = (ld_lds<uint32_t>(kOffSums + kSumNeg) | ld_lds<uint32_t>(kOffSums + kSumsB + kSumNeg)) != 0;
  const Loads nl = prepare_loads(a, W, S, BUF ^ 1, S.n0, S.n1 - S.n0);

  const int li = W.li, g = W.g, q = W.q;
  const int cbuf = kOffC + BUF * kTileB, bbuf = kOffB + BUF * kTileB, xbuf = kOffX + BUF * kTileB;

  // ---- reads, in the order they are needed: G4's C operands; x, the G3
  // weights and exp(cs_t); the operands of this wave's first C.B tile
  bf16x8_t op[16];
  if (W.have_h) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        op[4 * tt + j] = ld_lds<bf16x8_t>(cbuf + W.o_c[j] + tt * 16 * kRowB);
  }
  fence();
  s16x4_t xr[4];  // x[s = 32k + 8g + 4r + ..][p = 16 ps + li]: [k][r]
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int r = 0; r < 2; ++r) xr[2 * k + r] = ld_tr(xbuf + W.o_x[r] + k * 32 * kRowB);
  f32x4_t wv[4];  // w_s, s = 32k + 8g + 4e .. +3: [k][e]
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      wv[2 * k + e] = ld_lds<f32x4_t>(W.sums + 3 * 256 + 4 * (32 * k + 8 * g + 4 * e));
  float ev[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) ev[tt] = ld_lds<float>(W.sums + 2 * 256 + 4 * (16 * tt + li));
  if (more) issue_part(nl, W, 0, BUF ^ 1);

  // ---- G4: y^T[p,t] = exp(cs_t) sum_n h_prev[p,n] C[t,n]
  if (W.have_h) {
    bf16x8_t ha[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ha[j] = state_operand(W.h[2 * j], W.h[2 * j + 1]);
#pragma unroll
    for (int i = 0; i < 16; ++i) pin(op[i]);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma(ha[j], op[4 * tt + j], acc);
      W.y[tt] = acc;
    }
  }
  // G1 tiles: waves 0..7 take (s tile a, t tile b) = (0,0) (1,1) (2,2) (3,3)
  // (0,1) (1,2) (2,3) (0,2); waves 0 and 1 also take (1,3) and (0,3)
  Tile t0 = tile_load(W, W.w, bbuf, cbuf);
  // ---- x and w x (G3's B operand), beside G4's products
  bf16x8_t xk[2], xt[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    pin(xr[2 * k]);
    pin(xr[2 * k + 1]);
    xk[k] = cat8(xr[2 * k], xr[2 * k + 1]);
    pin(wv[2 * k]);
    pin(wv[2 * k + 1]);
    const u32x4_t xv = __builtin_bit_cast(u32x4_t, xk[k]);
    const float w8[8] = {wv[2 * k][0], wv[2 * k][1], wv[2 * k][2], wv[2 * k][3],
                         wv[2 * k + 1][0], wv[2 * k + 1][1], wv[2 * k + 1][2], wv[2 * k + 1][3]};
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack2_bf16(__uint_as_float(xv[e] << 16) * w8[2 * e],
                        __uint_as_float(xv[e] & 0xffff0000u) * w8[2 * e + 1]);
    xt[k] = __builtin_bit_cast(bf16x8_t, o);
  }

  // ---- G1: C.B^T tiles masked per head into M
  tile_mask(W, S, t0, kOffDt + BUF * Q * 4);
  if (more) issue_part(nl, W, 1, BUF ^ 1);
  if (W.w < 2) {
    Tile t1 = tile_load(W, 8 + W.w, bbuf, cbuf);
    tile_mask(W, S, t1, kOffDt + BUF * Q * 4);
  }
  if (W.have_h) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) W.y[tt] *= ev[tt];
  } else {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) W.y[tt] = zero4();
  }

  // ---- G3: h^T <- lam h^T + B^T (w x)
  if (more) issue_part(nl, W, 2, BUF ^ 1);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < 2; ++k)
      op[2 * i + k] = cat8(ld_tr(bbuf + W.bt_base[0] + ((32 * i) ^ W.bt_xor[0]) + k * 32 * kRowB),
                           ld_tr(bbuf + W.bt_base[1] + ((32 * i) ^ W.bt_xor[1]) + k * 32 * kRowB));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    W.h[i] *= lam;
    pin(op[2 * i]);
    pin(op[2 * i + 1]);
#pragma unroll
    for (int k = 0; k < 2; ++k) W.h[i] = mfma(op[2 * i + k], xt[k], W.h[i]);
  }
  // the decay of state tile i + 1 is issued beside tile i's products
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMA
  }

  // checkpoints: the post-token state of t1 - 1
  const int hh = S.h0 + q;
  const size_t PN = (size_t)SP * SN;
  bool stored = false;
  for (int c = S.ck; c < ck_next; ++c) {
    float *dst = a.ckpt_out + ((size_t)m.ck_idx[c] * d.H + hh) * PN + (16 * W.ps + li) * SN + 4 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(f32x4_t *)(dst + 16 * i) = W.h[i];
    stored = true;
  }
  W.have_h = true;
  S.ck = ck_next;
  // the next block's dt has landed (wave 0 issued it before six more copies)
  if (more && W.w == 0) __asm__ volatile("s_waitcnt vmcnt(6)" ::: "memory");
  lds_barrier();  // [B] M is written; the next block's dt is visible

  // ---- G2: y^T[p,t] += sum_s x^T[p,s] M^T[s,t], s <= t
  const int mb = kOffM + q * kMHeadB;
  bf16x8_t mo[6];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) mo[tt] = ld_lds<bf16x8_t>(mb + tt * 16 * 128 + W.o_m[0]);
#pragma unroll
  for (int tt = 2; tt < 4; ++tt) mo[2 + tt] = ld_lds<bf16x8_t>(mb + tt * 16 * 128 + W.o_m[1]);
  // the next block's sums, while M is read (this block's were last read by G3)
  if (more && sums_wave(W)) block_sums(W, S, BUF ^ 1, S.n1 - S.n0, W.q);
#pragma unroll
  for (int i = 0; i < 6; ++i) pin(mo[i]);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) W.y[tt] = mfma(xk[0], mo[tt], W.y[tt]);
#pragma unroll
  for (int tt = 2; tt < 4; ++tt) W.y[tt] = mfma(xk[1], mo[2 + tt], W.y[tt]);
  // ---- y: lane (t = 16 tt + li, p = 16 ps + 4g .. +3), 8 bytes per store
  bf16_t *yb = (bf16_t *)a.y + ((size_t)S.t0 * d.H + hh) * SP + 16 * W.ps + 4 * g;
  const size_t ys = (size_t)d.H * SP;
  if (full) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) *(u32x2_t *)(yb + (16 * tt + li) * ys) = pk4(W.y[tt]);
  } else {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      if (16 * tt + li < len) *(u32x2_t *)(yb + (16 * tt + li) * ys) = pk4(W.y[tt]);
  }
  W.stores4 = full && !stored;
  S.t0 = S.n0;
  S.t1 = S.n1;
  return more;
}

__global__ __launch_bounds__(kPairThreads, 1) void scan_ssd_pair_kernel(ScanArgs a, ScanMeta m) {
  const Dims d = a.d;
  const int npair = d.H / 2;
  const int pair = blockIdx.x % npair;
  const ScanSeg sg = m.seg[blockIdx.x / npair];
  Wave W;
  Seg S;
  W.lane = threadIdx.x & 63;
  W.li = W.lane & 15;
  W.g = W.lane >> 4;
  W.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  W.q = W.w >> 2;
  W.ps = W.w & 3;
  S.h0 = 2 * pair;
  S.grp = S.h0 / (d.H / d.G);
  const float kLog2e = 1.4426950408889634f;
  S.al2[0] = a.A[S.h0] * kLog2e;
  S.al2[1] = a.A[S.h0 + 1] * kLog2e;
  S.Dq[0] = a.D[S.h0];
  S.Dq[1] = a.D[S.h0 + 1];
  const int li = W.li, g = W.g;

  // ---- per-lane LDS offsets
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // n = 32k + 8g .. +7 of row li
    W.o_c[k] = c_off(li, 4 * k + g);
    W.o_b1[k] = tile_off(li, 4 * k + g);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * g + 4 * r + (li >> 2);
    W.o_x[r] = tile_off(row, 8 * W.q + 2 * W.ps + ((li >> 1) & 1)) + 8 * (li & 1);
    // chunk 2i + b of the row sits at (2i + b) ^ f = 2 (i ^ (f >> 1)) + (b ^ (f & 1))
    const int f = fsw(row), b = (li >> 1) & 1;
    W.bt_base[r] = row * kRowB + 16 * (b ^ (f & 1)) + 8 * (li & 1);
    W.bt_xor[r] = 32 * (f >> 1);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) W.o_m[k] = m_off(li, 4 * k + g);
  W.sums = kOffSums + W.q * kSumsB;
  {
    const size_t sCB = (size_t)d.G * SN * 2, sX = (size_t)d.H * SP * 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * W.w + 4 * u + g;
      const int lc = (li ^ fsw(r)) << 4;
      W.v_b[u] = (uint32_t)(r * sCB + lc);
      W.v_x[u] = (uint32_t)(r * sX + lc);
      W.v_c[u] = (uint32_t)(r * sCB + ((li ^ (r & 15)) << 4));
    }
  }
  // M tiles above the diagonal that G2 reads (t tile 0 x s tile 1, t tile 2 x
  // s tile 3) stay zero; nothing else writes them
  {
    const int tid = threadIdx.x;  // 2 heads x 2 tiles x 16 rows x 2 chunks = 128 stores
    if (tid < 128) {
      const int hq = tid >> 6, tile = (tid >> 5) & 1, row = (tid >> 1) & 15, c = tid & 1;
      const int t = 32 * tile + row, chunk = 2 * (2 * tile + 1) + c;
      st_lds<u32x4_t>(kOffM + hq * kMHeadB + m_off(t, chunk), u32x4_t{0, 0, 0, 0});
    }
  }

  // ---- state in
  const size_t PN = (size_t)SP * SN;
  const int hh = S.h0 + W.q;
  float *seg_state = a.state + (size_t)sg.slot * a.d.H * PN;
  W.have_h = sg.init != 0;
  if (W.have_h) {
    const float *src = seg_state + hh * PN + (16 * W.ps + li) * SN + 4 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) W.h[i] = *(const f32x4_t *)(src + 16 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) W.h[i] = zero4();
  }
  S.ck = 0;
  while (S.ck < a.n_ck && m.ck_t[S.ck] < sg.t0) ++S.ck;
  S.seg_end = sg.t1;
  S.t0 = sg.t0;
  S.t1 = block_end(a, m, S.t0, S.seg_end, S.ck);
  {
    const Loads l0 = prepare_loads(a, W, S, 0, S.t0, S.t1 - S.t0);
    issue_part(l0, W, 0, 0);
    issue_part(l0, W, 1, 0);
    issue_part(l0, W, 2, 0);
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if (sums_wave(W)) block_sums(W, S, 0, S.t1 - S.t0, W.q);
  W.stores4 = false;

  while (pair_block<0>(a, m, W, S) && pair_block<1>(a, m, W, S)) {
  }

  if (sg.final) {
    float *dst = (sg.final == 1 ? seg_state : a.workspace) + hh * PN + (16 * W.ps + li) * SN + 4 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(f32x4_t *)(dst + 16 * i) = W.h[i];
  }
}

}  // namespace

bool ssd_pair_supported(const ScanArgs &a) {
  return a.d.H % 2 == 0 && (a.d.H / a.d.G) % 2 == 0 && ((uintptr_t)a.dt & 3) == 0;
}

hipError_t launch_scan_ssd_pair(const ScanArgs &a, const ScanMeta &m, hipStream_t s) {
  hipError_t err = allow_dynamic_lds(reinterpret_cast<const void *>(scan_ssd_pair_kernel), kSmemB);
  if (err != hipSuccess) return err;
  dim3 grid(a.n_seg * (a.d.H / 2)), block(kPairThreads);
  hipLaunchKernelGGL(scan_ssd_pair_kernel, grid, block, kSmemB, s, a, m);
  return hipGetLastError();
}

}  // namespace ssm
