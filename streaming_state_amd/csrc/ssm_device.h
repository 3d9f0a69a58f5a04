// ssm_device.h -- device helpers shared by the library's kernels: io-dtype
// loads/stores (fp32 or bf16 bits), the 64-row state-tile thread layout and
// the cross-lane row reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "ssm_internal.h"

namespace ssm {

// ------------------------------------------------------- launch attributes
// Allow `kernel` `bytes` of dynamic LDS on the current device.  Above the
// default 64 KiB the limit must be raised with hipFuncSetAttribute; it
// persists, so it is raised once per (kernel, device, size) rather than on
// every launch.
inline hipError_t allow_dynamic_lds(const void *kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  struct Set {
    const void *kernel;
    int dev;
    size_t bytes;
  };
  static std::mutex mu;
  static std::vector<Set> done;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lk(mu);
  for (const Set &e : done)
    if (e.kernel == kernel && e.dev == dev && e.bytes >= bytes) return hipSuccess;
  err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess) done.push_back(Set{kernel, dev, bytes});
  return err;
}

// ------------------------------------------------------------------ io types
// fp32 is stored as float, bf16 as its 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// Round to nearest even with the hardware conversion (v_cvt_pk_bf16_f32 on
// gfx950, two values per instruction); NaN stays NaN.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const bf16x2_hw v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Io;
template <> struct Io<float> {
  static __device__ __forceinline__ float ld(const float *p) { return *p; }
  static __device__ __forceinline__ float4 ld4(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
  }
  static __device__ __forceinline__ void st(float *p, float v) { *p = v; }
  static __device__ __forceinline__ void st4(float *p, float4 v) {
    *reinterpret_cast<float4 *>(p) = v;
  }
};
template <> struct Io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t *p) { return bf16_to_f(*p); }
  static __device__ __forceinline__ float4 ld4(const bf16_t *p) {
    uint2 r = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  }
  static __device__ __forceinline__ void st(bf16_t *p, float v) { *p = f_to_bf16(v); }
  static __device__ __forceinline__ void st4(bf16_t *p, float4 v) {
    uint2 r;
    r.x = pack2_bf16(v.x, v.y);
    r.y = pack2_bf16(v.z, v.w);
    *reinterpret_cast<uint2 *>(p) = r;
  }
};

// -------------------------------------------------------- state-tile layout
// A group of 256 threads (4 waves) owns an (8*R)-row x N tile of one head's
// fp32 state.  Lane l of wave w holds float4 column c = l & 31 (state entries
// n = 4c..4c+3) of rows r_i = 8*i + 2*w + (l >> 5), i = 0..R-1.  One wave-wide
// load instruction therefore covers two adjacent rows (2 * 512 B contiguous
// at N = 128).  With kContig the R rows of a lane are consecutive instead,
// r_i = R*(2*w + (l >> 5)) + i, so per-row values staged in LDS are read as
// whole vectors; each load instruction then covers two separate full rows.
template <int R, bool kContig = false>
struct TileR {
  static constexpr int kRowsPerTile = 8 * R;
  int lane, wave, c, rsub;
  __device__ __forceinline__ TileR() {
    lane = threadIdx.x & 63;
    wave = (threadIdx.x >> 6) & 3;  // wave within the tile's 256 threads
    c = lane & 31;
    rsub = lane >> 5;
  }
  __device__ __forceinline__ int row(int i) const {
    return kContig ? R * (2 * wave + rsub) + i : 8 * i + 2 * wave + rsub;
  }
  // Row (within the tile) whose total this lane holds after reduce_rows<R>().
  __device__ __forceinline__ int reduced_row() const {
    const int b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
    const int i = R == 8 ? b4 * 4 + b3 * 2 + b2 : R == 4 ? b4 * 2 + b3 : b4;
    return row(i);
  }
  // One lane of each group that holds the same reduced total.
  __device__ __forceinline__ bool reduced_writer() const {
    return R == 8 ? (lane & 3) == 0 : R == 4 ? (lane & 7) == 0 : (lane & 15) == 0;
  }
};
typedef TileR<8> Tile;

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float4 fma4(float s, float4 h, float u, float4 b) {
  return make_float4(s * h.x + u * b.x, s * h.y + u * b.y, s * h.z + u * b.z, s * h.w + u * b.w);
}
__device__ __forceinline__ float4 scale4(float4 h, float s) {
  return make_float4(s * h.x, s * h.y, s * h.z, s * h.w);
}

// Sum eight per-row partials across the 32 lanes of a row group by recursive
// halving: each exchange step halves the number of values a lane carries.
// Returns the total of row reduced_row() of the calling lane.
__device__ __forceinline__ float halve(float lo, float hi, int bit, int mask) {
  float send = bit ? lo : hi;
  float recv = __shfl_xor(send, mask);
  return (bit ? hi : lo) + recv;
}
__device__ __forceinline__ float reduce8(const float v[8], int lane) {
  const int b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
  float s4[4], s2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = halve(v[i], v[i + 4], b4, 16);
#pragma unroll
  for (int i = 0; i < 2; ++i) s2[i] = halve(s4[i], s4[i + 2], b3, 8);
  float s = halve(s2[0], s2[1], b2, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  return s;
}
// Four-row variant: after two halving steps each lane holds one row; the
// remaining three exchanges finish the 32-lane sum.
__device__ __forceinline__ float reduce4(const float v[4], int lane) {
  const int b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1;
  float s2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) s2[i] = halve(v[i], v[i + 2], b4, 16);
  float s = halve(s2[0], s2[1], b3, 8);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  return s;
}
// Two-row variant.
__device__ __forceinline__ float reduce2(const float v[2], int lane) {
  float s = halve(v[0], v[1], (lane >> 4) & 1, 16);
  s += __shfl_xor(s, 8);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  return s;
}
template <int R> __device__ __forceinline__ float reduce_rows(const float v[R], int lane);
template <> __device__ __forceinline__ float reduce_rows<2>(const float v[2], int lane) {
  return reduce2(v, lane);
}
template <> __device__ __forceinline__ float reduce_rows<8>(const float v[8], int lane) {
  return reduce8(v, lane);
}
template <> __device__ __forceinline__ float reduce_rows<4>(const float v[4], int lane) {
  return reduce4(v, lane);
}

// The same row totals with VALU lane moves only (no LDS round trips): the
// 32-lane halving step pairs lane j of a 16-lane row with lane j of the next
// row (v_permlane16_swap), the 8- and 4-lane steps pair mirrored lanes
// (DPP row_mirror, row_half_mirror), and the last two sums run inside quads.
// A lane keeps the same half as in the xor form, so reduced_row() and
// reduced_writer() hold for it too; only the association of the sum differs.
template <int kCtrl> __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E;  // quad_perm [1,0,3,2], [2,3,0,1]
// lanes of even rows keep lo, of odd rows hi; each gets its half's total over the row pair
__device__ __forceinline__ float halve_rows(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// bit set: keep hi, else lo; the partner is the mirrored lane (opposite bit)
template <int kCtrl> __device__ __forceinline__ float halve_mirror(float lo, float hi, int bit) {
  return (bit ? hi : lo) + dpp_f<kCtrl>(bit ? lo : hi);
}
template <int R> __device__ __forceinline__ float row_totals(const float v[R], int lane);
template <> __device__ __forceinline__ float row_totals<8>(const float v[8], int lane) {
  const int b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
  float s4[4], s2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = halve_rows(v[i], v[i + 4]);
#pragma unroll
  for (int i = 0; i < 2; ++i) s2[i] = halve_mirror<kDppRowMirror>(s4[i], s4[i + 2], b3);
  float s = halve_mirror<kDppRowHalfMirror>(s2[0], s2[1], b2);
  s += dpp_f<kDppQuadXor2>(s);
  s += dpp_f<kDppQuadXor1>(s);
  return s;
}
template <> __device__ __forceinline__ float row_totals<4>(const float v[4], int lane) {
  const int b3 = (lane >> 3) & 1;
  float s2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) s2[i] = halve_rows(v[i], v[i + 2]);
  float s = halve_mirror<kDppRowMirror>(s2[0], s2[1], b3);
  s += dpp_f<kDppRowHalfMirror>(s);
  s += dpp_f<kDppQuadXor2>(s);
  s += dpp_f<kDppQuadXor1>(s);
  return s;
}
template <> __device__ __forceinline__ float row_totals<2>(const float v[2], int lane) {
  float s = halve_rows(v[0], v[1]);
  s += dpp_f<kDppRowMirror>(s);
  s += dpp_f<kDppRowHalfMirror>(s);
  s += dpp_f<kDppQuadXor2>(s);
  s += dpp_f<kDppQuadXor1>(s);
  return s;
}

// Register tile of the verify kernels: each wave owns 16 state rows (four
// waves a 64-row tile, eight a 128-row one); lane l of wave w owns rows
// 16 w + 2 (l >> 3) + {0, 1} and, of each,
// the four 16-byte column chunks 32 q + 4 (l & 7), q = 0..3 (8 float4).  A
// wave load instruction then reads eight whole 128-byte lines, and the total
// of a row needs only the eight lanes of its group: one mirrored exchange
// that leaves each lane one of its two rows, then two sums inside quads.
struct ReplayTile {
  int lane, wave, c, rg;
  __device__ __forceinline__ ReplayTile() {
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    c = lane & 7;
    rg = lane >> 3;
  }
  __device__ __forceinline__ int row(int i) const { return 16 * wave + 2 * rg + i; }
  __device__ __forceinline__ int col(int q) const { return 32 * q + 4 * c; }
  // after totals(): the row whose total this lane holds, and one writer per total
  __device__ __forceinline__ int reduced_row() const { return row((lane >> 2) & 1); }
  __device__ __forceinline__ bool reduced_writer() const { return (lane & 3) == 0; }
  __device__ __forceinline__ float totals(float p0, float p1) const {
    float s = halve_mirror<kDppRowHalfMirror>(p0, p1, (lane >> 2) & 1);
    s += dpp_f<kDppQuadXor2>(s);
    s += dpp_f<kDppQuadXor1>(s);
    return s;
  }
  // the total of one row's eight partials, in all eight lanes of its group
  __device__ __forceinline__ static float row_sum(float p) {
    p += dpp_f<kDppQuadXor1>(p);
    p += dpp_f<kDppQuadXor2>(p);
    p += dpp_f<kDppRowHalfMirror>(p);
    return p;
  }
};

// Two consecutive io values from LDS (8-byte aligned for fp32, 4 for bf16).
__device__ __forceinline__ void lds_ld_pair(const float *p, float v[2]) {
  const float2 u = *reinterpret_cast<const float2 *>(p);
  v[0] = u.x;
  v[1] = u.y;
}
__device__ __forceinline__ void lds_ld_pair(const bf16_t *p, float v[2]) {
  const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
  v[0] = __uint_as_float(u << 16);
  v[1] = __uint_as_float(u & 0xffff0000u);
}

// Sum over the 32 lanes of a row group with DPP lane moves (no LDS round
// trip; the latency-critical form for the sequential scan).  Rotations by 1,
// 2, 4 and 8 inside each 16-lane row leave every lane with its row's sum;
// row_bcast:15 then adds row 0's sum into row 1 (and row 2's into row 3).
// The 32-lane total is valid in lanes 16..31 and 48..63.
#define SSM_DPP_ADD(v, ctrl)                                                                 \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), (ctrl), 0xF, 0xF, false))
__device__ __forceinline__ float sum32_dpp(float v) {
  SSM_DPP_ADD(v, 0x121);  // row_ror:1
  SSM_DPP_ADD(v, 0x122);  // row_ror:2
  SSM_DPP_ADD(v, 0x124);  // row_ror:4
  SSM_DPP_ADD(v, 0x128);  // row_ror:8
  // row_bcast:15 into rows 1 and 3 only (row_mask 0b1010)
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  return v;
}
// Inclusive prefix sum over the 64 lanes of a wave (lane l gets the sum of
// lanes 0..l) with DPP lane moves: shifts by 1, 2, 4 and 8 inside each
// 16-lane row (lanes shifted in from outside the row add 0), then row 0's
// total into row 1 and row 2's into row 3 (row_bcast:15), then the total of
// rows 0-1 into rows 2 and 3 (row_bcast:31).  Every partial is a sum of
// consecutive lanes' values, so nonnegative inputs lose nothing to
// cancellation.  All 64 lanes must be active.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  SSM_DPP_ADD(v, 0x111);  // row_shr:1
  SSM_DPP_ADD(v, 0x112);  // row_shr:2
  SSM_DPP_ADD(v, 0x114);  // row_shr:4
  SSM_DPP_ADD(v, 0x118);  // row_shr:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return v;
}
#undef SSM_DPP_ADD

// Division of an index i < 2^16 by a block-uniform divisor 1 <= d < 2^16:
// the high word of i * ceil(2^32 / d) is floor(i / d) in that range (the
// rounding error of the multiplier, below d / 2^32 per unit of i, cannot
// reach the next integer).  d = 1 is passed through (its multiplier would be 2^32).
struct FastDiv {
  uint32_t d, m;
  __device__ __forceinline__ explicit FastDiv(int dv) : d((uint32_t)dv), m(fastdiv_magic(dv)) {}
  // with the multiplier computed by the host (fastdiv_magic)
  __device__ __forceinline__ FastDiv(int dv, uint32_t mv) : d((uint32_t)dv), m(mv) {}
  __device__ __forceinline__ int div(int i) const {
    return d > 1 ? (int)__umulhi((uint32_t)i, m) : i;
  }
};

// Streaming (nontemporal) 128-bit state accesses: the state is touched once
// per step and the working set is far larger than the caches.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 nt_load4(const float *p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store4(float *p, float4 v) {
  const f32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t *>(p));
}

// ------------------------------------------------------------ LDS staging
typedef __attribute__((address_space(3))) void lds_void_t;

// Copy n 16-byte chunks global -> LDS: chunk i lands at lds + 16 i, read from
// src_of(i).  Each wave instruction fills 64 consecutive chunks (lane l
// writes 16 bytes at the wave's LDS base + 16 l; inactive lanes write
// nothing).  The copies complete asynchronously: wait on vmcnt before use.
template <int kWaves = kThreads / 64, typename SrcOf>
__device__ __forceinline__ void stage_lds(char *lds, int n, SrcOf src_of) {
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int blk = wave; blk * 64 < n; blk += kWaves) {
    const int i = blk * 64 + lane;
    if (i < n)
      __builtin_amdgcn_global_load_lds(src_of(i), (lds_void_t *)(lds + blk * 1024), 16, 0, 0);
  }
}

template <typename T> __device__ __forceinline__ float4 lds_ld4(const T *p);
template <> __device__ __forceinline__ float4 lds_ld4<float>(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
template <> __device__ __forceinline__ float4 lds_ld4<bf16_t>(const bf16_t *p) {
  const uint2 r = *reinterpret_cast<const uint2 *>(p);
  return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                     __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}

// R consecutive io values from LDS (16-byte aligned) as floats.
template <typename T, int R> __device__ __forceinline__ void lds_ld_rows(const T *p, float *v) {
  static_assert((R * sizeof(T)) % 16 == 0, "whole 16-byte reads");
#pragma unroll
  for (int q = 0; q < (int)(R * sizeof(T)) / 16; ++q) {
    const uint4 u = reinterpret_cast<const uint4 *>(p)[q];
    if (sizeof(T) == 4) {
      v[4 * q + 0] = __uint_as_float(u.x);
      v[4 * q + 1] = __uint_as_float(u.y);
      v[4 * q + 2] = __uint_as_float(u.z);
      v[4 * q + 3] = __uint_as_float(u.w);
    } else {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[8 * q + 2 * t] = __uint_as_float(w[t] << 16);
        v[8 * q + 2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
      }
    }
  }
}

// Sum over the 32 lanes of a row group (lanes 0-31 or 32-63), left in every
// one of them: rotations by 1, 2, 4 and 8 inside each 16-lane row give each
// lane its row's sum, and v_permlane16_swap adds the other row of the pair.
__device__ __forceinline__ float allsum32(float v) {
  v += dpp_f<0x121>(v);  // row_ror:1
  v += dpp_f<0x122>(v);  // row_ror:2
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same over all 64 lanes of the wave (v_permlane32_swap adds the halves).
__device__ __forceinline__ float allsum64(float v) {
  v = allsum32(v);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ----------------------------------------------------------- wave prefix sum
// Inclusive prefix sum over the 64 lanes: shifts of 1, 2, 4, 8 within each
// 16-lane row, then row 15's and row 31's totals broadcast forward.
__device__ __forceinline__ float scan64(float v) {
  const int z = 0;
#define SSD_SHR(ctrl, rmask)                                                               \
  v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), ctrl, rmask, 0xF, true))
  SSD_SHR(0x111, 0xF);  // row_shr:1
  SSD_SHR(0x112, 0xF);  // row_shr:2
  SSD_SHR(0x114, 0xF);  // row_shr:4
  SSD_SHR(0x118, 0xF);  // row_shr:8
  SSD_SHR(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
  SSD_SHR(0x143, 0xC);  // row_bcast:31 into rows 2 and 3
#undef SSD_SHR
  return v;
}

}  // namespace ssm
