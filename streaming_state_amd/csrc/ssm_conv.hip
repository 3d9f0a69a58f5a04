// ssm_conv.hip -- the steps on either side of the scan: the causal depthwise
// conv1d over the token axis with its carried conv state, and the gated
// output y * SiLU(z) with an optional group RMS norm.
//
//   y[t, c] = act( b[c] + sum_{k=0}^{K-1} w[c, k] x[t - (K-1) + k, c] )
//
// Tap K-1 meets the current token; act is SiLU or the identity.  The conv
// state of a stream is the K-1 inputs before its next token, oldest first
// ([C, K-1] fp32 per slot); a reset on token t hides every input before t.
// (The Mamba-2 block's definitions: the pages name the conv state as half of
// a Mamba layer's state but define neither step.)
//
// All three are streaming kernels bound by HBM: each thread loads everything
// it needs before its first store (on gfx9 a wait for a load also waits for
// the stores issued before it).
#include "ssm_device.h"

namespace ssm {

namespace {

__device__ __forceinline__ float silu(float v) { return __fdividef(v, 1.f + __expf(-v)); }
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16_t v) { return bf16_to_f(v); }

// V consecutive io elements as floats (V = 4: one 16- or 8-byte access)
template <typename T, int V> struct Vec;
template <typename T> struct Vec<T, 1> {
  static __device__ __forceinline__ void ld(const T *p, float *v) { v[0] = Io<T>::ld(p); }
  static __device__ __forceinline__ void st(T *p, const float *v) { Io<T>::st(p, v[0]); }
};
template <typename T> struct Vec<T, 4> {
  static __device__ __forceinline__ void ld(const T *p, float *v) {
    const float4 f = Io<T>::ld4(p);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
  static __device__ __forceinline__ void st(T *p, const float *v) {
    Io<T>::st4(p, make_float4(v[0], v[1], v[2], v[3]));
  }
};

template <> struct Vec<bf16_t, 8> {
  static __device__ __forceinline__ void ld(const bf16_t *p, float *v) {
    const uint4 r = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st(bf16_t *p, const float *v) {
    uint4 r;
    r.x = pack2_bf16(v[0], v[1]);
    r.y = pack2_bf16(v[2], v[3]);
    r.z = pack2_bf16(v[4], v[5]);
    r.w = pack2_bf16(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = r;
  }
};
template <> struct Vec<float, 8> {
  static __device__ __forceinline__ void ld(const float *p, float *v) {
    Vec<float, 4>::ld(p, v);
    Vec<float, 4>::ld(p + 4, v + 4);
  }
};

// Raw V-element vectors (bf16 stays packed in registers until used).
template <typename T, int V> struct Raw;
template <> struct Raw<float, 4> {
  typedef float4 type;
  static __device__ __forceinline__ type ld(const float *p) { return *reinterpret_cast<const float4 *>(p); }
  static __device__ __forceinline__ float get(const type &r, int v) {
    return v == 0 ? r.x : v == 1 ? r.y : v == 2 ? r.z : r.w;
  }
  static __device__ __forceinline__ type zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};
template <> struct Raw<bf16_t, 4> {
  typedef uint2 type;
  static __device__ __forceinline__ type ld(const bf16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
  static __device__ __forceinline__ float get(const type &r, int v) {
    const uint32_t w = v < 2 ? r.x : r.y;
    return __uint_as_float((v & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  static __device__ __forceinline__ type zero() { return make_uint2(0u, 0u); }
};
template <typename T> struct Raw<T, 1> {
  typedef T type;
  static __device__ __forceinline__ type ld(const T *p) { return *p; }
  static __device__ __forceinline__ float get(const type &r, int) { return to_f(r); }
  static __device__ __forceinline__ type zero() { return T{}; }
};
// Tokens per thread in the chunk kernel: all of a thread's inputs (its tokens
// and the K-1 before them) are loaded before any output is stored.
constexpr int kConvRun = 32;

// Grid (channel groups of blockDim.x * V, token runs of kConvRun).  The K-1
// window entries before the run are held as fp32 (they may come from the
// carried state), the run's own inputs as raw io vectors (bf16 stays packed).
// A run is "clean" when it is whole, has no reset inside and its window needs
// neither the carried state nor a zeroed entry: the common case takes a copy
// of the code without predicates.  Otherwise a reset at run position r zeroes
// the entries of the tokens before it; every index into the register arrays
// is a compile-time constant, so they stay in registers.
template <typename T, int K, int V>
__global__ __launch_bounds__(kThreads) void conv_chunk_kernel(ConvArgs a, ConvChunkMeta m) {
  typedef Raw<T, V> R;
  const int c0 = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (c0 >= a.C) return;
  const int C = a.C;
  const int t0 = a.t_begin + blockIdx.y * kConvRun;
  const int n = min(kConvRun, a.t_end - t0);
  const T *x = (const T *)a.x + c0;
  T *y = (T *)a.y + c0;
  constexpr int KW = K - 1;

  // latest reset at or before t0 (resets are uniform: kernel arguments)
  int first = m.first_before, ri = 0;
  while (ri < m.n_rst && m.rst[ri] <= t0) first = m.rst[ri++];
  const bool clean = n == kConvRun && t0 - KW >= max(first, 0) &&
                     (ri >= m.n_rst || m.rst[ri] >= t0 + kConvRun);

  float win[KW > 0 ? KW : 1][V];
  typename R::type run[kConvRun];
  float w[K][V], b[V];
  // entry j of the combined window + run, channel v
  auto in = [&](int j, int v) { return j < KW ? win[j][v] : R::get(run[j - KW], v); };
  auto emit = [&](int i) {
    float out[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float acc = b[v];
#pragma unroll
      for (int k = 0; k < K; ++k) acc += w[k][v] * in(i + k, v);
      out[v] = a.act ? silu(acc) : acc;
    }
    Vec<T, V>::st(y + (size_t)(t0 + i) * C, out);
  };
  if (clean) {
#pragma unroll
    for (int j = 0; j < KW; ++j) Vec<T, V>::ld(x + (size_t)(t0 - KW + j) * C, win[j]);
#pragma unroll
    for (int i = 0; i < kConvRun; ++i) run[i] = R::ld(x + (size_t)(t0 + i) * C);
  } else {
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const int src = t0 - KW + j;
      if (src >= first && src >= 0) {
        Vec<T, V>::ld(x + (size_t)src * C, win[j]);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
          win[j][v] = (src >= first) ? a.state[(size_t)(c0 + v) * KW + (src + KW)] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < kConvRun; ++i) run[i] = i < n ? R::ld(x + (size_t)(t0 + i) * C) : R::zero();
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) w[k][v] = a.w[(size_t)(c0 + v) * K + k];
    b[v] = a.bias ? a.bias[c0 + v] : 0.f;
  }
  if (clean) {
#pragma unroll
    for (int i = 0; i < kConvRun; ++i) emit(i);
    return;
  }
#pragma unroll
  for (int i = 0; i < kConvRun; ++i) {
    if (i < n) {
      if (ri < m.n_rst && m.rst[ri] == t0 + i) {  // hide the inputs before token t0 + i
        ++ri;
#pragma unroll
        for (int j = i; j < i + KW; ++j) {
          if (j < KW) {
#pragma unroll
            for (int v = 0; v < V; ++v) win[j][v] = 0.f;
          } else {
            run[j - KW] = R::zero();
          }
        }
      }
      emit(i);
    }
  }
}

// Thread per channel: the state becomes the last K-1 inputs of the chunk
// (older ones from the old state when the chunk is shorter than K-1), with
// the entries before the chunk's latest reset zeroed.
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void conv_state_kernel(ConvArgs a, int L, int first_final) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= a.C) return;
  constexpr int KW = K - 1;
  float *st = a.state + (size_t)c * KW;
  const T *x = (const T *)a.x + c;
  float old[KW > 0 ? KW : 1], nw[KW > 0 ? KW : 1];
#pragma unroll
  for (int j = 0; j < KW; ++j) old[j] = st[j];
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    const int src = L - KW + j;
    nw[j] = src < first_final ? 0.f : src < 0 ? old[src + KW] : to_f(x[(size_t)src * a.C]);
  }
#pragma unroll
  for (int j = 0; j < KW; ++j) st[j] = nw[j];
}

// Grid (channel blocks, entries): one token per slot.
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void conv_decode_kernel(ConvArgs a, DecodeMeta m) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= a.C) return;
  const int e = blockIdx.y;
  const uint32_t sr = m.slot_rst[e];
  const int slot = (int)(sr & ~kDecodeReset);
  const bool rst = (sr & kDecodeReset) != 0;
  constexpr int KW = K - 1;
  float *st = a.state + ((size_t)slot * a.C + c) * KW;
  float win[KW > 0 ? KW : 1];
#pragma unroll
  for (int j = 0; j < KW; ++j) win[j] = rst ? 0.f : st[j];
  const float xv = Io<T>::ld((const T *)a.x + (size_t)e * a.C + c);
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = a.w[(size_t)c * K + k];
  float acc = a.bias ? a.bias[c] : 0.f;
#pragma unroll
  for (int k = 0; k < KW; ++k) acc += w[k] * win[k];
  acc += w[KW] * xv;
  Io<T>::st((T *)a.y + (size_t)e * a.C + c, a.act ? silu(acc) : acc);
#pragma unroll
  for (int j = 0; j + 1 < KW; ++j) st[j] = win[j + 1];
  if (KW > 0) st[KW - 1] = xv;
}

// y * SiLU(z), elementwise (no norm).
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void gate_kernel(const T *y, const T *z, T *out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * V;
  if (i >= n) return;
  float yv[V], zv[V], o[V];
  Vec<T, V>::ld(y + i, yv);
  Vec<T, V>::ld(z + i, zv);
#pragma unroll
  for (int v = 0; v < V; ++v) o[v] = yv[v] * silu(zv[v]);
  Vec<T, V>::st(out + i, o);
}

// Gated group RMS norm: one workgroup per (row, group).  g = y * SiLU(z) is
// computed once and kept in registers (32 values per thread) while the
// group's sum of squares is reduced; groups larger than that take two passes,
// recomputing g from y and z (still in L2) in the second.  bf16 groups of a
// multiple of 8 use 16-byte vectors.
constexpr int kGateRegs = 8;

__device__ __forceinline__ float block_sum(float v, float *part) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) tot += part[i];
  return tot;
}

template <typename T, int V>
__global__ __launch_bounds__(kThreads) void gate_norm_kernel(const T *y, const T *z,
                                                             const float *w, int C, int group,
                                                             float eps, T *out) {
  __shared__ float part[kThreads / 64];
  const size_t base = (size_t)blockIdx.x * C + (size_t)blockIdx.y * group;
  const float *wg = w + (size_t)blockIdx.y * group;
  const int nv = group / V;  // vectors in the group
  constexpr int kRegs = kGateRegs * 4 / V;
  if (nv <= kThreads * kRegs) {
    float g[kRegs][V];
    float ss = 0.f;
    // the weights (shared by every row, so L2 hits) are in flight with y and z
    float wv[kRegs][V];
#pragma unroll
    for (int u = 0; u < kRegs; ++u) {
      const int i = threadIdx.x + u * kThreads;
      if (i < nv) Vec<float, V>::ld(wg + (size_t)i * V, wv[u]);
    }
#pragma unroll
    for (int u = 0; u < kRegs; ++u) {
      const int i = threadIdx.x + u * kThreads;
      float yv[V], zv[V];
      if (i < nv) {
        Vec<T, V>::ld(y + base + (size_t)i * V, yv);
        Vec<T, V>::ld(z + base + (size_t)i * V, zv);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v) yv[v] = zv[v] = 0.f;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        g[u][v] = yv[v] * silu(zv[v]);
        ss += g[u][v] * g[u][v];
      }
    }
    const float inv = rsqrtf(block_sum(ss, part) / (float)group + eps);
#pragma unroll
    for (int u = 0; u < kRegs; ++u) {
      const int i = threadIdx.x + u * kThreads;
      if (i < nv) {
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = g[u][v] * inv * wv[u][v];
        Vec<T, V>::st(out + base + (size_t)i * V, o);
      }
    }
    return;
  }
  constexpr int U = 4;
  float ss = 0.f;
  for (int i0 = threadIdx.x; i0 < nv; i0 += kThreads * U) {
    float yv[U][V], zv[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      if (i < nv) {
        Vec<T, V>::ld(y + base + (size_t)i * V, yv[u]);
        Vec<T, V>::ld(z + base + (size_t)i * V, zv[u]);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v) yv[u][v] = zv[u][v] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float gv = yv[u][v] * silu(zv[u][v]);
        ss += gv * gv;
      }
  }
  const float inv = rsqrtf(block_sum(ss, part) / (float)group + eps);
  for (int i0 = threadIdx.x; i0 < nv; i0 += kThreads * U) {
    float yv[U][V], zv[U][V], wv[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      if (i < nv) {
        Vec<T, V>::ld(y + base + (size_t)i * V, yv[u]);
        Vec<T, V>::ld(z + base + (size_t)i * V, zv[u]);
        Vec<float, V>::ld(wg + (size_t)i * V, wv[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      if (i < nv) {
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = yv[u][v] * silu(zv[u][v]) * inv * wv[u][v];
        Vec<T, V>::st(out + base + (size_t)i * V, o);
      }
    }
  }
}

// Threads per block (a multiple of 64, at most kThreads) that leaves the
// fewest idle threads over `units` channel vectors.
static int fit_block(int units) {
  int best = kThreads, waste = (units + kThreads - 1) / kThreads * kThreads - units;
  for (int b = kThreads - 64; b >= 64; b -= 64) {
    const int w = (units + b - 1) / b * b - units;
    if (w < waste) best = b, waste = w;
  }
  return best;
}

template <typename T, int K>
hipError_t conv_chunk_k(const ConvArgs &a, const ConvChunkMeta &m, hipStream_t s) {
  const int runs = (a.t_end - a.t_begin + kConvRun - 1) / kConvRun;
  const bool v4 = a.C % 4 == 0 && ((((uintptr_t)a.x | (uintptr_t)a.y) & (4 * sizeof(T) - 1)) == 0);
  if (v4) {
    const int b = fit_block(a.C / 4);
    dim3 grid((a.C / 4 + b - 1) / b, runs);
    hipLaunchKernelGGL((conv_chunk_kernel<T, K, 4>), grid, dim3(b), 0, s, a, m);
  } else {
    const int b = fit_block(a.C);
    dim3 grid((a.C + b - 1) / b, runs);
    hipLaunchKernelGGL((conv_chunk_kernel<T, K, 1>), grid, dim3(b), 0, s, a, m);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t conv_chunk_t(const ConvArgs &a, const ConvChunkMeta &m, hipStream_t s) {
  switch (a.K) {
    case 1: return conv_chunk_k<T, 1>(a, m, s);
    case 2: return conv_chunk_k<T, 2>(a, m, s);
    case 3: return conv_chunk_k<T, 3>(a, m, s);
    default: return conv_chunk_k<T, 4>(a, m, s);
  }
}

template <typename T>
hipError_t conv_state_t(const ConvArgs &a, int L, int ff, hipStream_t s) {
  const dim3 grid((a.C + kThreads - 1) / kThreads), block(kThreads);
  switch (a.K) {
    case 1: return hipSuccess;  // no state
    case 2: hipLaunchKernelGGL((conv_state_kernel<T, 2>), grid, block, 0, s, a, L, ff); break;
    case 3: hipLaunchKernelGGL((conv_state_kernel<T, 3>), grid, block, 0, s, a, L, ff); break;
    default: hipLaunchKernelGGL((conv_state_kernel<T, 4>), grid, block, 0, s, a, L, ff); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t conv_decode_t(const ConvArgs &a, const DecodeMeta &m, hipStream_t s) {
  const dim3 grid((a.C + kThreads - 1) / kThreads, a.n), block(kThreads);
  switch (a.K) {
    case 1: hipLaunchKernelGGL((conv_decode_kernel<T, 1>), grid, block, 0, s, a, m); break;
    case 2: hipLaunchKernelGGL((conv_decode_kernel<T, 2>), grid, block, 0, s, a, m); break;
    case 3: hipLaunchKernelGGL((conv_decode_kernel<T, 3>), grid, block, 0, s, a, m); break;
    default: hipLaunchKernelGGL((conv_decode_kernel<T, 4>), grid, block, 0, s, a, m); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t gate_t(int64_t rows, int C, int group, const void *y, const void *z, const float *w,
                  float eps, void *out, hipStream_t s) {
  const T *yp = (const T *)y, *zp = (const T *)z;
  T *op = (T *)out;
  const bool aligned4 = ((((uintptr_t)y | (uintptr_t)z | (uintptr_t)out)) & (4 * sizeof(T) - 1)) == 0;
  if (!w) {
    const int64_t n = rows * C;
    if (n % 4 == 0 && aligned4) {
      const int64_t blocks = (n / 4 + kThreads - 1) / kThreads;
      hipLaunchKernelGGL((gate_kernel<T, 4>), dim3((unsigned)blocks), dim3(kThreads), 0, s, yp, zp,
                         op, n);
    } else {
      const int64_t blocks = (n + kThreads - 1) / kThreads;
      hipLaunchKernelGGL((gate_kernel<T, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, s, yp, zp,
                         op, n);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)rows, C / group);
  if (sizeof(T) == 2 && group % 8 == 0 &&
      ((((uintptr_t)y | (uintptr_t)z | (uintptr_t)out | (uintptr_t)w)) & 15) == 0)
    hipLaunchKernelGGL((gate_norm_kernel<bf16_t, 8>), grid, dim3(kThreads), 0, s,
                       (const bf16_t *)y, (const bf16_t *)z, w, C, group, eps, (bf16_t *)out);
  else if (group % 4 == 0 && aligned4 && ((uintptr_t)w & 15) == 0)
    hipLaunchKernelGGL((gate_norm_kernel<T, 4>), grid, dim3(kThreads), 0, s, yp, zp, w, C, group,
                       eps, op);
  else
    hipLaunchKernelGGL((gate_norm_kernel<T, 1>), grid, dim3(kThreads), 0, s, yp, zp, w, C, group,
                       eps, op);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_chunk(int io, const ConvArgs &a, const ConvChunkMeta &m, hipStream_t s) {
  if (a.t_end <= a.t_begin) return hipSuccess;
  return io == kBF16 ? conv_chunk_t<bf16_t>(a, m, s) : conv_chunk_t<float>(a, m, s);
}

hipError_t launch_conv_state(int io, const ConvArgs &a, int L, int first_final, hipStream_t s) {
  return io == kBF16 ? conv_state_t<bf16_t>(a, L, first_final, s)
                     : conv_state_t<float>(a, L, first_final, s);
}

hipError_t launch_conv_decode(int io, const ConvArgs &a, const DecodeMeta &m, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  return io == kBF16 ? conv_decode_t<bf16_t>(a, m, s) : conv_decode_t<float>(a, m, s);
}

hipError_t launch_gate(int io, int64_t rows, int C, int group, const void *y, const void *z,
                       const float *norm_w, float eps, void *out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return io == kBF16 ? gate_t<bf16_t>(rows, C, group, y, z, norm_w, eps, out, s)
                     : gate_t<float>(rows, C, group, y, z, norm_w, eps, out, s);
}

}  // namespace ssm
