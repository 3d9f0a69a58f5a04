// ssm_internal.h -- launch-side declarations shared by the host runtime
// (ssm_host.cpp) and the kernels (*.hip).  Library-internal: not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssm_stream.h"

namespace ssm {

// Batch entries per launch for decode / copy / replay.  Per-entry metadata
// travels in the kernel arguments (no staging copies, nothing to allocate);
// larger batches are split into several launches by the host.
constexpr int kBatchPerLaunch = 256;
// Segments (runs between resets) and checkpoints per scan launch.
constexpr int kSegPerLaunch = 32;
constexpr int kCkptPerLaunch = 64;
// Rows of one workgroup's state tile and threads per workgroup.
constexpr int kRows = 64;
constexpr int kThreads = 256;
// Largest supported state size N (one float4 per lane of a 32-lane row group).
constexpr int kMaxN = 128;
// Largest replay window and in-flight count.
constexpr int kMaxW = 64;
constexpr int kMaxInFlight = 16;

enum IoType { kF32 = 0, kBF16 = 2 };

struct Dims {
  int H, P, N, G;
  int PT;  // ceil(P / kRows): row tiles per head
};

// ---------------------------------------------------------------- decode
// Entry k of a launch is row k of x, dt, B, C and y.  One 32-bit word per
// entry (read through the scalar cache): the slot id in bits 0-30, the reset
// flag in bit 31.
constexpr uint32_t kDecodeReset = 0x80000000u;
struct DecodeMeta {
  uint32_t slot_rst[kBatchPerLaunch];
};
struct DecodeArgs {
  const void *x, *dt, *B, *C;  // this launch's first batch entry
  void *y;
  float *state;
  const float *A, *D;
  Dims d;
  int n;  // entries in this launch
};
hipError_t launch_decode(int io, const DecodeArgs &a, const DecodeMeta &m, hipStream_t s);

// ------------------------------------------------------------ copy baseline
struct CopyMeta {
  int32_t slot[kBatchPerLaunch];
  int8_t src[kBatchPerLaunch];  // -1: read the slot state; k: read copy k
};
struct CopyArgs {
  const void *x, *dt, *B, *C;  // [n, n_in, ...] for this launch
  const void *beta;            // Gated DeltaNet: [n, n_in, H]
  void *y;
  const float *state;
  float *copies;  // [S, n_in_max, H, P, N]
  const float *A, *D;
  Dims d;
  int n, n_in, n_in_max;
};
hipError_t launch_copy(int io, const CopyArgs &a, const CopyMeta &m, hipStream_t s);
// The same baseline for the Gated DeltaNet recurrence (x = v, B = k, C = q).
hipError_t launch_gdn_copy(int io, const CopyArgs &a, const CopyMeta &m, hipStream_t s);

// ------------------------------------------------------------------ replay
// Per entry: the slot and one 32-bit word (read through the scalar cache) with
// the entries folded into the checkpoint first (bits 0-7, 0: none), the
// committed entries the in-flight tokens follow (bits 8-15), the half read by
// the fold (bit 16) and the half of the live log (bit 17).
struct ReplayMeta {
  int32_t slot[kBatchPerLaunch];
  uint32_t info[kBatchPerLaunch];
};
__host__ __device__ inline uint32_t replay_info(int fold_len, int base_len, int fold_half,
                                                int live_half) {
  return (uint32_t)fold_len | (uint32_t)base_len << 8 | (uint32_t)fold_half << 16 |
         (uint32_t)live_half << 17;
}
__host__ __device__ inline int info_fold(uint32_t u) { return (int)(u & 0xffu); }
__host__ __device__ inline int info_base(uint32_t u) { return (int)((u >> 8) & 0xffu); }
__host__ __device__ inline int info_fold_half(uint32_t u) { return (int)((u >> 16) & 1u); }
__host__ __device__ inline int info_live_half(uint32_t u) { return (int)((u >> 17) & 1u); }
// Bits 18-25: the entry's row in the launch's inputs, outputs and B.C scratch
// (set by the launcher; a launch may carry a subset of the batch's entries).
__host__ __device__ inline uint32_t info_with_entry(uint32_t u, int e) {
  return (u & 0x3ffffu) | (uint32_t)e << 18;
}
__host__ __device__ inline int info_entry(uint32_t u) { return (int)((u >> 18) & 0xffu); }
// Row stride (floats) of the B.C scratch: one row per in-flight token, the
// window's entries along it, rounded up to whole 16-byte chunks.
__host__ __device__ inline int bc_stride(int W) { return (W + 3) & ~3; }
// Multiplier of the kernels' division by a small divisor d (FastDiv):
// ceil(2^32 / d) for d > 1.
__host__ __device__ inline uint32_t fastdiv_magic(int d) {
  return d > 1 ? 0xffffffffu / (uint32_t)d + 1u : 0u;
}

struct ReplayArgs {
  const void *x, *dt, *B, *C;  // [n, n_in, ...] for this launch
  const void *beta;            // Gated DeltaNet: [n, n_in, H]
  void *y;
  float *state;                // checkpoints [S, H, P, N]
  void *log;                   // [S][2][W] entries (see log_offsets)
  float *bc;                   // scratch [n][G][W + n_in][n_in] inside the log buffer tail
  const float *A, *D;
  Dims d;
  int n, n_in, W;
  uint32_t nin_magic;          // fastdiv_magic(n_in)
  int vrows, xrows;            // LDS rows reserved for B/C rows and x rows (set by the launcher)
};
// Log layout: arrays of [S][2 halves][W entries][...] in the io dtype (dt:
// [H], x: [H*P], B: [G*N]; Gated DeltaNet also beta: [H]), then for Mamba-2
// the fp32 B.C scratch.
struct LogLayout {
  size_t dt_off, beta_off, x_off, B_off, bc_off, total;  // byte offsets
};
LogLayout log_layout(int io, const Dims &d, int S, int W, bool gdn);
hipError_t launch_replay(int io, const ReplayArgs &a, const ReplayMeta &m, const LogLayout &lay,
                         hipStream_t s);
// ReplaySSM verify of the Gated DeltaNet recurrence (x = v, B = k, C = q):
// the same metadata and log halves, the gated delta rule for the fold.
hipError_t launch_gdn_replay(int io, const ReplayArgs &a, const ReplayMeta &m,
                             const LogLayout &lay, hipStream_t s);

// -------------------------------------------------------------------- scan
struct ScanSeg {
  int32_t t0, t1;   // token range [t0, t1) of the chunk
  int32_t init;     // 1: start from the segment's state; 0: from zero
  int32_t final;    // 0: drop; 1: write the segment's state; 2: write the workspace
  int32_t slot;     // the segment's state is state + slot * H*P*N
};
struct ScanMeta {
  ScanSeg seg[kSegPerLaunch];
  int32_t ck_t[kCkptPerLaunch];    // token index (post-token state)
  int32_t ck_idx[kCkptPerLaunch];  // destination index into ckpt_out
};
struct ScanArgs {
  const void *x, *dt, *B, *C;
  void *y;
  float *state;      // [.., H, P, N]: segment i reads/writes state[seg[i].slot]
  float *workspace;  // [H, P, N] or null
  float *ckpt_out;   // [n_ckpt, H, P, N]
  const float *A, *D;
  Dims d;
  int n_seg, n_ck;
};
hipError_t launch_scan(int io, const ScanArgs &a, const ScanMeta &m, hipStream_t s);
// SSD/MFMA form of the scan: bf16 inputs with P = 64 and N = 128 (x, B, C
// 16-byte aligned).
bool ssd_supported(int io, const Dims &d);
hipError_t launch_scan_ssd(const ScanArgs &a, const ScanMeta &m, hipStream_t s);
// The same form for a pair of heads per workgroup (heads 2i, 2i+1 share a B/C
// group): H and H/G even, dt 4-byte aligned.
bool ssd_pair_supported(const ScanArgs &a);
hipError_t launch_scan_ssd_pair(const ScanArgs &a, const ScanMeta &m, hipStream_t s);

// -------------------------------------------------- scan, tile-parallel form
// Tiles of kChunkTile tokens; at most kChunkTilesPerLaunch tiles per launch
// (longer chunks run as consecutive pieces, each carrying the state through
// the slot buffer).
constexpr int kChunkTile = 64;
constexpr int kChunkTilesPerLaunch = 64;
struct ChunkMeta {
  uint64_t rmask[kChunkTilesPerLaunch];  // bit j: reset before token j of the tile
  int32_t ck_t[kCkptPerLaunch];          // chunk token index (post-token state)
  int32_t ck_idx[kCkptPerLaunch];        // destination index into ckpt_out
};
struct ChunkArgs {
  const void *x, *dt, *B, *C;  // the whole chunk (token 0 of the chunk)
  void *y;
  float *state;     // the slot's [H, P, N]: carry-in, then carry-out
  float *ws;        // [n_tiles][H][P][N]: tile states, then tile carry-ins
  float *lam;       // [n_tiles][H]: tile decays (0: a reset inside the tile)
  float *ckpt_out;  // [n_ckpt, H, P, N]
  const float *A, *D;
  Dims d;
  int t0, len;      // this piece: tokens [t0, t0 + len) of the chunk
  int n_tiles, n_ck;
};
// Shapes the tile-parallel form covers (P in {32, 64}, N a multiple of 32 up
// to 128); workspace floats it needs for a chunk of L tokens.
bool chunk_supported(int io, const Dims &d);
size_t chunk_ws_floats(const Dims &d, int64_t L);
hipError_t launch_chunk(int io, const ChunkArgs &a, const ChunkMeta &m, hipStream_t s);

// ------------------------------------------------------ static device scratch
// A file-scope device array (ssm_static.hip): the workspace of
// ssm_scan_chunk_static, then the finite-check flag.
constexpr size_t kStaticFlagOff = SSM_STATIC_WORKSPACE_BYTES;
constexpr size_t kStaticScratchBytes = kStaticFlagOff + 256;
// This device's copy of the array (its address looked up once per device).
hipError_t static_scratch(void **out);

// --------------------------------------------------------------- state ops
hipError_t launch_zero(float *dst, size_t n_floats, hipStream_t s);
hipError_t launch_copy_f32(float *dst, const float *src, size_t n_floats, hipStream_t s);
// sum_i w_i * (2*i + 1) mod 2^64 over the 32-bit words of src; *acc must be
// zeroed first (launch_zero_u64).
hipError_t launch_checksum(const float *src, size_t n_words, unsigned long long *acc,
                           hipStream_t s);
hipError_t launch_zero_u64(unsigned long long *p, int n, hipStream_t s);
// Sets *flag to 1 if any of the n elements (io dtype) is not finite.
hipError_t launch_finite_check(int io, const void *p, size_t n, unsigned int *flag,
                               hipStream_t s);

// ------------------------------------------------- conv1d and gated output
// Causal depthwise conv over the token axis (width K <= kMaxConvK) with the
// carried conv state [C, K-1] (the K-1 previous inputs, oldest first).
constexpr int kMaxConvK = 4;
constexpr int kConvResetsPerLaunch = 32;
struct ConvChunkMeta {
  int32_t n_rst;                       // resets inside [t_begin, t_end)
  int32_t rst[kConvResetsPerLaunch];   // their token indices, ascending
  int32_t first_before;                // latest reset before t_begin; -K: none (state visible)
};
struct ConvArgs {
  const void *x;          // chunk: [L, C]; decode: [batch, C] (io dtype)
  void *y;                // same layout
  float *state;           // chunk: the slot's [C, K-1]; decode: every slot's [S, C, K-1]
  const float *w, *bias;  // [C, K], [C] or null
  int C, K, act;          // act: 1 = SiLU
  int t_begin, t_end;     // chunk: the token range of this launch
  int n;                  // decode: entries in this launch
};
hipError_t launch_conv_chunk(int io, const ConvArgs &a, const ConvChunkMeta &m, hipStream_t s);
// after every launch of a chunk: the state becomes the last K-1 inputs
// (first_final: latest reset in the chunk, or -K)
hipError_t launch_conv_state(int io, const ConvArgs &a, int L, int first_final, hipStream_t s);
hipError_t launch_conv_decode(int io, const ConvArgs &a, const DecodeMeta &m, hipStream_t s);
// y * SiLU(z), then (norm_w non-null) each group of `group` channels divided
// by its root mean square and scaled by norm_w
hipError_t launch_gate(int io, int64_t rows, int C, int group, const void *y, const void *z,
                       const float *norm_w, float eps, void *out, hipStream_t s);

}  // namespace ssm
