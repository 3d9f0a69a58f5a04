// ssm_host.cpp -- host runtime behind include/ssm_stream.h: handles, argument
// and lifecycle validation, exact integer metadata (positions, chunk sequence
// numbers, replay log lengths, live copies), and kernel launches on the
// caller's stream.  Every check runs before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <utility>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "ssm_stream.h"
#include "ssm_internal.h"

using namespace ssm;

namespace {

constexpr uint64_t kCodeRev = 1;

thread_local std::string t_err;

ssm_status fail(ssm_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_err = buf;
  return st;
}

enum Pend { kNone = 0, kReplayPend = 1, kCopyPend = 2 };

struct Slot {
  int64_t pos = 0;
  uint64_t chunk_seq = 0;
  uint64_t stream_id = 0;
  int log_len = 0;    // committed replay log entries
  int log_half = 0;   // half of the log that holds them
  int pend = kNone;   // a verify step awaits commit
  int pend_n = 0;     // its n_in
  int pend_base = 0;  // replay: committed length the step saw
  int live = -1;      // copy baseline: live copy index, -1 = the state buffer
};

struct Handle {
  ssm_layer_desc desc;
  Dims d;
  int io;
  int rec;  // SSM_MAMBA2 or SSM_GATED_DELTA
  int S;
  float *state;
  const float *A, *D;
  uint32_t flags;
  std::vector<Slot> slots;
  std::vector<uint32_t> stamp;  // per-slot epoch marks for distinctness checks
  uint32_t epoch = 0;
  // replay
  int W = 0;
  void *log = nullptr;
  LogLayout lay{};
  // copy baseline
  int n_in_max = 0;
  float *copies = nullptr;
  // causal conv before the scan (0 channels: not attached)
  int conv_C = 0, conv_K = 0, conv_act = 0;
  float *conv_state = nullptr;  // [S, C, K-1]
  const float *conv_w = nullptr, *conv_b = nullptr;
  // device scratch slice (checksum accumulators, finite flag) and its device
  void *scratch = nullptr;
  int scratch_dev = 0;
  ssm_counters cnt{};
  size_t state_bytes() const { return (size_t)d.H * d.P * d.N * sizeof(float); }
  float *slot_state(int s) const { return state + (size_t)s * d.H * d.P * d.N; }
  size_t conv_floats() const { return (size_t)conv_C * (conv_K > 0 ? conv_K - 1 : 0); }
};

std::mutex g_mu;
std::unordered_map<int64_t, Handle *> g_handles;
int64_t g_next_handle = 1;
uint64_t g_next_stream = 1;

Handle *lookup(ssm_handle h) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_handles.find(h);
  return it == g_handles.end() ? nullptr : it->second;
}

uint64_t new_stream_id() {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_next_stream++;
}

#define GET_HANDLE(var, h)                                                              \
  Handle *var = lookup(h);                                                              \
  if (!var) return fail(SSM_E_INVALID_STATE, "handle %lld is not live", (long long)(h))

#define HIP_TRY(expr)                                                          \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess)                                                      \
      return fail(SSM_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));   \
  } while (0)

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

size_t io_size(int io) { return io == kBF16 ? 2 : 4; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The kernels load B and C rows four elements at a time and the state as
// float4: x, dt, y must be aligned to the element size, B and C to four
// elements, fp32 state buffers to 16 bytes.
ssm_status check_io_align(int io, const void *x, const void *dt, const void *B, const void *C,
                          const void *y, const char *what) {
  const size_t es = io_size(io);
  if (!aligned(x, es) || !aligned(dt, es) || !aligned(y, es) || !aligned(B, 4 * es) ||
      !aligned(C, 4 * es))
    return fail(SSM_E_INVALID_ARG, "%s: misaligned input or output pointer", what);
  return SSM_OK;
}

ssm_status check_desc(const ssm_layer_desc *desc) {
  if (!desc) return fail(SSM_E_INVALID_ARG, "desc is NULL");
  if (desc->H < 1 || desc->P < 1 || desc->G < 1 || desc->H % desc->G != 0)
    return fail(SSM_E_INVALID_ARG, "need H, P, G >= 1 and H %% G == 0 (H=%d P=%d G=%d)",
                desc->H, desc->P, desc->G);
  if (desc->N < 4 || desc->N > kMaxN || desc->N % 4 != 0)
    return fail(SSM_E_INVALID_ARG, "N must be a multiple of 4 in [4, %d] (N=%d)", kMaxN,
                desc->N);
  if (desc->io_dtype != SSM_F32 && desc->io_dtype != SSM_BF16)
    return fail(SSM_E_INVALID_ARG, "io_dtype %d not supported (fp32 or bf16)", desc->io_dtype);
  if (desc->recurrence != SSM_MAMBA2 && desc->recurrence != SSM_GATED_DELTA)
    return fail(SSM_E_INVALID_ARG, "unknown recurrence %d", desc->recurrence);
  return SSM_OK;
}

// Calls of one recurrence refuse handles of the other.
ssm_status need_rec(const Handle *H, int rec, const char *what) {
  if (H->rec == rec) return SSM_OK;
  return fail(SSM_E_INVALID_ARG, "%s: this handle holds a %s layer", what,
              H->rec == SSM_GATED_DELTA ? "Gated DeltaNet" : "Mamba-2");
}

Dims dims_of(const ssm_layer_desc *desc) {
  return Dims{desc->H, desc->P, desc->N, desc->G, (desc->P + kRows - 1) / kRows};
}

// Shortest chunk that takes the tile-parallel form: below it the three passes
// cost more than walking the tokens.
constexpr int64_t kChunkMinTokens = 64;

// Validate a batch of slot ids: in range and pairwise distinct.
ssm_status check_slots(Handle *H, int n, const int32_t *slots, const char *what) {
  if (n < 0) return fail(SSM_E_INVALID_ARG, "%s: negative count", what);
  if (n > 0 && !slots) return fail(SSM_E_INVALID_ARG, "%s: slot ids are NULL", what);
  if (++H->epoch == 0) {
    std::fill(H->stamp.begin(), H->stamp.end(), 0u);
    H->epoch = 1;
  }
  for (int i = 0; i < n; ++i) {
    const int s = slots[i];
    if (s < 0 || s >= H->S) return fail(SSM_E_INVALID_ARG, "%s: slot %d out of range", what, s);
    if (H->stamp[s] == H->epoch) return fail(SSM_E_INVALID_ARG, "%s: slot %d repeated", what, s);
    H->stamp[s] = H->epoch;
  }
  return SSM_OK;
}

// Per-handle device scratch: kSums checksum accumulators (u64), then the
// finite-check flag.
constexpr size_t kScratchBytes = 4096;
constexpr int kSums = 256;
constexpr size_t kFlagOff = kSums * sizeof(unsigned long long);
static_assert(kFlagOff + sizeof(unsigned int) <= kScratchBytes, "scratch layout");

// Scratch slices come from a per-device pool that is never freed: every call
// that uses a handle's slice synchronises its stream before it returns, so a
// slice returned by ssm_destroy is idle and can serve the next handle without
// any device-wide wait (hipFree would synchronise the whole device).
constexpr int kSlicesPerBlock = 64;
struct ScratchPool {
  std::mutex mu;
  std::unordered_map<int, std::vector<void *>> free_slices;  // by device
};
ScratchPool g_pool;

ssm_status ensure_scratch(Handle *H) {
  if (H->scratch) return SSM_OK;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_pool.mu);
  std::vector<void *> &fl = g_pool.free_slices[dev];
  if (fl.empty()) {
    char *block = nullptr;
    HIP_TRY(hipMalloc((void **)&block, kScratchBytes * kSlicesPerBlock));
    for (int i = kSlicesPerBlock - 1; i >= 0; --i) fl.push_back(block + i * kScratchBytes);
  }
  H->scratch = fl.back();
  H->scratch_dev = dev;
  fl.pop_back();
  return SSM_OK;
}

void release_scratch(Handle *H) {
  if (!H->scratch) return;
  std::lock_guard<std::mutex> lk(g_pool.mu);
  g_pool.free_slices[H->scratch_dev].push_back(H->scratch);
  H->scratch = nullptr;
}

// Device-side finite check of a list of io-dtype buffers; synchronises.  The
// flag (8 bytes of device memory) is the handle's scratch, or `fixed_flag`.
ssm_status check_finite(Handle *H, hipStream_t s,
                        std::initializer_list<std::pair<const void *, size_t>> bufs,
                        unsigned int *fixed_flag = nullptr) {
  if (!(H->flags & SSM_FLAG_CHECK_FINITE)) return SSM_OK;
  unsigned int *flag = fixed_flag;
  if (!flag) {
    ssm_status st = ensure_scratch(H);
    if (st != SSM_OK) return st;
    flag = reinterpret_cast<unsigned int *>((char *)H->scratch + kFlagOff);
  }
  HIP_TRY(launch_zero_u64(reinterpret_cast<unsigned long long *>(flag), 1, s));
  for (auto &b : bufs) HIP_TRY(launch_finite_check(H->io, b.first, b.second, flag, s));
  unsigned int host = 0;
  HIP_TRY(hipMemcpyAsync(&host, flag, sizeof host, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (host) return fail(SSM_E_INVALID_CHUNK, "non-finite input");
  return SSM_OK;
}

// Receipt checksums of n states srcs[i] (each [H,P,N] fp32, device), taken on
// the device in batches of kSums; synchronises the stream.
ssm_status device_checksums(Handle *H, const float *const *srcs, int n, hipStream_t s,
                            uint64_t *out) {
  ssm_status st = ensure_scratch(H);
  if (st != SSM_OK) return st;
  unsigned long long *acc = reinterpret_cast<unsigned long long *>(H->scratch);
  unsigned long long host[kSums];
  for (int i0 = 0; i0 < n; i0 += kSums) {
    const int k = std::min(kSums, n - i0);
    HIP_TRY(launch_zero_u64(acc, k, s));
    for (int i = 0; i < k; ++i)
      HIP_TRY(launch_checksum(srcs[i0 + i], H->state_bytes() / 4, acc + i, s));
    HIP_TRY(hipMemcpyAsync(host, acc, k * sizeof(unsigned long long), hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    for (int i = 0; i < k; ++i) out[i0 + i] = host[i];
  }
  return SSM_OK;
}

ssm_status device_checksum(Handle *H, const float *src, hipStream_t s, uint64_t *out) {
  return device_checksums(H, &src, 1, s, out);
}

// The receipt of a slot's current stream for a state whose checksum is `sum`.
ssm_receipt slot_receipt(const Handle *H, const Slot &sl, uint64_t sum);

ssm_status slot_is_plain(Handle *H, int s, const char *what) {
  const Slot &sl = H->slots[s];
  if (sl.pend != kNone)
    return fail(SSM_E_LOG, "%s: slot %d has a verify step awaiting commit", what, s);
  if (sl.log_len > 0 || sl.live >= 0)
    return fail(SSM_E_LOG, "%s: slot %d holds a replay log or live copy (materialize it first)",
                what, s);
  return SSM_OK;
}

void fresh_stream(Slot &sl) {
  sl.pos = 0;
  sl.chunk_seq = 0;
  sl.stream_id = new_stream_id();
  sl.log_len = 0;
  sl.pend = kNone;
  sl.pend_n = 0;
  sl.live = -1;
}

// Fold the replay log of the given slots into their checkpoints (n_in = 0).
ssm_status fold_logs(Handle *H, const std::vector<int> &slots, hipStream_t s) {
  for (size_t i0 = 0; i0 < slots.size(); i0 += kBatchPerLaunch) {
    const int n = (int)std::min<size_t>(kBatchPerLaunch, slots.size() - i0);
    ReplayMeta m;
    for (int i = 0; i < n; ++i) {
      Slot &sl = H->slots[slots[i0 + i]];
      m.slot[i] = slots[i0 + i];
      m.info[i] = replay_info(sl.log_len, 0, sl.log_half, 1 - sl.log_half);
    }
    ReplayArgs a{};
    a.state = H->state;
    a.log = H->log;
    a.bc = reinterpret_cast<float *>((char *)H->log + H->lay.bc_off);
    a.A = H->A;
    a.D = H->D;
    a.d = H->d;
    a.n = n;
    a.n_in = 0;
    a.W = H->W;
    a.nin_magic = fastdiv_magic(a.n_in);
    if (H->rec == SSM_GATED_DELTA)
      HIP_TRY(launch_gdn_replay(H->io, a, m, H->lay, s));
    else
      HIP_TRY(launch_replay(H->io, a, m, H->lay, s));
  }
  for (int sidx : slots) {
    Slot &sl = H->slots[sidx];
    sl.log_half = 1 - sl.log_half;
    sl.log_len = 0;
    H->cnt.replay_flushes++;
    H->cnt.state_bytes_read += H->state_bytes();
    H->cnt.state_bytes_written += H->state_bytes();
  }
  return SSM_OK;
}

ssm_status materialize(Handle *H, int n, const int32_t *slots, hipStream_t s) {
  std::vector<int> folds;
  for (int i = 0; i < n; ++i) {
    const Slot &sl = H->slots[slots[i]];
    if (sl.pend != kNone)
      return fail(SSM_E_LOG, "materialize: slot %d has a verify step awaiting commit", slots[i]);
  }
  for (int i = 0; i < n; ++i) {
    Slot &sl = H->slots[slots[i]];
    if (sl.log_len > 0) folds.push_back(slots[i]);
  }
  if (!folds.empty()) {
    ssm_status st = fold_logs(H, folds, s);
    if (st != SSM_OK) return st;
  }
  const size_t nf = H->state_bytes() / 4;
  for (int i = 0; i < n; ++i) {
    Slot &sl = H->slots[slots[i]];
    if (sl.live >= 0) {
      const float *src = H->copies + ((size_t)slots[i] * H->n_in_max + sl.live) * nf;
      HIP_TRY(launch_copy_f32(H->slot_state(slots[i]), src, nf, s));
      sl.live = -1;
    }
  }
  return SSM_OK;
}

ssm_receipt slot_receipt(const Handle *H, const Slot &sl, uint64_t sum) {
  ssm_receipt r{};
  r.stream_id = sl.stream_id;
  r.model_rev = H->desc.model_rev;
  r.code_rev = kCodeRev;
  r.schema_version = H->desc.schema_version;
  r.state_dtype = SSM_F32;
  r.H = H->d.H;
  r.P = H->d.P;
  r.N = H->d.N;
  r.G = H->d.G;
  r.position = sl.pos;
  r.chunk_seq = sl.chunk_seq;
  r.checksum = sum;
  r.recurrence = (uint32_t)H->rec;
  return r;
}

// Launch the per-segment forms of the scan over `segs` (in token order): the
// head-pair or one-head SSD kernel for bf16 with P = 64, N = 128, the
// recurrent kernel otherwise.  Segment i starts from state[segs[i].slot] (or
// zero) and ends in it (or the workspace, or nowhere: see ScanSeg).  The
// state right after token ck_at[i] goes to ckpt_out[i].
ssm_status launch_seg_forms(Handle *H, float *state, float *ws, const std::vector<ScanSeg> &segs,
                            const void *x, const void *dt, const void *B, const void *C, void *y,
                            int n_ckpt, const int64_t *ck_at, float *ckpt_out, hipStream_t s) {
  const bool ssd = ssd_supported(H->io, H->d);
  for (size_t i0 = 0; i0 < segs.size(); i0 += kSegPerLaunch) {
    const int ns = (int)std::min<size_t>(kSegPerLaunch, segs.size() - i0);
    ScanMeta m{};
    for (int i = 0; i < ns; ++i) m.seg[i] = segs[i0 + i];
    if (ssd)  // longest segments first: one workgroup per (segment, head) runs it in order
      std::stable_sort(m.seg, m.seg + ns, [](const ScanSeg &a, const ScanSeg &b) {
        return a.t1 - a.t0 > b.t1 - b.t0;
      });
    const int32_t lo = segs[i0].t0, hi = segs[i0 + ns - 1].t1;
    int nck = 0;
    for (int i = 0; i < n_ckpt; ++i)
      if (ck_at[i] >= lo && ck_at[i] < hi) {
        m.ck_t[nck] = (int32_t)ck_at[i];
        m.ck_idx[nck] = i;
        ++nck;
      }
    ScanArgs a{};
    a.x = x;
    a.dt = dt;
    a.B = B;
    a.C = C;
    a.y = y;
    a.state = state;
    a.workspace = ws;
    a.ckpt_out = ckpt_out;
    a.A = H->A;
    a.D = H->D;
    a.d = H->d;
    a.n_seg = ns;
    a.n_ck = nck;
    if (ssd && ssd_pair_supported(a))
      HIP_TRY(launch_scan_ssd_pair(a, m, s));
    else if (ssd)
      HIP_TRY(launch_scan_ssd(a, m, s));
    else
      HIP_TRY(launch_scan(H->io, a, m, s));
  }
  return SSM_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char *ssm_last_error(void) { return t_err.c_str(); }
uint64_t ssm_code_rev(void) { return kCodeRev; }

ssm_status ssm_create(const ssm_layer_desc *desc, int32_t n_slots, float *d_state,
                      const float *d_A, const float *d_D, uint32_t flags, ssm_handle *out) {
  ssm_status st = check_desc(desc);
  if (st != SSM_OK) return st;
  if (!out) return fail(SSM_E_INVALID_ARG, "out is NULL");
  if (n_slots < 1) return fail(SSM_E_INVALID_ARG, "n_slots must be >= 1");
  if (!d_state || !d_A || (!d_D && desc->recurrence == SSM_MAMBA2))
    return fail(SSM_E_INVALID_ARG, "state, A and (for Mamba-2) D are required");
  if (flags & ~SSM_FLAG_CHECK_FINITE) return fail(SSM_E_INVALID_ARG, "unknown flags 0x%x", flags);
  if (!aligned(d_state, 16)) return fail(SSM_E_INVALID_ARG, "state must be 16-byte aligned");
  Handle *H = new Handle();
  H->desc = *desc;
  H->d = dims_of(desc);
  H->io = desc->io_dtype;
  H->rec = desc->recurrence;
  H->S = n_slots;
  H->state = d_state;
  H->A = d_A;
  H->D = d_D;
  H->flags = flags;
  H->slots.resize(n_slots);
  H->stamp.assign(n_slots, 0u);
  for (auto &sl : H->slots) fresh_stream(sl);
  std::lock_guard<std::mutex> lk(g_mu);
  const int64_t id = g_next_handle++;
  g_handles[id] = H;
  *out = id;
  return SSM_OK;
}

ssm_status ssm_destroy(ssm_handle h) {
  Handle *H = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_handles.find(h);
    if (it == g_handles.end())
      return fail(SSM_E_INVALID_STATE, "handle %lld is not live", (long long)h);
    H = it->second;
    g_handles.erase(it);
  }
  release_scratch(H);  // idle: its last user synchronised its stream
  delete H;
  return SSM_OK;
}

static ssm_status reset_or_init(ssm_handle h, int32_t n, const int32_t *slots, const float *init,
                                void *stream, const char *what) {
  GET_HANDLE(H, h);
  ssm_status st = check_slots(H, n, slots, what);
  if (st != SSM_OK) return st;
  for (int i = 0; i < n; ++i)
    if (H->slots[slots[i]].pend != kNone)
      return fail(SSM_E_LOG, "%s: slot %d has a verify step awaiting commit", what, slots[i]);
  hipStream_t s = as_stream(stream);
  const size_t nf = H->state_bytes() / 4;
  for (int i = 0; i < n; ++i) {
    if (init)
      HIP_TRY(launch_copy_f32(H->slot_state(slots[i]), init + (size_t)i * nf, nf, s));
    else
      HIP_TRY(launch_zero(H->slot_state(slots[i]), nf, s));
    if (H->conv_floats())  // both halves of the slot's state start fresh
      HIP_TRY(launch_zero(H->conv_state + (size_t)slots[i] * H->conv_floats(), H->conv_floats(), s));
  }
  for (int i = 0; i < n; ++i) fresh_stream(H->slots[slots[i]]);
  H->cnt.resets += n;
  H->cnt.state_bytes_written += (size_t)n * H->state_bytes();
  return SSM_OK;
}

ssm_status ssm_state_reset(ssm_handle h, int32_t n, const int32_t *h_slots, void *stream) {
  return reset_or_init(h, n, h_slots, nullptr, stream, "ssm_state_reset");
}

ssm_status ssm_state_init(ssm_handle h, int32_t n, const int32_t *h_slots, const float *d_init,
                          void *stream) {
  if (!d_init || !aligned(d_init, 16))
    return fail(SSM_E_INVALID_ARG, "ssm_state_init: d_init must be non-NULL and 16-byte aligned");
  return reset_or_init(h, n, h_slots, d_init, stream, "ssm_state_init");
}

// ------------------------------------------------------------------- scan
size_t ssm_scan_workspace_bytes(const ssm_layer_desc *desc, int64_t L) {
  if (check_desc(desc) != SSM_OK || L < 0) return 0;
  const Dims d = dims_of(desc);
  const size_t state = (size_t)d.H * d.P * d.N * sizeof(float);
  if (ssd_supported(desc->io_dtype, d) || !chunk_supported(desc->io_dtype, d) ||
      L < kChunkMinTokens)
    return state;
  return std::max(state, chunk_ws_floats(d, L) * sizeof(float));
}

// The chunk scan behind ssm_scan_chunk and ssm_scan_chunk_static.  With
// `fixed_flag` set, the workspace is the library's static scratch (its size is
// not the caller's to change) and the finite-check flag lives there too.
static ssm_status scan_chunk_impl(Handle *H, int32_t slot, uint64_t chunk_seq, int64_t L,
                                  const void *x, const void *dt, const void *B, const void *C,
                                  const uint8_t *h_reset, void *y, int32_t n_ckpt,
                                  const int64_t *h_ckpt_at, float *d_ckpt_out, void *d_workspace,
                                  size_t ws_bytes, unsigned int *fixed_flag, void *stream) {
  const bool fixed = fixed_flag != nullptr;
  if (ssm_status st0 = need_rec(H, SSM_MAMBA2, "scan"); st0 != SSM_OK) return st0;
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "scan: slot %d out of range", slot);
  Slot &sl = H->slots[slot];
  if (chunk_seq != sl.chunk_seq) {
    H->cnt.chunks_rejected++;
    return fail(SSM_E_SEQUENCE, "scan: slot %d expects chunk %llu, got %llu (%s)", slot,
                (unsigned long long)sl.chunk_seq, (unsigned long long)chunk_seq,
                chunk_seq < sl.chunk_seq ? "duplicate" : "reordered or gap");
  }
  ssm_status st = slot_is_plain(H, slot, "scan");
  if (st != SSM_OK) return st;
  if (L < 0 || L > (int64_t)INT32_MAX) return fail(SSM_E_INVALID_ARG, "scan: bad L %lld", (long long)L);
  if (n_ckpt < 0 || n_ckpt > kCkptPerLaunch)
    return fail(SSM_E_INVALID_ARG, "scan: n_ckpt must be in [0, %d]", kCkptPerLaunch);
  if (n_ckpt > 0 && (!h_ckpt_at || !d_ckpt_out))
    return fail(SSM_E_INVALID_ARG, "scan: checkpoints need h_ckpt_at and d_ckpt_out");
  for (int i = 0; i < n_ckpt; ++i) {
    if (h_ckpt_at[i] < 0 || h_ckpt_at[i] >= L)
      return fail(SSM_E_INVALID_ARG, "scan: checkpoint %d at token %lld outside [0, L)", i,
                  (long long)h_ckpt_at[i]);
    if (i > 0 && h_ckpt_at[i] <= h_ckpt_at[i - 1])
      return fail(SSM_E_INVALID_ARG, "scan: checkpoint tokens must increase");
  }
  if (L == 0) {  // an empty chunk is legal: it only advances the sequence number
    sl.chunk_seq++;
    H->cnt.chunks_admitted++;
    return SSM_OK;
  }
  if (!x || !dt || !B || !C || !y) return fail(SSM_E_INVALID_ARG, "scan: NULL input or output");
  st = check_io_align(H->io, x, dt, B, C, y, "scan");
  if (st != SSM_OK) return st;
  const bool ssd = ssd_supported(H->io, H->d);
  if (ssd && (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16)))
    return fail(SSM_E_INVALID_ARG, "scan: bf16 x, B and C must be 16-byte aligned");
  if ((n_ckpt > 0 && !aligned(d_ckpt_out, 16)) || !aligned(d_workspace, 16))
    return fail(SSM_E_INVALID_ARG, "scan: checkpoint and workspace buffers must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  // Tile-parallel form: long enough chunks of the shapes it covers, given the
  // workspace it needs; otherwise the recurrent form (same results up to
  // rounding order).
  const bool par = !ssd && chunk_supported(H->io, H->d) && L >= kChunkMinTokens &&
                   aligned(x, 4 * io_size(H->io)) && d_workspace &&
                   ws_bytes >= chunk_ws_floats(H->d, L) * sizeof(float);
  if (par) {
    st = check_finite(H, s, {{x, (size_t)L * H->d.H * H->d.P}, {dt, (size_t)L * H->d.H},
                             {B, (size_t)L * H->d.G * H->d.N}, {C, (size_t)L * H->d.G * H->d.N}}, fixed_flag);
    if (st != SSM_OK) return st;
    const int64_t piece = (int64_t)kChunkTile * kChunkTilesPerLaunch;
    for (int64_t t0 = 0; t0 < L; t0 += piece) {
      const int len = (int)std::min<int64_t>(piece, L - t0);
      ChunkArgs a{};
      ChunkMeta m{};
      a.x = x;
      a.dt = dt;
      a.B = B;
      a.C = C;
      a.y = y;
      a.state = H->slot_state(slot);
      a.ws = (float *)d_workspace;
      a.lam = a.ws + chunk_ws_floats(H->d, L) - (size_t)kChunkTilesPerLaunch * H->d.H;
      a.ckpt_out = d_ckpt_out;
      a.A = H->A;
      a.D = H->D;
      a.d = H->d;
      a.t0 = (int)t0;
      a.len = len;
      a.n_tiles = (len + kChunkTile - 1) / kChunkTile;
      if (h_reset)
        for (int j = 0; j < len; ++j)
          if (h_reset[t0 + j]) m.rmask[j / kChunkTile] |= 1ull << (j % kChunkTile);
      for (int i = 0; i < n_ckpt; ++i)
        if (h_ckpt_at[i] >= t0 && h_ckpt_at[i] < t0 + len) {
          m.ck_t[a.n_ck] = (int32_t)h_ckpt_at[i];
          m.ck_idx[a.n_ck] = i;
          ++a.n_ck;
        }
      HIP_TRY(launch_chunk(H->io, a, m, s));
    }
  }
  // segments: runs between resets
  std::vector<ScanSeg> segs;
  {
    int32_t t0 = 0;
    const bool first_init = !(h_reset && h_reset[0]);
    for (int64_t t = 1; t <= L; ++t) {
      if (t == L || (h_reset && h_reset[t])) {
        segs.push_back(ScanSeg{t0, (int32_t)t, (int32_t)(segs.empty() ? first_init : 0), 0, 0});
        t0 = (int32_t)t;
      }
    }
  }
  const bool need_ws = !par && segs.size() > 1 && segs.front().init;
  segs.back().final = need_ws ? 2 : 1;
  if (need_ws && (!d_workspace || ws_bytes < H->state_bytes())) {
    if (fixed)
      return fail(SSM_E_INVALID_ARG,
                  "scan (static scratch): this chunk carries state in and resets later; it "
                  "needs %zu bytes of workspace, above the static scratch's %zu (use "
                  "ssm_scan_chunk with a workspace, or split the chunk at the reset)",
                  H->state_bytes(), ws_bytes);
    return fail(SSM_E_INVALID_ARG,
                "scan: this chunk carries state in and resets later; it needs a workspace of "
                "%zu bytes",
                H->state_bytes());
  }
  if (!par) {
    st = check_finite(H, s, {{x, (size_t)L * H->d.H * H->d.P}, {dt, (size_t)L * H->d.H},
                             {B, (size_t)L * H->d.G * H->d.N}, {C, (size_t)L * H->d.G * H->d.N}},
                      fixed_flag);
    if (st != SSM_OK) return st;
  }
  if (!par) {
    st = launch_seg_forms(H, H->slot_state(slot), (float *)d_workspace, segs, x, dt, B, C, y,
                          n_ckpt, h_ckpt_at, d_ckpt_out, s);
    if (st != SSM_OK) return st;
  }
  if (need_ws)
    HIP_TRY(launch_copy_f32(H->slot_state(slot), (const float *)d_workspace,
                            H->state_bytes() / 4, s));
  // exact host metadata
  int64_t pos = sl.pos;
  for (int64_t t = 0; t < L; ++t) {
    if (h_reset && h_reset[t]) pos = 0;
    pos += 1;
  }
  sl.pos = pos;
  sl.chunk_seq++;
  H->cnt.chunks_admitted++;
  H->cnt.tokens_scanned += (uint64_t)L;
  if (segs.front().init) H->cnt.state_bytes_read += H->state_bytes();
  H->cnt.state_bytes_written += H->state_bytes() * (1 + (size_t)n_ckpt);
  return SSM_OK;
}

ssm_status ssm_scan_chunk(ssm_handle h, int32_t slot, uint64_t chunk_seq, int64_t L,
                          const void *x, const void *dt, const void *B, const void *C,
                          const uint8_t *h_reset, void *y, int32_t n_ckpt,
                          const int64_t *h_ckpt_at, float *d_ckpt_out, void *d_workspace,
                          size_t ws_bytes, void *stream) {
  GET_HANDLE(H, h);
  return scan_chunk_impl(H, slot, chunk_seq, L, x, dt, B, C, h_reset, y, n_ckpt, h_ckpt_at,
                         d_ckpt_out, d_workspace, ws_bytes, nullptr, stream);
}

ssm_status ssm_scan_chunk_static(ssm_handle h, int32_t slot, uint64_t chunk_seq, int64_t L,
                                 const void *x, const void *dt, const void *B, const void *C,
                                 const uint8_t *h_reset, void *y, int32_t n_ckpt,
                                 const int64_t *h_ckpt_at, float *d_ckpt_out, void *stream) {
  GET_HANDLE(H, h);
  char *base = nullptr;  // this device's copy of the static scratch
  HIP_TRY(static_scratch((void **)&base));
  return scan_chunk_impl(H, slot, chunk_seq, L, x, dt, B, C, h_reset, y, n_ckpt, h_ckpt_at,
                         d_ckpt_out, base, SSM_STATIC_WORKSPACE_BYTES,
                         reinterpret_cast<unsigned int *>(base + kStaticFlagOff), stream);
}

ssm_status ssm_scan_packed(ssm_handle h, int32_t nseq, const int32_t *h_cu_seqlens,
                           const int32_t *h_seq_slots, const uint8_t *h_continue,
                           const uint64_t *h_chunk_seq, const void *x, const void *dt,
                           const void *B, const void *C, void *y, float *d_final,
                           ssm_receipt *h_receipts, void *stream) {
  GET_HANDLE(H, h);
  if (ssm_status st0 = need_rec(H, SSM_MAMBA2, "scan packed"); st0 != SSM_OK) return st0;
  if (nseq < 0) return fail(SSM_E_INVALID_ARG, "scan packed: negative sequence count");
  if (nseq == 0) return SSM_OK;
  if (!h_cu_seqlens) return fail(SSM_E_INVALID_ARG, "scan packed: cu_seqlens is NULL");
  if (h_cu_seqlens[0] != 0) return fail(SSM_E_INVALID_ARG, "scan packed: cu_seqlens[0] must be 0");
  for (int i = 0; i < nseq; ++i)
    if (h_cu_seqlens[i + 1] < h_cu_seqlens[i])
      return fail(SSM_E_INVALID_ARG, "scan packed: cu_seqlens decreases at %d", i + 1);
  ssm_status st = check_slots(H, nseq, h_seq_slots, "scan packed");
  if (st != SSM_OK) return st;
  for (int i = 0; i < nseq; ++i) {
    st = slot_is_plain(H, h_seq_slots[i], "scan packed");
    if (st != SSM_OK) return st;
  }
  bool any_cont = false;
  for (int i = 0; i < nseq; ++i) any_cont |= h_continue && h_continue[i];
  if (any_cont && !h_chunk_seq)
    return fail(SSM_E_INVALID_ARG, "scan packed: continuing sequences need h_chunk_seq");
  for (int i = 0; i < nseq; ++i) {
    if (!(h_continue && h_continue[i])) continue;
    const Slot &sl = H->slots[h_seq_slots[i]];
    if (h_chunk_seq[i] != sl.chunk_seq) {
      H->cnt.chunks_rejected++;
      return fail(SSM_E_SEQUENCE, "scan packed: slot %d expects chunk %llu, got %llu (%s)",
                  h_seq_slots[i], (unsigned long long)sl.chunk_seq,
                  (unsigned long long)h_chunk_seq[i],
                  h_chunk_seq[i] < sl.chunk_seq ? "duplicate" : "reordered or gap");
    }
  }
  const int64_t L = h_cu_seqlens[nseq];
  if (L > 0) {
    if (!x || !dt || !B || !C || !y)
      return fail(SSM_E_INVALID_ARG, "scan packed: NULL input or output");
    st = check_io_align(H->io, x, dt, B, C, y, "scan packed");
    if (st != SSM_OK) return st;
    if (ssd_supported(H->io, H->d) && (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16)))
      return fail(SSM_E_INVALID_ARG, "scan packed: bf16 x, B and C must be 16-byte aligned");
  }
  if (d_final && !aligned(d_final, 16))
    return fail(SSM_E_INVALID_ARG, "scan packed: d_final must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  if (L > 0) {
    st = check_finite(H, s, {{x, (size_t)L * H->d.H * H->d.P}, {dt, (size_t)L * H->d.H},
                             {B, (size_t)L * H->d.G * H->d.N}, {C, (size_t)L * H->d.G * H->d.N}});
    if (st != SSM_OK) return st;
  }
  // every sequence is one segment writing its own slot; slots are distinct, so
  // no segment reads a state another one writes
  const size_t nf = H->state_bytes() / 4;
  std::vector<ScanSeg> segs;
  // with d_final, sequence i's last token is checkpoint i (-1: an empty
  // sequence, which no launch's token range holds)
  std::vector<int64_t> ck_at(d_final ? nseq : 0, -1);
  for (int i = 0; i < nseq; ++i) {
    const int32_t t0 = h_cu_seqlens[i], t1 = h_cu_seqlens[i + 1];
    const int cont = h_continue && h_continue[i] ? 1 : 0;
    float *slot_st = H->slot_state(h_seq_slots[i]);
    if (t1 == t0) {  // an empty sequence: a fresh stream is zero, a continued one unchanged
      if (!cont) HIP_TRY(launch_zero(slot_st, nf, s));
      if (d_final) {
        if (cont)
          HIP_TRY(launch_copy_f32(d_final + (size_t)i * nf, slot_st, nf, s));
        else
          HIP_TRY(launch_zero(d_final + (size_t)i * nf, nf, s));
      }
      continue;
    }
    segs.push_back(ScanSeg{t0, t1, cont, 1, h_seq_slots[i]});
    if (d_final) ck_at[i] = t1 - 1;
  }
  if (!segs.empty()) {
    st = launch_seg_forms(H, H->state, nullptr, segs, x, dt, B, C, y, (int)ck_at.size(),
                          ck_at.data(), d_final, s);
    if (st != SSM_OK) return st;
  }
  for (int i = 0; i < nseq; ++i) {
    Slot &sl = H->slots[h_seq_slots[i]];
    const int64_t len = h_cu_seqlens[i + 1] - h_cu_seqlens[i];
    if (h_continue && h_continue[i]) {
      sl.pos += len;
      sl.chunk_seq++;
      if (len) H->cnt.state_bytes_read += H->state_bytes();
    } else {
      fresh_stream(sl);
      sl.pos = len;
      sl.chunk_seq = 1;
      H->cnt.resets++;
    }
    H->cnt.chunks_admitted++;
    H->cnt.state_bytes_written += H->state_bytes() * (d_final ? 2 : 1);
  }
  H->cnt.tokens_scanned += (uint64_t)L;
  if (h_receipts) {
    std::vector<const float *> src(nseq);
    std::vector<uint64_t> sums(nseq);
    for (int i = 0; i < nseq; ++i) src[i] = H->slot_state(h_seq_slots[i]);
    st = device_checksums(H, src.data(), nseq, s, sums.data());
    if (st != SSM_OK) return st;
    for (int i = 0; i < nseq; ++i)
      h_receipts[i] = slot_receipt(H, H->slots[h_seq_slots[i]], sums[i]);
  }
  return SSM_OK;
}

// ----------------------------------------------------------------- decode
ssm_status ssm_decode_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                           const void *x, const void *dt, const void *B, const void *C,
                           const uint8_t *h_reset, void *y, void *stream) {
  GET_HANDLE(H, h);
  if (ssm_status st0 = need_rec(H, SSM_MAMBA2, "decode"); st0 != SSM_OK) return st0;
  ssm_status st = check_slots(H, batch, h_slot_ids, "decode");
  if (st != SSM_OK) return st;
  for (int i = 0; i < batch; ++i) {
    st = slot_is_plain(H, h_slot_ids[i], "decode");
    if (st != SSM_OK) return st;
  }
  if (batch == 0) return SSM_OK;
  if (!x || !dt || !B || !C || !y) return fail(SSM_E_INVALID_ARG, "decode: NULL input or output");
  st = check_io_align(H->io, x, dt, B, C, y, "decode");
  if (st != SSM_OK) return st;
  hipStream_t s = as_stream(stream);
  const Dims &d = H->d;
  st = check_finite(H, s, {{x, (size_t)batch * d.H * d.P}, {dt, (size_t)batch * d.H},
                           {B, (size_t)batch * d.G * d.N}, {C, (size_t)batch * d.G * d.N}});
  if (st != SSM_OK) return st;
  const size_t es = io_size(H->io);
  for (int i0 = 0; i0 < batch; i0 += kBatchPerLaunch) {
    const int n = std::min(kBatchPerLaunch, batch - i0);
    DecodeMeta m;
    for (int k = 0; k < n; ++k)
      m.slot_rst[k] = (uint32_t)h_slot_ids[i0 + k] |
                      (h_reset && h_reset[i0 + k] ? kDecodeReset : 0u);
    DecodeArgs a{};
    a.x = (const char *)x + (size_t)i0 * d.H * d.P * es;
    a.dt = (const char *)dt + (size_t)i0 * d.H * es;
    a.B = (const char *)B + (size_t)i0 * d.G * d.N * es;
    a.C = (const char *)C + (size_t)i0 * d.G * d.N * es;
    a.y = (char *)y + (size_t)i0 * d.H * d.P * es;
    a.state = H->state;
    a.A = H->A;
    a.D = H->D;
    a.d = d;
    a.n = n;
    HIP_TRY(launch_decode(H->io, a, m, s));
  }
  for (int i = 0; i < batch; ++i) {
    Slot &sl = H->slots[h_slot_ids[i]];
    const bool r = h_reset && h_reset[i];
    if (r) {
      sl.pos = 0;
      H->cnt.resets++;
    } else {
      H->cnt.state_bytes_read += H->state_bytes();
    }
    sl.pos += 1;
    H->cnt.state_bytes_written += H->state_bytes();
  }
  H->cnt.decode_tokens += batch;
  return SSM_OK;
}

// ----------------------------------------------------------------- replay
size_t ssm_replay_log_bytes(const ssm_layer_desc *desc, int32_t n_slots, int32_t W) {
  if (check_desc(desc) != SSM_OK || n_slots < 1 || W < 1 || W > kMaxW) return 0;
  const Dims d{desc->H, desc->P, desc->N, desc->G, (desc->P + kRows - 1) / kRows};
  return log_layout(desc->io_dtype, d, n_slots, W, desc->recurrence == SSM_GATED_DELTA).total;
}

ssm_status ssm_replay_attach(ssm_handle h, int32_t W, void *d_log, size_t log_bytes) {
  GET_HANDLE(H, h);
  if (W < 1 || W > kMaxW) return fail(SSM_E_INVALID_ARG, "replay: W must be in [1, %d]", kMaxW);
  if (!d_log || !aligned(d_log, 256))
    return fail(SSM_E_INVALID_ARG, "replay: log must be non-NULL and 256-byte aligned");
  const LogLayout lay = log_layout(H->io, H->d, H->S, W, H->rec == SSM_GATED_DELTA);
  if (log_bytes < lay.total)
    return fail(SSM_E_INVALID_ARG, "replay: log needs %zu bytes, got %zu", lay.total, log_bytes);
  for (int s = 0; s < H->S; ++s)
    if (H->slots[s].log_len > 0 || H->slots[s].pend != kNone)
      return fail(SSM_E_LOG, "replay: slot %d still uses the current log", s);
  H->W = W;
  H->log = d_log;
  H->lay = lay;
  for (auto &sl : H->slots) {
    sl.log_len = 0;
    sl.log_half = 0;
  }
  return SSM_OK;
}

static ssm_status replay_step_impl(Handle *H, int32_t batch, const int32_t *h_slot_ids,
                                   int32_t n_in, const void *x, const void *dt, const void *beta,
                                   const void *B, const void *C, void *y, void *stream) {
  if (!H->log) return fail(SSM_E_LOG, "replay: no log attached");
  if (n_in < 1 || n_in > H->W || n_in > kMaxInFlight)
    return fail(SSM_E_INVALID_ARG, "replay: n_in must be in [1, min(W, %d)]", kMaxInFlight);
  ssm_status st = check_slots(H, batch, h_slot_ids, "replay");
  if (st != SSM_OK) return st;
  for (int i = 0; i < batch; ++i) {
    const Slot &sl = H->slots[h_slot_ids[i]];
    if (sl.pend != kNone)
      return fail(SSM_E_LOG, "replay: slot %d has a verify step awaiting commit", h_slot_ids[i]);
    if (sl.live >= 0)
      return fail(SSM_E_LOG, "replay: slot %d holds a live copy (materialize it first)",
                  h_slot_ids[i]);
  }
  if (batch == 0) return SSM_OK;
  if (!x || !dt || !B || !C || !y) return fail(SSM_E_INVALID_ARG, "replay: NULL input or output");
  st = check_io_align(H->io, x, dt, B, C, y, "replay");
  if (st != SSM_OK) return st;
  hipStream_t s = as_stream(stream);
  const Dims &d = H->d;
  const size_t nt = (size_t)batch * n_in;
  const bool gdn = H->rec == SSM_GATED_DELTA;
  if (gdn && (!beta || !aligned(beta, io_size(H->io))))
    return fail(SSM_E_INVALID_ARG, "replay: beta is NULL or misaligned");
  st = check_finite(H, s, {{x, nt * d.H * d.P}, {dt, nt * d.H}, {B, nt * d.G * d.N},
                           {C, nt * d.G * d.N}, {gdn ? beta : nullptr, gdn ? nt * d.H : 0}});
  if (st != SSM_OK) return st;
  const size_t es = io_size(H->io);
  for (int i0 = 0; i0 < batch; i0 += kBatchPerLaunch) {
    const int n = std::min(kBatchPerLaunch, batch - i0);
    ReplayMeta m;
    for (int i = 0; i < n; ++i) {
      const Slot &sl = H->slots[h_slot_ids[i0 + i]];
      m.slot[i] = h_slot_ids[i0 + i];
      if (sl.log_len + n_in > H->W)  // the log is full: fold, then start the other half
        m.info[i] = replay_info(sl.log_len, 0, sl.log_half, 1 - sl.log_half);
      else
        m.info[i] = replay_info(0, sl.log_len, sl.log_half, sl.log_half);
    }
    const size_t off = (size_t)i0 * n_in;
    ReplayArgs a{};
    a.x = (const char *)x + off * d.H * d.P * es;
    a.dt = (const char *)dt + off * d.H * es;
    a.beta = gdn ? (const char *)beta + off * d.H * es : nullptr;
    a.B = (const char *)B + off * d.G * d.N * es;
    a.C = (const char *)C + off * d.G * d.N * es;
    a.y = (char *)y + off * d.H * d.P * es;
    a.state = H->state;
    a.log = H->log;
    a.bc = reinterpret_cast<float *>((char *)H->log + H->lay.bc_off);
    a.A = H->A;
    a.D = H->D;
    a.d = d;
    a.n = n;
    a.n_in = n_in;
    a.W = H->W;
    a.nin_magic = fastdiv_magic(a.n_in);
    if (gdn)
      HIP_TRY(launch_gdn_replay(H->io, a, m, H->lay, s));
    else
      HIP_TRY(launch_replay(H->io, a, m, H->lay, s));
  }
  for (int i = 0; i < batch; ++i) {
    Slot &sl = H->slots[h_slot_ids[i]];
    if (sl.log_len + n_in > H->W) {
      sl.log_half = 1 - sl.log_half;
      sl.log_len = 0;
      H->cnt.replay_flushes++;
      H->cnt.state_bytes_written += H->state_bytes();
    }
    sl.pend = kReplayPend;
    sl.pend_n = n_in;
    sl.pend_base = sl.log_len;
    H->cnt.state_bytes_read += H->state_bytes();
  }
  H->cnt.replay_steps++;
  return SSM_OK;
}

ssm_status ssm_replay_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, int32_t n_in,
                           const void *x, const void *dt, const void *B, const void *C, void *y,
                           void *stream) {
  GET_HANDLE(H, h);
  if (ssm_status st = need_rec(H, SSM_MAMBA2, "replay"); st != SSM_OK) return st;
  return replay_step_impl(H, batch, h_slot_ids, n_in, x, dt, nullptr, B, C, y, stream);
}

ssm_status ssm_gdn_replay_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                               int32_t n_in, const void *v, const void *dt, const void *beta,
                               const void *k, const void *q, void *y, void *stream) {
  GET_HANDLE(H, h);
  if (ssm_status st = need_rec(H, SSM_GATED_DELTA, "gdn replay"); st != SSM_OK) return st;
  return replay_step_impl(H, batch, h_slot_ids, n_in, v, dt, beta, k, q, y, stream);
}

ssm_status ssm_replay_commit(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                             const int32_t *h_accepted) {
  GET_HANDLE(H, h);
  ssm_status st = check_slots(H, batch, h_slot_ids, "replay commit");
  if (st != SSM_OK) return st;
  if (batch > 0 && !h_accepted) return fail(SSM_E_INVALID_ARG, "replay commit: accepted is NULL");
  for (int i = 0; i < batch; ++i) {
    const Slot &sl = H->slots[h_slot_ids[i]];
    if (sl.pend != kReplayPend)
      return fail(SSM_E_LOG, "replay commit: slot %d has no replay step to commit", h_slot_ids[i]);
    if (h_accepted[i] < 1 || h_accepted[i] > sl.pend_n)
      return fail(SSM_E_LOG, "replay commit: slot %d accepted %d outside [1, %d]", h_slot_ids[i],
                  h_accepted[i], sl.pend_n);
  }
  for (int i = 0; i < batch; ++i) {
    Slot &sl = H->slots[h_slot_ids[i]];
    sl.log_len = sl.pend_base + h_accepted[i];
    sl.pos += h_accepted[i];
    sl.pend = kNone;
    sl.pend_n = 0;
    H->cnt.replay_tokens_committed += h_accepted[i];
  }
  return SSM_OK;
}

// ---------------------------------------------------------- copy baseline
size_t ssm_copy_buffer_bytes(const ssm_layer_desc *desc, int32_t n_slots, int32_t n_in_max) {
  if (check_desc(desc) != SSM_OK || n_slots < 1 || n_in_max < 1) return 0;
  return (size_t)n_slots * n_in_max * desc->H * desc->P * desc->N * sizeof(float);
}

ssm_status ssm_copy_attach(ssm_handle h, int32_t n_in_max, float *d_copies, size_t bytes) {
  GET_HANDLE(H, h);
  if (n_in_max < 1 || n_in_max > 127)
    return fail(SSM_E_INVALID_ARG, "copy: n_in_max must be in [1, 127]");
  if (!d_copies || !aligned(d_copies, 16))
    return fail(SSM_E_INVALID_ARG, "copy: buffer must be non-NULL and 16-byte aligned");
  const size_t need = (size_t)H->S * n_in_max * H->state_bytes();
  if (bytes < need) return fail(SSM_E_INVALID_ARG, "copy: need %zu bytes, got %zu", need, bytes);
  for (int s = 0; s < H->S; ++s)
    if (H->slots[s].live >= 0 || H->slots[s].pend == kCopyPend)
      return fail(SSM_E_LOG, "copy: slot %d still uses the current buffer", s);
  H->n_in_max = n_in_max;
  H->copies = d_copies;
  return SSM_OK;
}

static ssm_status copy_step_impl(Handle *H, int32_t batch, const int32_t *h_slot_ids,
                                 int32_t n_in, const void *x, const void *dt, const void *beta,
                                 const void *B, const void *C, void *y, void *stream) {
  if (!H->copies) return fail(SSM_E_LOG, "copy: no buffer attached");
  if (n_in < 1 || n_in > H->n_in_max)
    return fail(SSM_E_INVALID_ARG, "copy: n_in must be in [1, %d]", H->n_in_max);
  ssm_status st = check_slots(H, batch, h_slot_ids, "copy");
  if (st != SSM_OK) return st;
  for (int i = 0; i < batch; ++i) {
    const Slot &sl = H->slots[h_slot_ids[i]];
    if (sl.pend != kNone)
      return fail(SSM_E_LOG, "copy: slot %d has a verify step awaiting commit", h_slot_ids[i]);
    if (sl.log_len > 0)
      return fail(SSM_E_LOG, "copy: slot %d holds a replay log (materialize it first)",
                  h_slot_ids[i]);
  }
  if (batch == 0) return SSM_OK;
  if (!x || !dt || !B || !C || !y) return fail(SSM_E_INVALID_ARG, "copy: NULL input or output");
  st = check_io_align(H->io, x, dt, B, C, y, "copy");
  if (st != SSM_OK) return st;
  hipStream_t s = as_stream(stream);
  const Dims &d = H->d;
  const size_t nt = (size_t)batch * n_in;
  const bool gdn = H->rec == SSM_GATED_DELTA;
  if (gdn && (!beta || !aligned(beta, io_size(H->io))))
    return fail(SSM_E_INVALID_ARG, "copy: beta is NULL or misaligned");
  st = check_finite(H, s, {{x, nt * d.H * d.P}, {dt, nt * d.H}, {B, nt * d.G * d.N},
                           {C, nt * d.G * d.N}, {gdn ? beta : nullptr, gdn ? nt * d.H : 0}});
  if (st != SSM_OK) return st;
  const size_t es = io_size(H->io);
  for (int i0 = 0; i0 < batch; i0 += kBatchPerLaunch) {
    const int n = std::min(kBatchPerLaunch, batch - i0);
    CopyMeta m;
    for (int i = 0; i < n; ++i) {
      m.slot[i] = h_slot_ids[i0 + i];
      m.src[i] = (int8_t)H->slots[h_slot_ids[i0 + i]].live;
    }
    const size_t off = (size_t)i0 * n_in;
    CopyArgs a{};
    a.x = (const char *)x + off * d.H * d.P * es;
    a.dt = (const char *)dt + off * d.H * es;
    a.beta = gdn ? (const char *)beta + off * d.H * es : nullptr;
    a.B = (const char *)B + off * d.G * d.N * es;
    a.C = (const char *)C + off * d.G * d.N * es;
    a.y = (char *)y + off * d.H * d.P * es;
    a.state = H->state;
    a.copies = H->copies;
    a.A = H->A;
    a.D = H->D;
    a.d = d;
    a.n = n;
    a.n_in = n_in;
    a.n_in_max = H->n_in_max;
    if (gdn)
      HIP_TRY(launch_gdn_copy(H->io, a, m, s));
    else
      HIP_TRY(launch_copy(H->io, a, m, s));
  }
  for (int i = 0; i < batch; ++i) {
    Slot &sl = H->slots[h_slot_ids[i]];
    sl.pend = kCopyPend;
    sl.pend_n = n_in;
    H->cnt.state_bytes_read += H->state_bytes();
    H->cnt.state_bytes_written += (size_t)n_in * H->state_bytes();
  }
  H->cnt.copy_steps++;
  return SSM_OK;
}

ssm_status ssm_copy_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, int32_t n_in,
                         const void *x, const void *dt, const void *B, const void *C, void *y,
                         void *stream) {
  GET_HANDLE(H, h);
  if (ssm_status st = need_rec(H, SSM_MAMBA2, "copy"); st != SSM_OK) return st;
  return copy_step_impl(H, batch, h_slot_ids, n_in, x, dt, nullptr, B, C, y, stream);
}

ssm_status ssm_gdn_copy_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, int32_t n_in,
                             const void *v, const void *dt, const void *beta, const void *k,
                             const void *q, void *y, void *stream) {
  GET_HANDLE(H, h);
  if (ssm_status st = need_rec(H, SSM_GATED_DELTA, "gdn copy"); st != SSM_OK) return st;
  return copy_step_impl(H, batch, h_slot_ids, n_in, v, dt, beta, k, q, y, stream);
}

ssm_status ssm_copy_commit(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                           const int32_t *h_accepted) {
  GET_HANDLE(H, h);
  ssm_status st = check_slots(H, batch, h_slot_ids, "copy commit");
  if (st != SSM_OK) return st;
  if (batch > 0 && !h_accepted) return fail(SSM_E_INVALID_ARG, "copy commit: accepted is NULL");
  for (int i = 0; i < batch; ++i) {
    const Slot &sl = H->slots[h_slot_ids[i]];
    if (sl.pend != kCopyPend)
      return fail(SSM_E_LOG, "copy commit: slot %d has no copy step to commit", h_slot_ids[i]);
    if (h_accepted[i] < 1 || h_accepted[i] > sl.pend_n)
      return fail(SSM_E_LOG, "copy commit: slot %d accepted %d outside [1, %d]", h_slot_ids[i],
                  h_accepted[i], sl.pend_n);
  }
  for (int i = 0; i < batch; ++i) {
    Slot &sl = H->slots[h_slot_ids[i]];
    sl.live = h_accepted[i] - 1;
    sl.pos += h_accepted[i];
    sl.pend = kNone;
    sl.pend_n = 0;
  }
  return SSM_OK;
}

// -------------------------------------------------------- state operations
ssm_status ssm_state_materialize(ssm_handle h, int32_t n, const int32_t *h_slots, void *stream) {
  GET_HANDLE(H, h);
  ssm_status st = check_slots(H, n, h_slots, "materialize");
  if (st != SSM_OK) return st;
  return materialize(H, n, h_slots, as_stream(stream));
}

ssm_status ssm_state_checkpoint(ssm_handle h, int32_t slot, float *d_dst, ssm_receipt *out,
                                void *stream) {
  GET_HANDLE(H, h);
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "checkpoint: bad slot %d", slot);
  if (!d_dst || !out || !aligned(d_dst, 16))
    return fail(SSM_E_INVALID_ARG, "checkpoint: NULL or misaligned destination, or NULL receipt");
  if (H->slots[slot].pend != kNone)
    return fail(SSM_E_LOG, "checkpoint: slot %d has a verify step awaiting commit", slot);
  hipStream_t s = as_stream(stream);
  const int32_t one = slot;
  ssm_status st = materialize(H, 1, &one, s);
  if (st != SSM_OK) return st;
  HIP_TRY(launch_copy_f32(d_dst, H->slot_state(slot), H->state_bytes() / 4, s));
  uint64_t sum = 0;
  st = device_checksum(H, d_dst, s, &sum);
  if (st != SSM_OK) return st;
  *out = slot_receipt(H, H->slots[slot], sum);
  H->cnt.checkpoints++;
  H->cnt.state_bytes_read += H->state_bytes();
  return SSM_OK;
}

namespace {

// A receipt field that does not match the handle, or nullptr.
static const char *receipt_mismatch(const Handle *H, const ssm_receipt *r) {
  if (r->schema_version != H->desc.schema_version) return "schema version";
  if (r->recurrence != (uint32_t)H->rec) return "recurrence";
  if (r->state_dtype != SSM_F32) return "state dtype";
  if (r->H != H->d.H || r->P != H->d.P || r->N != H->d.N || r->G != H->d.G) return "dimensions";
  if (r->model_rev != H->desc.model_rev) return "model revision";
  if (r->code_rev != kCodeRev) return "code revision";
  if (r->position < 0) return "position";
  return nullptr;
}

// The slot continues the stream the receipt names: its position, chunk
// sequence and id; no replay log and no live copy.
static void adopt_receipt(Handle *H, int slot, const ssm_receipt *r) {
  Slot &sl = H->slots[slot];
  sl.pos = r->position;
  sl.chunk_seq = r->chunk_seq;
  sl.stream_id = r->stream_id;
  sl.log_len = 0;
  sl.live = -1;
  sl.pend = kNone;
  H->cnt.restores++;
  H->cnt.state_bytes_written += H->state_bytes();
}

}  // namespace

ssm_status ssm_state_restore(ssm_handle h, int32_t slot, const float *d_src,
                             const ssm_receipt *r, void *stream) {
  GET_HANDLE(H, h);
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "restore: bad slot %d", slot);
  if (!d_src || !r || !aligned(d_src, 16))
    return fail(SSM_E_INVALID_ARG, "restore: NULL or misaligned source, or NULL receipt");
  if (H->slots[slot].pend != kNone)
    return fail(SSM_E_LOG, "restore: slot %d has a verify step awaiting commit", slot);
  if (const char *bad = receipt_mismatch(H, r)) {
    H->cnt.restores_rejected++;
    return fail(SSM_E_SCHEMA, "restore: receipt %s does not match the handle", bad);
  }
  hipStream_t s = as_stream(stream);
  uint64_t sum = 0;
  ssm_status st = device_checksum(H, d_src, s, &sum);
  if (st != SSM_OK) return st;
  if (sum != r->checksum) {
    H->cnt.restores_rejected++;
    return fail(SSM_E_SCHEMA, "restore: checksum mismatch (state does not match its receipt)");
  }
  HIP_TRY(launch_copy_f32(H->slot_state(slot), d_src, H->state_bytes() / 4, s));
  adopt_receipt(H, slot, r);
  return SSM_OK;
}

// ------------------------------------------------------------- state blobs
// The byte format of the recurrent-state companion store ("SSM.PREFIX.* --
// recurrent-state companion", its reference serialization format): a u32
// version (1) and a u32 array count, then per array a u32 rank, the u32
// extents, a u32 dtype code (0 fp32, 1 fp16, 2 bf16 widened to fp32) and the
// raw element bytes.  Every u32 and element is little-endian.
static_assert(__BYTE_ORDER__ == __ORDER_LITTLE_ENDIAN__, "blob payloads are copied as host words");

namespace {

constexpr uint32_t kBlobVersion = 1;
constexpr uint32_t kBlobMaxRank = 16;
constexpr uint32_t kBlobF32 = 0, kBlobF16 = 1, kBlobBF16 = 2;

static size_t blob_size(const Dims &d) {
  return 8 + 4 + 3 * 4 + 4 + (size_t)d.H * d.P * d.N * sizeof(float);
}

static void put_u32(uint8_t *p, uint32_t v) {
  for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

static uint32_t get_u32(const uint8_t *p) {
  return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

// The receipt's checksum, taken on the host.
static uint64_t host_checksum(const float *v, size_t n) {
  uint64_t sum = 0;
  for (size_t i = 0; i < n; ++i) {
    uint32_t w;
    memcpy(&w, v + i, 4);
    sum += (uint64_t)w * (2ull * i + 1ull);
  }
  return sum;
}

// IEEE 754 binary16 to binary32.  Every binary16 value is exact in binary32;
// subnormals (m * 2^-24) go through ldexpf, which is exact for them.
static float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  uint32_t bits;
  if (e == 0x1fu) {
    bits = sign | 0x7f800000u | (m << 13);  // infinity, NaN keeps its payload
  } else if (e != 0) {
    bits = sign | ((e + 127u - 15u) << 23) | (m << 13);
  } else {
    const float mag = ldexpf((float)m, -24);
    memcpy(&bits, &mag, 4);
    bits |= sign;
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

struct BlobArray {
  std::vector<uint32_t> shape;
  uint32_t dtype = 0;
  const uint8_t *data = nullptr;
  size_t count = 0;
};

// Walk a blob with every length checked against `len`; nullptr on success,
// else what is wrong.  Trailing bytes after the last array are an error.
static const char *parse_blob(const uint8_t *p, size_t len, std::vector<BlobArray> *out) {
  size_t at = 0;
  auto have = [&](size_t n) { return n <= len - at; };
  if (!have(8)) return "shorter than its header";
  if (get_u32(p) != kBlobVersion) return "version is not 1";
  const uint32_t n_arrays = get_u32(p + 4);
  at = 8;
  if (n_arrays == 0) return "holds no arrays";
  if (n_arrays > (len - at) / 8) return "array count exceeds its length";
  out->clear();
  for (uint32_t a = 0; a < n_arrays; ++a) {
    BlobArray arr;
    if (!have(4)) return "truncated in an array header";
    const uint32_t rank = get_u32(p + at);
    at += 4;
    if (rank > kBlobMaxRank) return "array rank above 16";
    if (!have((size_t)rank * 4 + 4)) return "truncated in an array header";
    size_t count = 1;
    for (uint32_t k = 0; k < rank; ++k) {
      const uint32_t ext = get_u32(p + at);
      at += 4;
      arr.shape.push_back(ext);
      if (ext != 0 && count > SIZE_MAX / 4 / ext) return "array size overflows";
      count *= ext;
    }
    arr.dtype = get_u32(p + at);
    at += 4;
    if (arr.dtype > kBlobBF16) return "unknown dtype code";
    const size_t bytes = count * (arr.dtype == kBlobF16 ? 2 : 4);
    if (!have(bytes)) return "truncated in array data";
    arr.data = p + at;
    arr.count = count;
    at += bytes;
    out->push_back(std::move(arr));
  }
  if (at != len) return "has trailing bytes after its last array";
  return nullptr;
}

// Decode array `a` into fp32 words if its extents are `want` after any
// leading extents of 1; nullptr on success, else what is wrong.
static const char *decode_array(const BlobArray &a, std::initializer_list<uint32_t> want,
                                const char *wrong_shape, std::vector<float> *out) {
  const size_t rank = a.shape.size(), nw = want.size();
  if (rank < nw) return wrong_shape;
  size_t k = 0;
  for (; k + nw < rank; ++k)
    if (a.shape[k] != 1) return wrong_shape;
  for (uint32_t e : want)
    if (a.shape[k++] != e) return wrong_shape;
  out->resize(a.count);
  if (a.dtype == kBlobF16) {
    for (size_t i = 0; i < a.count; ++i)
      (*out)[i] = half_to_float((uint16_t)(a.data[2 * i] | a.data[2 * i + 1] << 8));
  } else {
    memcpy(out->data(), a.data, a.count * 4);
    if (a.dtype == kBlobBF16)
      for (size_t i = 0; i < a.count; ++i) {
        uint32_t w;
        memcpy(&w, &(*out)[i], 4);
        if (w & 0xffffu) return "bf16 array holds a value bf16 cannot represent";
      }
  }
  return nullptr;
}

// Blob of a handle's slot: [conv_state [C, K-1], ssm_state [H, P, N]] with a
// conv of K > 1 attached (a Mamba layer's pair), else [ssm_state].
static size_t conv_blob_part(const Handle *H) {
  return H->conv_floats() ? 4 + 2 * 4 + 4 + H->conv_floats() * sizeof(float) : 0;
}
static size_t handle_blob_size(const Handle *H) { return blob_size(H->d) + conv_blob_part(H); }

}  // namespace

size_t ssm_state_blob_bytes(ssm_handle h) {
  Handle *H = lookup(h);
  return H ? handle_blob_size(H) : 0;
}

size_t ssm_blob_bytes(const ssm_layer_desc *desc) {
  if (check_desc(desc) != SSM_OK) return 0;
  return blob_size(dims_of(desc));
}

ssm_status ssm_state_serialize(ssm_handle h, int32_t slot, void *h_blob, size_t cap,
                               size_t *written, ssm_receipt *out, void *stream) {
  GET_HANDLE(H, h);
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "serialize: bad slot %d", slot);
  if (!h_blob || !written || !out)
    return fail(SSM_E_INVALID_ARG, "serialize: NULL blob, length or receipt pointer");
  const size_t need = handle_blob_size(H);
  if (cap < need)
    return fail(SSM_E_INVALID_ARG, "serialize: blob capacity %zu below the %zu bytes needed", cap,
                need);
  if (H->slots[slot].pend != kNone)
    return fail(SSM_E_LOG, "serialize: slot %d has a verify step awaiting commit", slot);
  hipStream_t s = as_stream(stream);
  const int32_t one = slot;
  ssm_status st = materialize(H, 1, &one, s);
  if (st != SSM_OK) return st;
  // Bounce through an aligned host buffer: the payload sits 28 bytes into the blob.
  const size_t nf = H->state_bytes() / 4, nc = H->conv_floats();
  std::vector<float> host(nf), conv(nc);
  HIP_TRY(hipMemcpyAsync(host.data(), H->slot_state(slot), H->state_bytes(),
                         hipMemcpyDeviceToHost, s));
  if (nc)
    HIP_TRY(hipMemcpyAsync(conv.data(), H->conv_state + (size_t)slot * nc, nc * sizeof(float),
                           hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  uint8_t *b = static_cast<uint8_t *>(h_blob);
  put_u32(b, kBlobVersion);
  put_u32(b + 4, nc ? 2u : 1u);
  uint8_t *p = b + 8;
  if (nc) {
    const uint32_t ch[4] = {2u, (uint32_t)H->conv_C, (uint32_t)(H->conv_K - 1), kBlobF32};
    for (int i = 0; i < 4; ++i) put_u32(p + 4 * i, ch[i]);
    memcpy(p + 16, conv.data(), nc * sizeof(float));
    p += 16 + nc * sizeof(float);
  }
  const uint32_t head[5] = {3u, (uint32_t)H->d.H, (uint32_t)H->d.P, (uint32_t)H->d.N, kBlobF32};
  for (int i = 0; i < 5; ++i) put_u32(p + 4 * i, head[i]);
  memcpy(p + 20, host.data(), H->state_bytes());
  *written = need;
  *out = slot_receipt(H, H->slots[slot], host_checksum(host.data(), nf));
  H->cnt.checkpoints++;
  H->cnt.state_bytes_read += H->state_bytes();
  return SSM_OK;
}

ssm_status ssm_state_deserialize(ssm_handle h, int32_t slot, const void *h_blob, size_t len,
                                 const ssm_receipt *r, void *stream) {
  GET_HANDLE(H, h);
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "deserialize: bad slot %d", slot);
  if (!h_blob || !r) return fail(SSM_E_INVALID_ARG, "deserialize: NULL blob or receipt");
  if (H->slots[slot].pend != kNone)
    return fail(SSM_E_LOG, "deserialize: slot %d has a verify step awaiting commit", slot);
  auto reject = [&](const char *what) {
    H->cnt.restores_rejected++;
    return fail(SSM_E_SCHEMA, "deserialize: blob %s", what);
  };
  if (const char *bad = receipt_mismatch(H, r)) {
    H->cnt.restores_rejected++;
    return fail(SSM_E_SCHEMA, "deserialize: receipt %s does not match the handle", bad);
  }
  std::vector<BlobArray> arrays;
  if (const char *bad = parse_blob(static_cast<const uint8_t *>(h_blob), len, &arrays))
    return reject(bad);
  // The recurrent state is the last array, [H, P, N] after any leading
  // extents of 1.  With a conv attached the one before it is the conv state,
  // [C, K-1] (a Mamba blob is [conv_state, ssm_state]).
  std::vector<float> host, conv;
  if (const char *bad = decode_array(arrays.back(),
                                     {(uint32_t)H->d.H, (uint32_t)H->d.P, (uint32_t)H->d.N},
                                     "state array is not [H, P, N] for this handle", &host))
    return reject(bad);
  const size_t nf = host.size(), nc = H->conv_floats();
  if (nc) {
    if (arrays.size() < 2) return reject("lacks the conv state this handle carries");
    if (const char *bad = decode_array(arrays[arrays.size() - 2],
                                       {(uint32_t)H->conv_C, (uint32_t)(H->conv_K - 1)},
                                       "conv state array is not [C, K-1] for this handle", &conv))
      return reject(bad);
  }
  if (host_checksum(host.data(), nf) != r->checksum) {
    H->cnt.restores_rejected++;
    return fail(SSM_E_SCHEMA, "deserialize: checksum mismatch (state does not match its receipt)");
  }
  hipStream_t s = as_stream(stream);
  HIP_TRY(hipMemcpyAsync(H->slot_state(slot), host.data(), H->state_bytes(),
                         hipMemcpyHostToDevice, s));
  if (nc)
    HIP_TRY(hipMemcpyAsync(H->conv_state + (size_t)slot * nc, conv.data(), nc * sizeof(float),
                           hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  adopt_receipt(H, slot, r);
  return SSM_OK;
}

// --------------------------------------------------- conv1d and gated output
size_t ssm_conv_state_bytes(int32_t n_slots, int32_t C, int32_t K) {
  if (n_slots < 1 || C < 1 || K < 1 || K > kMaxConvK) return 0;
  return (size_t)n_slots * C * (K - 1) * sizeof(float);
}

ssm_status ssm_conv_attach(ssm_handle h, int32_t C, int32_t K, int32_t act, float *d_conv_state,
                           const float *d_w, const float *d_bias) {
  GET_HANDLE(H, h);
  if (C < 1 || K < 1 || K > kMaxConvK)
    return fail(SSM_E_INVALID_ARG, "conv: need C >= 1 and 1 <= K <= %d (C=%d K=%d)", kMaxConvK,
                C, K);
  if (act != 0 && act != 1) return fail(SSM_E_INVALID_ARG, "conv: act must be 0 or 1");
  if (!d_w || (K > 1 && !d_conv_state))
    return fail(SSM_E_INVALID_ARG, "conv: weights and (for K > 1) the conv state are required");
  if (!aligned(d_w, 4) || !aligned(d_conv_state, 4) || !aligned(d_bias, 4))
    return fail(SSM_E_INVALID_ARG, "conv: misaligned weight, bias or state pointer");
  H->conv_C = C;
  H->conv_K = K;
  H->conv_act = act;
  H->conv_state = K > 1 ? d_conv_state : nullptr;
  H->conv_w = d_w;
  H->conv_b = d_bias;
  return SSM_OK;
}

namespace {

ConvArgs conv_args(const Handle *H) {
  ConvArgs a{};
  a.w = H->conv_w;
  a.bias = H->conv_b;
  a.C = H->conv_C;
  a.K = H->conv_K;
  a.act = H->conv_act;
  return a;
}

// Tokens per conv launch: bounded by the grid's y extent (runs of 8 tokens).
constexpr int64_t kConvTokensPerLaunch = 1 << 18;

}  // namespace

ssm_status ssm_conv_chunk(ssm_handle h, int32_t slot, int64_t L, const void *x,
                          const uint8_t *h_reset, void *y, void *stream) {
  GET_HANDLE(H, h);
  if (!H->conv_C) return fail(SSM_E_INVALID_STATE, "conv: no conv attached");
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "conv: bad slot %d", slot);
  if (L < 0 || L > INT32_MAX) return fail(SSM_E_INVALID_ARG, "conv: bad chunk length");
  if (L == 0) return SSM_OK;
  if (!x || !y) return fail(SSM_E_INVALID_ARG, "conv: NULL input or output");
  const size_t es = io_size(H->io);
  if (!aligned(x, es) || !aligned(y, es)) return fail(SSM_E_INVALID_ARG, "conv: misaligned x or y");
  const size_t bytes = (size_t)L * H->conv_C * es;
  if ((const char *)x < (const char *)y + bytes && (const char *)y < (const char *)x + bytes)
    return fail(SSM_E_INVALID_ARG, "conv: x and y overlap");
  hipStream_t s = as_stream(stream);
  ssm_status st = check_finite(H, s, {{x, (size_t)L * H->conv_C}});
  if (st != SSM_OK) return st;
  std::vector<int32_t> rst;
  if (h_reset)
    for (int64_t t = 0; t < L; ++t)
      if (h_reset[t]) rst.push_back((int32_t)t);
  ConvArgs a = conv_args(H);
  a.x = x;
  a.y = y;
  a.state = H->conv_state ? H->conv_state + (size_t)slot * H->conv_floats() : nullptr;
  const int none = -H->conv_K;  // no reset yet: the carried state is visible
  size_t ri = 0;
  int first = none;
  for (int64_t t0 = 0; t0 < L;) {
    // a piece holds at most kConvResetsPerLaunch resets and kConvTokensPerLaunch tokens
    int64_t t1 = std::min(L, t0 + kConvTokensPerLaunch);
    if (rst.size() - ri > (size_t)kConvResetsPerLaunch && rst[ri + kConvResetsPerLaunch] < t1)
      t1 = rst[ri + kConvResetsPerLaunch];
    ConvChunkMeta m{};
    m.first_before = first;
    while (ri < rst.size() && rst[ri] < t1) {
      m.rst[m.n_rst++] = rst[ri];
      first = rst[ri++];
    }
    a.t_begin = (int)t0;
    a.t_end = (int)t1;
    HIP_TRY(launch_conv_chunk(H->io, a, m, s));
    t0 = t1;
  }
  HIP_TRY(launch_conv_state(H->io, a, (int)L, first, s));
  return SSM_OK;
}

ssm_status ssm_conv_decode(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, const void *x,
                           const uint8_t *h_reset, void *y, void *stream) {
  GET_HANDLE(H, h);
  if (!H->conv_C) return fail(SSM_E_INVALID_STATE, "conv: no conv attached");
  ssm_status st = check_slots(H, batch, h_slot_ids, "conv decode");
  if (st != SSM_OK) return st;
  if (batch == 0) return SSM_OK;
  if (!x || !y) return fail(SSM_E_INVALID_ARG, "conv decode: NULL input or output");
  const size_t es = io_size(H->io);
  if (!aligned(x, es) || !aligned(y, es))
    return fail(SSM_E_INVALID_ARG, "conv decode: misaligned x or y");
  hipStream_t s = as_stream(stream);
  st = check_finite(H, s, {{x, (size_t)batch * H->conv_C}});
  if (st != SSM_OK) return st;
  for (int i0 = 0; i0 < batch; i0 += kBatchPerLaunch) {
    const int n = std::min(kBatchPerLaunch, batch - i0);
    DecodeMeta m;
    for (int k = 0; k < n; ++k)
      m.slot_rst[k] = (uint32_t)h_slot_ids[i0 + k] |
                      (h_reset && h_reset[i0 + k] ? kDecodeReset : 0u);
    ConvArgs a = conv_args(H);
    a.x = (const char *)x + (size_t)i0 * H->conv_C * es;
    a.y = (char *)y + (size_t)i0 * H->conv_C * es;
    a.state = H->conv_state;
    a.n = n;
    HIP_TRY(launch_conv_decode(H->io, a, m, s));
  }
  return SSM_OK;
}

ssm_status ssm_gate(int32_t io_dtype, int64_t rows, int32_t C, int32_t group, const void *y,
                    const void *z, const float *d_norm_w, float eps, void *out, void *stream) {
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16)
    return fail(SSM_E_INVALID_ARG, "gate: io dtype must be SSM_F32 or SSM_BF16");
  if (rows < 0 || rows > INT32_MAX || C < 1) return fail(SSM_E_INVALID_ARG, "gate: bad shape");
  if (d_norm_w && (group < 1 || C % group != 0 || C / group > 65535))
    return fail(SSM_E_INVALID_ARG, "gate: group must divide C (at most 65535 groups)");
  if (d_norm_w && !(eps >= 0.f)) return fail(SSM_E_INVALID_ARG, "gate: eps must be >= 0");
  if (rows == 0) return SSM_OK;
  if (!y || !z || !out) return fail(SSM_E_INVALID_ARG, "gate: NULL input or output");
  const size_t es = io_size(io_dtype);
  if (!aligned(y, es) || !aligned(z, es) || !aligned(out, es) || !aligned(d_norm_w, 4))
    return fail(SSM_E_INVALID_ARG, "gate: misaligned pointer");
  HIP_TRY(launch_gate(io_dtype, rows, C, group, y, z, d_norm_w, eps, out, as_stream(stream)));
  return SSM_OK;
}

ssm_status ssm_get_position(ssm_handle h, int32_t slot, int64_t *pos, uint64_t *chunk_seq) {
  GET_HANDLE(H, h);
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "bad slot %d", slot);
  if (pos) *pos = H->slots[slot].pos;
  if (chunk_seq) *chunk_seq = H->slots[slot].chunk_seq;
  return SSM_OK;
}

ssm_status ssm_get_log_state(ssm_handle h, int32_t slot, int32_t *log_len, int32_t *pending) {
  GET_HANDLE(H, h);
  if (slot < 0 || slot >= H->S) return fail(SSM_E_INVALID_ARG, "bad slot %d", slot);
  if (log_len) *log_len = H->slots[slot].log_len;
  if (pending) *pending = H->slots[slot].pend;
  return SSM_OK;
}

ssm_status ssm_get_counters(ssm_handle h, ssm_counters *out) {
  GET_HANDLE(H, h);
  if (!out) return fail(SSM_E_INVALID_ARG, "out is NULL");
  *out = H->cnt;
  return SSM_OK;
}

}  // extern "C"
