// host_fuzz.cpp -- drives the host runtime's input checks under AddressSanitizer
// and UndefinedBehaviorSanitizer, on the CPU, with no GPU: the state-blob
// parser (truncations at every length, every single-byte change of a valid
// blob, random bytes, hostile array counts, ranks and extents), resume
// receipts, and the metadata of packed and chunked scans.  Every case must be
// refused before any device work (the device pointers passed are never
// dereferenced), so a sanitizer report or a crash is a host bug.  Bounded and
// seeded; exits non-zero at the first unexpected result.
//
// usage: host_fuzz [iterations]
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "ssm_stream.h"

static void *const FAKE = (void *)0x1000;  // never dereferenced

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545f4914f6cdd1dull;
}

static void put_u32(std::vector<uint8_t> &b, uint32_t v) {
  for (int i = 0; i < 4; ++i) b.push_back((uint8_t)(v >> (8 * i)));
}

static uint64_t checksum(const float *v, size_t n) {
  uint64_t s = 0;
  for (size_t i = 0; i < n; ++i) {
    uint32_t w;
    memcpy(&w, v + i, 4);
    s += (uint64_t)w * (2ull * i + 1ull);
  }
  return s;
}

static int fails = 0;
#define EXPECT(cond, ...)                  \
  do {                                     \
    if (!(cond)) {                         \
      fprintf(stderr, __VA_ARGS__);        \
      fprintf(stderr, "\n");               \
      ++fails;                             \
      return;                              \
    }                                      \
  } while (0)

static const int H = 2, P = 4, N = 8;

static ssm_handle make_handle(int recurrence) {
  ssm_layer_desc d = {H, P, N, 1, SSM_F32, 3, 77, recurrence, 0};
  ssm_handle h = 0;
  if (ssm_create(&d, 4, (float *)FAKE, (const float *)FAKE,
                 recurrence == SSM_MAMBA2 ? (const float *)FAKE : nullptr, 0, &h) != SSM_OK) {
    fprintf(stderr, "create failed: %s\n", ssm_last_error());
    exit(2);
  }
  return h;
}

// A well-formed one-array blob of a [H, P, N] state and its receipt.
static void good_blob(std::vector<uint8_t> &b, ssm_receipt &r, std::vector<float> &state) {
  state.resize(H * P * N);
  for (size_t i = 0; i < state.size(); ++i) state[i] = (float)i / 64.f;
  b.clear();
  put_u32(b, 1);  // version
  put_u32(b, 1);  // arrays
  put_u32(b, 3);
  put_u32(b, H);
  put_u32(b, P);
  put_u32(b, N);
  put_u32(b, 0);  // fp32
  const uint8_t *p = (const uint8_t *)state.data();
  b.insert(b.end(), p, p + state.size() * 4);
  memset(&r, 0, sizeof r);
  r.stream_id = 5;
  r.model_rev = 77;
  r.code_rev = ssm_code_rev();
  r.schema_version = 3;
  r.state_dtype = SSM_F32;
  r.H = H;
  r.P = P;
  r.N = N;
  r.G = 1;
  r.position = 10;
  r.chunk_seq = 2;
  r.checksum = checksum(state.data(), state.size());
  r.recurrence = SSM_MAMBA2;
}

// A blob that parses and checks out would be copied to the device: with no
// GPU the copy fails (SSM_E_HIP).  Anything else must be a refusal.
static bool refused_or_hip(ssm_status st) {
  return st == SSM_E_SCHEMA || st == SSM_E_INVALID_ARG || st == SSM_E_HIP;
}

static void fuzz_blobs(ssm_handle h, long iters) {
  std::vector<uint8_t> b;
  ssm_receipt r;
  std::vector<float> state;
  good_blob(b, r, state);
  // every truncation
  for (size_t n = 0; n < b.size(); ++n) {
    std::vector<uint8_t> t(b.begin(), b.begin() + n);
    t.reserve(1);  // a real pointer even for the empty prefix
    const ssm_status st = ssm_state_deserialize(h, 1, t.data(), t.size(), &r, nullptr);
    EXPECT(st == SSM_E_SCHEMA, "truncated blob of %zu bytes: status %d", n, (int)st);
  }
  // every single-byte change
  for (size_t i = 0; i < b.size(); ++i)
    for (int bit = 0; bit < 8; ++bit) {
      std::vector<uint8_t> t = b;
      t[i] ^= (uint8_t)(1u << bit);
      const ssm_status st = ssm_state_deserialize(h, 1, t.data(), t.size(), &r, nullptr);
      EXPECT(refused_or_hip(st), "flipped bit %d of byte %zu: status %d", bit, i, (int)st);
      EXPECT(i < 28 || st != SSM_E_HIP, "a changed payload passed its checksum");
    }
  // hostile headers: huge counts, ranks and extents
  const uint32_t hostile[] = {0u, 1u, 2u, 16u, 17u, 0x7fffffffu, 0x80000000u, 0xffffffffu};
  for (uint32_t n_arrays : hostile)
    for (uint32_t rank : hostile)
      for (uint32_t ext : hostile) {
        std::vector<uint8_t> t;
        put_u32(t, 1);
        put_u32(t, n_arrays);
        put_u32(t, rank);
        for (uint32_t k = 0; k < (rank < 20 ? rank : 20u); ++k) put_u32(t, ext);
        put_u32(t, 0);
        t.resize(t.size() + 64, 0);
        const ssm_status st = ssm_state_deserialize(h, 1, t.data(), t.size(), &r, nullptr);
        EXPECT(st == SSM_E_SCHEMA, "hostile header %u/%u/%u: status %d", n_arrays, rank, ext,
               (int)st);
      }
  // random mutations and random bytes
  for (long it = 0; it < iters; ++it) {
    std::vector<uint8_t> t = b;
    const int k = 1 + (int)(next_u64() % 8);
    for (int j = 0; j < k; ++j) {
      const uint64_t u = next_u64();
      switch (u % 4) {
        case 0: if (!t.empty()) t[(u >> 8) % t.size()] = (uint8_t)(u >> 40); break;
        case 1: t.resize((u >> 8) % (t.size() + 64)); break;
        case 2: t.insert(t.begin() + (u >> 8) % (t.size() + 1), (uint8_t)(u >> 40)); break;
        default: if (!t.empty()) t.erase(t.begin() + (u >> 8) % t.size());
      }
    }
    if (next_u64() % 16 == 0) {
      t.resize(next_u64() % 512);
      for (auto &c : t) c = (uint8_t)next_u64();
    }
    ssm_receipt rr = r;
    if (next_u64() % 4 == 0) rr.checksum = next_u64();
    t.reserve(1);
    const ssm_status st = ssm_state_deserialize(h, 1, t.data(), t.size(), &rr, nullptr);
    EXPECT(refused_or_hip(st), "random blob: status %d", (int)st);
  }
  int64_t pos = -1;
  uint64_t cs = 9;
  ssm_get_position(h, 1, &pos, &cs);
  EXPECT(pos == 0 && cs == 0, "a refused blob changed the slot (pos %lld)", (long long)pos);
}

static void fuzz_receipts(ssm_handle h, long iters) {
  std::vector<uint8_t> b;
  ssm_receipt good;
  std::vector<float> state;
  good_blob(b, good, state);
  for (long it = 0; it < iters; ++it) {
    ssm_receipt r = good;
    uint8_t *p = (uint8_t *)&r;
    const int k = 1 + (int)(next_u64() % 3);
    for (int j = 0; j < k; ++j) p[next_u64() % sizeof r] = (uint8_t)next_u64();
    const ssm_status st = ssm_state_restore(h, 0, (const float *)FAKE, &r, nullptr);
    EXPECT(refused_or_hip(st), "restore with a changed receipt: status %d", (int)st);
  }
}

static void fuzz_scan_metadata(ssm_handle h, long iters) {
  for (long it = 0; it < iters; ++it) {
    const int nseq = (int)(next_u64() % 6);
    std::vector<int32_t> cu(nseq + 1), slots(nseq + 1);
    std::vector<uint8_t> cont(nseq + 1);
    std::vector<uint64_t> seq(nseq + 1);
    for (int i = 0; i <= nseq; ++i) {
      cu[i] = (int32_t)(next_u64() % 5) - 1 + (i ? cu[i - 1] : 0);
      slots[i] = (int32_t)(next_u64() % 6) - 1;
      cont[i] = (uint8_t)(next_u64() % 2);
      seq[i] = next_u64() % 3;
    }
    cu[0] = (int32_t)(next_u64() % 3) - 1;
    // only a continuation of empty sequences may pass on the host; a fresh
    // empty sequence or a token would reach the device
    for (int i = 0; i < nseq; ++i)
      if (!cont[i] || cu[i + 1] != cu[i]) cu[i + 1] = cu[i] - 1;  // keep it a refusal
    const ssm_status st =
        ssm_scan_packed(h, nseq, cu.data(), slots.data(), cont.data(), seq.data(), FAKE, FAKE,
                        FAKE, FAKE, FAKE, nullptr, nullptr, nullptr);
    EXPECT(st == SSM_OK || st == SSM_E_INVALID_ARG || st == SSM_E_SEQUENCE,
           "scan packed: status %d", (int)st);
    // chunked scan: checkpoint lists and lengths
    const int n_ck = (int)(next_u64() % 4);
    std::vector<int64_t> ck(n_ck + 1);
    for (auto &c : ck) c = (int64_t)(next_u64() % 12) - 2;
    const int64_t L = (int64_t)(next_u64() % 10) - 2;
    uint64_t expect = 0;
    ssm_get_position(h, 3, nullptr, &expect);
    const uint64_t cseq = expect + (next_u64() % 3) - 1;
    const ssm_status s2 = ssm_scan_chunk(h, 3, cseq, L, FAKE, FAKE, FAKE, FAKE, nullptr, FAKE,
                                         n_ck, ck.data(), (float *)FAKE, nullptr, 0, nullptr);
    EXPECT(s2 == SSM_OK || s2 == SSM_E_INVALID_ARG || s2 == SSM_E_SEQUENCE || s2 == SSM_E_HIP,
           "scan chunk: status %d", (int)s2);
    EXPECT(s2 != SSM_OK || L == 0, "a non-empty chunk passed with no GPU");
  }
}

int main(int argc, char **argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 20000;
  ssm_handle h = make_handle(SSM_MAMBA2);
  ssm_handle g = make_handle(SSM_GATED_DELTA);
  fuzz_blobs(h, iters);
  fuzz_receipts(h, iters);
  fuzz_receipts(g, iters / 4);
  fuzz_scan_metadata(h, iters);
  ssm_destroy(h);
  ssm_destroy(g);
  if (fails) return 1;
  printf("host_fuzz: %ld iterations per part, no failure\n", iters);
  return 0;
}
