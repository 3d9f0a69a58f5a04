// abi_latency.cpp -- per-call cost of ssm_scan_chunk through the C ABI with no
// binding in the loop.  One stream of a Mamba-130M-shaped layer (H = 24,
// P = 64, N = 128, fp32 io, 2,048 tokens) is scanned in chunks of each given
// size; for every size it reports, per call:
//   enqueue_us  host time spent inside ssm_scan_chunk (validation, metadata,
//               kernel launches; nothing in the loop synchronises),
//   wall_us     host time from the first call until the stream has finished,
//   gpu_us      device time between events recorded around all the calls.
// Small chunks "underuse hardware" ("Mamba Streaming State That Survives
// Chunking", section "Separate Mamba-2 algebra from kernel behavior"): these
// three figures separate what the library's host side, the launches and the
// kernels each cost.  Inputs are zeros (finite; the kernels do the same work
// for any values).  Prints one JSON object.
//
// usage: ssm_abi_latency [chunk sizes...]   (default 1 17 64 256 2048)
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <chrono>
#include <vector>

#include "ssm_stream.h"

#define CHECK_HIP(e)                                                              \
  do {                                                                            \
    hipError_t r_ = (e);                                                          \
    if (r_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s: %s\n", #e, hipGetErrorString(r_));                     \
      return 1;                                                                   \
    }                                                                             \
  } while (0)
#define CHECK_SSM(e)                                                              \
  do {                                                                            \
    ssm_status r_ = (e);                                                          \
    if (r_ != SSM_OK) {                                                           \
      fprintf(stderr, "%s: %d %s\n", #e, (int)r_, ssm_last_error());              \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

static double now_us() {
  using namespace std::chrono;
  return duration<double, std::micro>(steady_clock::now().time_since_epoch()).count();
}

int main(int argc, char **argv) {
  const int L = 2048, H = 24, P = 64, N = 128, G = 1;
  std::vector<int> sizes;
  for (int i = 1; i < argc; ++i) sizes.push_back(atoi(argv[i]));
  if (sizes.empty()) sizes = {1, 17, 64, 256, 2048};
  for (int c : sizes)
    if (c < 1 || c > L) {
      fprintf(stderr, "chunk sizes must be in [1, %d]\n", L);
      return 2;
    }
  const size_t fb = sizeof(float);
  float *x, *dt, *B, *C, *y, *state, *A, *D;
  void *ws;
  ssm_layer_desc desc = {H, P, N, G, SSM_F32, 1, 0};
  const size_t ws_bytes = ssm_scan_workspace_bytes(&desc, L);
  CHECK_HIP(hipMalloc(&x, (size_t)L * H * P * fb));
  CHECK_HIP(hipMalloc(&y, (size_t)L * H * P * fb));
  CHECK_HIP(hipMalloc(&dt, (size_t)L * H * fb));
  CHECK_HIP(hipMalloc(&B, (size_t)L * G * N * fb));
  CHECK_HIP(hipMalloc(&C, (size_t)L * G * N * fb));
  CHECK_HIP(hipMalloc(&state, (size_t)H * P * N * fb));
  CHECK_HIP(hipMalloc(&A, H * fb));
  CHECK_HIP(hipMalloc(&D, H * fb));
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMemset(x, 0, (size_t)L * H * P * fb));
  CHECK_HIP(hipMemset(dt, 0, (size_t)L * H * fb));
  CHECK_HIP(hipMemset(B, 0, (size_t)L * G * N * fb));
  CHECK_HIP(hipMemset(C, 0, (size_t)L * G * N * fb));
  CHECK_HIP(hipMemset(A, 0, H * fb));
  CHECK_HIP(hipMemset(D, 0, H * fb));
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  ssm_handle h;
  CHECK_SSM(ssm_create(&desc, 1, state, A, D, 0, &h));
  const int32_t slot0 = 0;
  printf("{\"layer\": \"H=%d P=%d N=%d fp32, %d tokens\", \"chunks\": [", H, P, N, L);
  for (size_t k = 0; k < sizes.size(); ++k) {
    const int c = sizes[k];
    const int calls = (L + c - 1) / c;
    double enq = 0, wall = 0;
    float gpu_ms = 0;
    for (int rep = 0; rep < 3; ++rep) {  // the first pass warms caches and code
      CHECK_SSM(ssm_state_reset(h, 1, &slot0, s));
      CHECK_HIP(hipStreamSynchronize(s));
      const double t0 = now_us();
      CHECK_HIP(hipEventRecord(e0, s));
      double inside = 0;
      for (int q = 0; q < calls; ++q) {
        const int64_t t = (int64_t)q * c, n = t + c <= L ? c : L - t;
        const double a = now_us();
        CHECK_SSM(ssm_scan_chunk(h, 0, (uint64_t)q, n, x + t * H * P, dt + t * H, B + t * G * N,
                                 C + t * G * N, nullptr, y + t * H * P, 0, nullptr, nullptr, ws,
                                 ws_bytes, s));
        inside += now_us() - a;
      }
      CHECK_HIP(hipEventRecord(e1, s));
      CHECK_HIP(hipEventSynchronize(e1));
      const double t1 = now_us();
      if (rep > 0) {  // mean of the two warm passes
        float ms = 0;
        CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
        gpu_ms += ms / 2;
        enq += inside / 2;
        wall += (t1 - t0) / 2;
      }
    }
    printf("%s{\"chunk\": %d, \"calls\": %d, \"enqueue_us\": %.3f, \"wall_us\": %.3f, "
           "\"gpu_us\": %.3f}",
           k ? ", " : "", c, calls, enq / calls, wall / calls, gpu_ms * 1e3 / calls);
  }
  printf("]}\n");
  CHECK_SSM(ssm_destroy(h));
  return 0;
}
