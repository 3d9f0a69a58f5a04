// ssm_static.hip -- the library's fixed device scratch, for callers that
// cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid hipMalloc): ssm_scan_chunk_static runs the
// chunk scan with this array as its workspace.
//
// Every GPU the library runs on holds its own copy of the array, from module
// load until the process ends.  In host code the array's name only stands in
// for it: the device address of a device's copy comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept; kernels and copies are only ever given that address.
#include <mutex>

#include "ssm_internal.h"
#include "ssm_stream.h"

namespace ssm {

// [0, SSM_STATIC_WORKSPACE_BYTES): the scan workspace; then the finite-check
// flag (8 bytes used).
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace ssm
