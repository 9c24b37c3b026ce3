// Static device scratch for xattn_run_noalloc: the split workspace of callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The array is a file-scope device variable: every GPU the library runs on holds its own
// copy for the life of the process. Host code never passes the array's name to a kernel
// (in host code that name is a host-side stand-in, not a device address); it resolves each
// device's address once, with that device current, through hipGetSymbolAddress, and keeps
// it per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace xattn {

namespace {
constexpr size_t kScratchBytes = size_t{32} << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

size_t static_scratch_bytes() { return kScratchBytes; }

hipError_t static_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace xattn
