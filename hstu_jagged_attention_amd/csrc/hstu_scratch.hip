// Static device scratch of the allocation-free entry point (hstu_fwd_noalloc).
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the workspace of
// the tile scheduler from a fixed array in the library's own device memory.
// Each GPU the library runs on holds its own copy of the array until the
// process ends. The host-side name `scratch` is only a stand-in for the
// device variable; its device address on the current GPU is taken once per
// device with hipGetSymbolAddress and used everywhere the host needs it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_workspace(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

}  // namespace hstu
