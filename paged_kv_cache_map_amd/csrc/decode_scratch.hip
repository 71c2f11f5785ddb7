// Device scratch of the decode call that allocates nothing
// (pkv_paged_decode_noalloc): a static array of this file, one copy per GPU,
// which the stream-K and split-K decode kernels use for their partial
// results in place of a caller-provided workspace.

#include <mutex>

#include <hip/hip_runtime.h>

#include "pkv_internal.h"

// Each GPU the library runs on holds its own copy until the process ends.
// In host code this name is a stand-in, not the device address: host code
// uses the address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[pkv::kNoAllocScratchBytes];

namespace pkv {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {  // first call on this device, which is current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pkv
