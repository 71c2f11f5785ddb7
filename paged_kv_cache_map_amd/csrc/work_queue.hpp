// Run-time work distribution of the persistent prefill: counters that the
// workgroups of one launch take work items from, one counter per XCD, each
// on a 128-byte line of its own.
//
// The counters live in one static device array of kSlots sets.  Each stream
// gets a set on first use (kernels on one stream never overlap, so one set
// per stream is enough); once kSlots streams hold one, later streams get -1
// and their launches run without counters.  Included into one translation
// unit.
#pragma once

#include <mutex>

#include <hip/hip_runtime.h>

namespace pkv {
namespace wq {

constexpr int kSlots = 64;
constexpr int kStride = 32;              // words from one counter to the next
constexpr int kSetWords = 8 * kStride;   // one set: a counter per XCD

__device__ uint32_t g_counters[kSlots * kSetWords];

// The counter set of a slot, device side.
__device__ __forceinline__ uint32_t* counters(int slot) { return g_counters + slot * kSetWords; }

__global__ void reset_kernel(int slot) {
  if (threadIdx.x < 8) counters(slot)[threadIdx.x * kStride] = 0u;
}

// Clear a counter set on `stream` (a fill kernel rather than a memset, so
// that the call can be captured in a graph).
__host__ inline hipError_t reset(int slot, hipStream_t stream) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(64), 0, stream, slot);
  return hipGetLastError();
}

// The slot of `stream` (-1 once every slot is taken).
__host__ inline int slot_of(hipStream_t stream) {
  static std::mutex mu;
  static hipStream_t keys[kSlots];
  static int used = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (keys[i] == stream) return i;
  if (used == kSlots) return -1;
  keys[used] = stream;
  return used++;
}

}  // namespace wq
}  // namespace pkv
