// Copy-on-write of whole cache blocks.
//
// [ch15] "KV cache / batching / paged attention", section "PagedAttention：メモ
// リを「ページ」で貸し出す": because the cache is handed out in blocks, several
// answers generated from one prompt can share the prompt's blocks, and a
// shared block is copied only at the moment one of them has to write into it
// (copy-on-write).  The host-side block manager decides which blocks to copy;
// this kernel moves their bytes: for each pair (src, dst), block src of the K
// cache and of the V cache is copied to block dst.
//
// Design (gfx950): pure data movement, HBM-bound (every byte read once and
// written once).  One workgroup moves 16 KiB of one block of one cache: each
// lane issues its four 16-byte loads before any store, consecutive lanes touch
// consecutive bytes, and loads and stores go through buffer descriptors whose
// size is the block's, so a pair naming a block outside the pool moves
// nothing (its descriptors have size zero).

#include "pkv_device.hpp"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                            // 16-byte pieces in flight per lane
constexpr int kBytesPerWg = kThreads * kUnroll * 16;  // 16 KiB
constexpr int kWord3 = 0x00020000;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyBlocksArgs a, int parts) {
  const int64_t job = blockIdx.x;  // (pair, cache, part)
  const int part = (int)(job % parts);
  const int cache = (int)((job / parts) & 1);
  const int64_t pair = job / parts / 2;
  const int32_t src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
  const bool ok = src >= 0 && src < a.num_blocks && dst >= 0 && dst < a.num_blocks;
  uint8_t* base = cache == 0 ? a.k_cache : a.v_cache;
  const int nrec = ok ? (int)a.block_bytes : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (ok ? (int64_t)src * a.block_bytes : 0)), 0, nrec, kWord3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (ok ? (int64_t)dst * a.block_bytes : 0)), 0, nrec, kWord3);
  const int off0 = part * kBytesPerWg + threadIdx.x * 16;
  u32x4_t x[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + u * kThreads * 16, 0, 0);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) __builtin_amdgcn_raw_buffer_store_b128(x[u], rd, off0 + u * kThreads * 16, 0, 0);
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  const int parts = (int)((a.block_bytes + kBytesPerWg - 1) / kBytesPerWg);
  const int64_t grid = (int64_t)a.num_pairs * 2 * parts;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a, parts);
  return hipGetLastError();
}

}  // namespace pkv
