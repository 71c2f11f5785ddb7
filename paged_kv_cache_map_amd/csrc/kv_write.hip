// Slot-map scatter of new K/V rows into the paged cache.
//
// [KV-mgmt] "効率的な KV キャッシュ管理と Attention 計算", section "Triton カーネル
// による KV キャッシュ書き込み": every new token copies its whole
// [num_kv_heads, head_dim] K row and V row to cache slot slot_map[t], the slot
// addressing row slot * (heads * head_dim) of the cache.
//
// Design (gfx950): one wave64 moves one token: its K row and its V row, seen
// as one run of 16-byte source pieces (K's pieces, then V's).  Every lane
// issues all of its loads first, with no branch in front of them (addresses
// are clamped into the rows), and only then learns the token's slot; the
// stores go through buffer descriptors whose size is zero when the slot is
// -1 or out of range, so the hardware drops them, and are non-temporal.  Consecutive lanes touch
// consecutive bytes of source and destination, every access is a full piece,
// and no lane waits on the slot map before its reads are in flight.  The
// kernel is HBM-bound (every byte is read and written once); there is no LDS
// and no reuse.
//
// For an fp8 cache each source element x becomes e4m3(x / scale[head]) with an
// IEEE fp32 division (the library is built with correctly rounded division)
// and round-to-nearest-even, saturating at +-448; for an int8 cache the
// quotient is rounded to the nearest integer (ties to even) and saturated to
// [-127, 127].

#include "pkv_device.hpp"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kTokensPerWg = 4;  // one token per wave
#ifndef PKV_WRITE_UNROLL
#define PKV_WRITE_UNROLL 4
#endif
constexpr int kUnroll = PKV_WRITE_UNROLL;  // source pieces in flight per lane per pass
constexpr int kWord3 = 0x00020000;
// Cache policy of the row stores: non-temporal (the rows are not read again
// by this kernel, and leaving them out of the caches keeps the source rows,
// often fresh from the kernel that produced them, resident).
constexpr int kStoreNT = 2;
constexpr int kDropped = 0x7ffffff0;  // a buffer offset past any row: the store is dropped

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int SRC, int DST>
__device__ __forceinline__ void store_piece(__amdgpu_buffer_rsrc_t r, int off, u32x4_t v) {
  if constexpr (SRC == DST) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStoreNT);
  } else if constexpr (SRC == kBF16) {
    const u32x2_t w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kStoreNT);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(v.x, r, off, 0, kStoreNT);
  }
}

template <int SRC, int DST>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerWg +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.num_tokens) return;

  constexpr int src_elt = Elt<SRC>::bytes;
  constexpr int dst_piece = 16 * Elt<DST>::bytes / src_elt;  // cache bytes per source piece
  const int row_elems = a.num_kv_heads * a.head_dim;
  const int pieces = row_elems * src_elt / 16;               // per row
  const int dst_row_bytes = row_elems * Elt<DST>::bytes;
  const uint4* ksrc = reinterpret_cast<const uint4*>(a.k + t * a.k_stride_bytes);
  const uint4* vsrc = reinterpret_cast<const uint4*>(a.v + t * a.v_stride_bytes);
  const int elems_per_piece = 16 / src_elt;

  for (int base = 0; base < 2 * pieces; base += 64 * kUnroll) {
    uint4 buf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = min(base + u * 64 + lane, 2 * pieces - 1);
      buf[u] = q < pieces ? ksrc[q] : vsrc[q - pieces];
    }
    // the slot is needed only by the stores
    const int32_t slot = a.slot_map[t];
    const bool ok = slot >= 0 && (int64_t)slot < a.num_slots;
    const int64_t dst_off = ok ? (int64_t)slot * dst_row_bytes : 0;
    const int nrec = ok ? dst_row_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_cache + dst_off), 0, nrec, kWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.v_cache + dst_off), 0, nrec, kWord3);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = base + u * 64 + lane;
      const bool is_k = q < pieces;
      const bool is_v = !is_k && q < 2 * pieces;
      float sc = 1.0f;
      if constexpr (scaled8(DST)) {
        const int qq = min(q, 2 * pieces - 1);
        const int e = (is_k ? qq : qq - pieces) * elems_per_piece;
        sc = (is_k ? a.k_scale : a.v_scale)[e / a.head_dim];
      }
      const u32x4_t v = convert_piece<SRC, DST>(buf[u], sc);
      store_piece<SRC, DST>(kr, is_k ? q * dst_piece : kDropped, v);
      store_piece<SRC, DST>(vr, is_v ? (q - pieces) * dst_piece : kDropped, v);
    }
  }
}

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.num_tokens + kTokensPerWg - 1) / kTokensPerWg));
  const dim3 block(64 * kTokensPerWg);
  if (a.src_dtype == kF32 && a.cache_dtype == kF32) {
    hipLaunchKernelGGL((kv_write_kernel<kF32, kF32>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kBF16 && a.cache_dtype == kBF16) {
    hipLaunchKernelGGL((kv_write_kernel<kBF16, kBF16>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kBF16 && a.cache_dtype == kFP8) {
    hipLaunchKernelGGL((kv_write_kernel<kBF16, kFP8>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kF32 && a.cache_dtype == kFP8) {
    hipLaunchKernelGGL((kv_write_kernel<kF32, kFP8>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kBF16 && a.cache_dtype == kI8) {
    hipLaunchKernelGGL((kv_write_kernel<kBF16, kI8>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kF32 && a.cache_dtype == kI8) {
    hipLaunchKernelGGL((kv_write_kernel<kF32, kI8>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
