// Slot-map scatter of new K/V rows into the paged cache.
//
// [KV-mgmt] "効率的な KV キャッシュ管理と Attention 計算", section "Triton カーネル
// による KV キャッシュ書き込み": every new token copies its whole
// [num_kv_heads, head_dim] K row and V row to cache slot slot_map[t], the slot
// addressing row slot * (heads * head_dim) of the cache.
//
// Design (gfx950): one wave64 moves one row (a token's K or a token's V), so a
// 256-thread workgroup handles two tokens.  Lanes stride the row in 16-byte
// pieces: consecutive lanes touch consecutive bytes of both the source and the
// destination row, every access is a full dwordx4, and all of a lane's loads
// are issued before its stores.  The kernel is HBM-bound (it reads and writes
// every byte once); there is no LDS and no reuse to exploit.
//
// For an fp8 cache each source element x becomes e4m3(x / scale[head]) with an
// IEEE fp32 division (the library is built with correctly rounded division)
// and round-to-nearest-even, saturating at +-448.

#include "pkv_device.hpp"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kRowsPerWg = 4;  // one row per wave
constexpr int kUnroll = 4;     // 16-byte pieces in flight per lane

// src and dst dtype equal: 16-byte pieces copied unchanged.
__device__ __forceinline__ void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                         int pieces, int lane) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int base = 0; base < pieces; base += 64 * kUnroll) {
    uint4 buf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + u * 64 + lane;
      if (p < pieces) buf[u] = s[p];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + u * 64 + lane;
      if (p < pieces) d[p] = buf[u];
    }
  }
}

// bf16 source -> fp8 cache: 16 source bytes (8 elements) -> 8 cache bytes.
__device__ __forceinline__ void quant_row_bf16(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                               const float* __restrict__ scale, int pieces,
                                               int head_dim, int lane) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint2* d = reinterpret_cast<uint2*>(dst);
  for (int base = 0; base < pieces; base += 64 * kUnroll) {
    uint4 buf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + u * 64 + lane;
      if (p < pieces) buf[u] = s[p];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + u * 64 + lane;
      if (p < pieces) {
        const float sc = scale[(p * 8) / head_dim];
        const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
        uint32_t out[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = w[e >> 1];
          const float x = (e & 1) ? bf16_hi(word) : bf16_lo(word);
          out[e >> 2] |= f32_to_e4m3(x / sc) << ((e & 3) * 8);
        }
        d[p] = make_uint2(out[0], out[1]);
      }
    }
  }
}

// fp32 source -> fp8 cache: 16 source bytes (4 elements) -> 4 cache bytes.
__device__ __forceinline__ void quant_row_f32(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                              const float* __restrict__ scale, int pieces,
                                              int head_dim, int lane) {
  const float4* s = reinterpret_cast<const float4*>(src);
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  for (int base = 0; base < pieces; base += 64 * kUnroll) {
    float4 buf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + u * 64 + lane;
      if (p < pieces) buf[u] = s[p];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + u * 64 + lane;
      if (p < pieces) {
        const float sc = scale[(p * 4) / head_dim];
        d[p] = f32_to_e4m3(buf[u].x / sc) | (f32_to_e4m3(buf[u].y / sc) << 8) |
               (f32_to_e4m3(buf[u].z / sc) << 16) | (f32_to_e4m3(buf[u].w / sc) << 24);
      }
    }
  }
}

template <int SRC, int DST>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + wave;  // 2 * token + (0: K, 1: V)
  if (row >= 2 * (int64_t)a.num_tokens) return;
  const int64_t t = row >> 1;
  const bool is_v = row & 1;
  const int32_t slot = a.slot_map[t];
  if (slot < 0 || (int64_t)slot >= a.num_slots) return;  // -1: no slot; others: out of range

  const int row_elems = a.num_kv_heads * a.head_dim;
  const int src_row_bytes = row_elems * Elt<SRC>::bytes;
  const int dst_row_bytes = row_elems * Elt<DST>::bytes;
  const uint8_t* src = (is_v ? a.v : a.k) + t * (is_v ? a.v_stride_bytes : a.k_stride_bytes);
  uint8_t* dst = (is_v ? a.v_cache : a.k_cache) + (int64_t)slot * dst_row_bytes;
  const int pieces = src_row_bytes / 16;

  if constexpr (SRC == DST) {
    copy_row(src, dst, pieces, lane);
  } else if constexpr (SRC == kBF16) {
    quant_row_bf16(src, dst, is_v ? a.v_scale : a.k_scale, pieces, a.head_dim, lane);
  } else {
    quant_row_f32(src, dst, is_v ? a.v_scale : a.k_scale, pieces, a.head_dim, lane);
  }
}

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int64_t rows = 2 * (int64_t)a.num_tokens;
  const dim3 grid((unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg));
  const dim3 block(64 * kRowsPerWg);
  if (a.src_dtype == kF32 && a.cache_dtype == kF32) {
    hipLaunchKernelGGL((kv_write_kernel<kF32, kF32>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kBF16 && a.cache_dtype == kBF16) {
    hipLaunchKernelGGL((kv_write_kernel<kBF16, kBF16>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kBF16 && a.cache_dtype == kFP8) {
    hipLaunchKernelGGL((kv_write_kernel<kBF16, kFP8>), grid, block, 0, stream, a);
  } else if (a.src_dtype == kF32 && a.cache_dtype == kFP8) {
    hipLaunchKernelGGL((kv_write_kernel<kF32, kFP8>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
