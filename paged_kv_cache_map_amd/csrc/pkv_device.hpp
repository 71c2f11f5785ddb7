// Device helpers shared by the HIP kernels of libpkv (gfx950 only).
//
// bf16 is handled as raw 16-bit patterns packed two per 32-bit word (the low
// half holds the lower-indexed element); fp32 values come from a bf16 by
// placing its bits in the upper half of the word.  fp8 is OCP E4M3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kI8 = 3 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so exp2 never sees inf - inf

// Caches of one byte per element, decoded as code x per-head scale.
constexpr bool scaled8(int ct) { return ct == kFP8 || ct == kI8; }

template <int T>
struct Elt;
template <>
struct Elt<kF32> { static constexpr int bytes = 4; };
template <>
struct Elt<kBF16> { static constexpr int bytes = 2; };
template <>
struct Elt<kFP8> { static constexpr int bytes = 1; };
template <>
struct Elt<kI8> { static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round an fp32 to bf16, nearest-even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// a.lo*b.lo + a.hi*b.hi + c, both operands bf16 pairs (products exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> two bf16 in one word.  Every E4M3
// value is exactly representable in bf16, so this is exact.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}

// Two E4M3 codes -> two fp32 (exact).
template <bool HIGH>
__device__ __forceinline__ float2_t e4m3x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HIGH);
}

// Two int8 codes (bytes 0,1 or 2,3 of w) -> two bf16 in one word.  Exact:
// an integer of magnitude <= 128 has at most 8 significant bits, so its fp32
// value has zero low halves and the bf16 is its upper half.
template <bool HIGH>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w) {
  constexpr int sh = HIGH ? 16 : 0;
  const uint32_t lo = __float_as_uint((float)((int32_t)(w << (24 - sh)) >> 24));
  const uint32_t hi = __float_as_uint((float)((int32_t)(w << (16 - sh)) >> 24));
  return (lo >> 16) | (hi & 0xffff0000u);
}

template <bool HIGH>
__device__ __forceinline__ float2_t i8x2_to_f32x2(uint32_t w) {
  constexpr int sh = HIGH ? 16 : 0;
  return float2_t{(float)((int32_t)(w << (24 - sh)) >> 24), (float)((int32_t)(w << (16 - sh)) >> 24)};
}

// The one-byte cache codes of type CT (fp8 E4M3 or int8) -> bf16 / fp32, exactly.
template <int CT, bool HIGH>
__device__ __forceinline__ uint32_t code8x2_to_bf16x2(uint32_t w) {
  if constexpr (CT == kI8) return i8x2_to_bf16x2<HIGH>(w);
  else return e4m3x2_to_bf16x2<HIGH>(w);
}

template <int CT, bool HIGH>
__device__ __forceinline__ float2_t code8x2_to_f32x2(uint32_t w) {
  if constexpr (CT == kI8) return i8x2_to_f32x2<HIGH>(w);
  else return e4m3x2_to_f32x2<HIGH>(w);
}

// fp32 -> int8 code: round to nearest, ties to even; saturated to [-127, 127]
// (symmetric: -128 is never produced); NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_i8(float x) {
  if (x != x) return 0u;
  const float r = __builtin_rintf(fminf(fmaxf(x, -127.0f), 127.0f));
  return (uint32_t)(int32_t)r & 0xffu;
}

// fp32 -> E4M3 code: round to nearest, ties to even mantissa; |x| >= 448 and
// +-inf saturate to +-448; NaN -> 0x7F.  Integer formulation on the fp32 bits.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // 448.0f
  if (a < 0x3c800000u) {                      // below 2^-6: spacing 2^-9
    // a * 2^9 is exact; rint rounds half to even; m == 8 is the smallest normal
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)m;
  }
  // normal binade: keep 3 mantissa bits, nearest-even; rebias 127 -> 7
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int DST>
__device__ __forceinline__ uint32_t encode8(float x) {
  if constexpr (DST == kI8) return f32_to_i8(x);
  else return f32_to_e4m3(x);
}

// 16 source bytes of a K or V row -> the cache's bytes for them (16, 8 or 4,
// in the low words): a bit copy when the types match, else the one-byte
// encoding (fp8 E4M3 or int8) of x / scale with an IEEE fp32 division (the
// library is built with correctly rounded division).  Every cache write of the library goes through
// this one function, so the slot-map scatter and the appending decode store
// identical bits.
template <int SRC, int DST>
__device__ __forceinline__ u32x4_t convert_piece(uint4 x, float sc) {
  u32x4_t o = {x.x, x.y, x.z, x.w};
  if constexpr (SRC == kBF16 && scaled8(DST)) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
      out[e >> 2] |= encode8<DST>(v / sc) << ((e & 3) * 8);
    }
    o.x = out[0];
    o.y = out[1];
  } else if constexpr (SRC == kF32 && scaled8(DST)) {
    o.x = encode8<DST>(__uint_as_float(x.x) / sc) | (encode8<DST>(__uint_as_float(x.y) / sc) << 8) |
          (encode8<DST>(__uint_as_float(x.z) / sc) << 16) |
          (encode8<DST>(__uint_as_float(x.w) / sc) << 24);
  }
  return o;
}

// Keys a decode attends: cache_seqlens[b] (raw) plus bias (1 when the call
// appends the step's token itself), clamped to [0, cap].
__device__ __forceinline__ int clamp_keys(int raw, int bias, int cap) {
  const int64_t x = (int64_t)raw + bias;
  return x < 0 ? 0 : (x > cap ? cap : (int)x);
}

// ---------------------------------------------------------------------------
// cross-lane helpers (wave64)
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xf, 0xf, true));
}

// Sum over the 4 lanes of each quad, result in every lane of the quad.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<0xb1>(x);  // quad_perm [1,0,3,2]
  x += dpp<0x4e>(x);  // quad_perm [2,3,0,1]
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// Max / sum over lanes that share (lane & 3), i.e. across the 16 quads.
__device__ __forceinline__ float max_across_quads(float x) {
  x = fmaxf(x, shfl_xor(x, 4));
  x = fmaxf(x, shfl_xor(x, 8));
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float sum_across_quads(float x) {
  x += shfl_xor(x, 4);
  x += shfl_xor(x, 8);
  x += shfl_xor(x, 16);
  x += shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes
// 0..31 of its second.  Given x twice, the two results hold, in every lane l,
// x[l] and x[l ^ 32] in some order: enough for a symmetric combine.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace pkv
