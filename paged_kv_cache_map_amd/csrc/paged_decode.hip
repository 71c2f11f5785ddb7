// Paged decode: one query token per sequence over its cached keys, with a
// split-K plan over long contexts and a merge pass.
//
// [paged-doc] "ページド・アテンション", section デコードパス: a decode batch has one
// query per sequence; the kernel reads the sequence's K/V through its
// block-table row and its cached length.  [ch15] "KV cache / batching / paged
// attention", section "生成は2つのフェーズでできている": decode re-reads memory
// while the arithmetic units idle, so this kernel is built to stream HBM.
// [ch15] section "FlashAttention：注意計算そのものを速く": tiling with an online
// softmax gives exactly the plain result, which is what makes splitting the
// keys and merging partial (max, sum, output) triples exact algebra.
//
// Work decomposition (gfx950):
// * workgroup = (split s, KV head g [x q-head group], sequence b), 4 waves;
//   it serves all G q heads that share KV head g, so every K/V byte is read
//   from HBM once per step.
// * each wave takes every 4th chunk of 32 keys of the split and runs its own
//   online softmax; the four waves merge in LDS at the end; splits of one
//   sequence merge in a second kernel (or the workgroup writes the final row
//   when the sequence fits in one split).
// * Q.K layout: lane = 4 * key + quarter.  The four lanes of a quad read one
//   key's row in 16-byte pieces (a 64-byte contiguous run per instruction per
//   key), dot their quarter of head_dim against every q head held in
//   registers, and a two-step DPP quad sum finishes the dot product.
// * P.V layout: lane = slice of head_dim; each key's V row is read by the whole
//   wave with 4-byte (or 8-byte) loads, fully coalesced; p is broadcast from
//   LDS.
// * Loads of the next chunk are issued before the current chunk is computed
//   (two register buffers), keeping 2 x 16 KiB per wave in flight.
// * fp8 caches are dequantised in registers (exact E4M3 -> bf16); the K scale
//   folds into the logit scale and the V scale into the output.

#include "pkv_device.hpp"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = kDecodeWaves;
constexpr int kChunk = kDecodeChunk;  // keys per wave iteration (2 sub-steps of 16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;   // running-max start: finite, so exp2 never sees inf - inf

template <int CT, int D, int GW>
struct Cfg {
  static constexpr int elt = Elt<CT>::bytes;
  static constexpr int row_bytes = D * elt;  // one KV head's row
  // Q.K layout: 4 lanes per key
  static constexpr int qk_loads = row_bytes / 64;  // 16-byte loads per lane per key
  static constexpr int qk_elems = D / 4;
  // q words per head: bf16 pairs (bf16/fp8 caches) or fp32 values (fp32 cache)
  static constexpr int q_words = (CT == kF32) ? qk_elems : qk_elems / 2;
  // P.V layout
  static constexpr int pv_vec = (row_bytes / 64 > 4) ? row_bytes / 64 : 4;  // bytes per lane per key
  static constexpr int pv_lanes = row_bytes / pv_vec;                        // lanes per key row
  static constexpr int pv_kp = 64 / pv_lanes;                                // keys per load instr
  static constexpr int pv_nv = pv_vec / elt;                                 // elements per lane
  static constexpr int pv_loads = kChunk / pv_kp;                            // per chunk
  static_assert(qk_loads >= 1 && pv_kp >= 1 && pv_kp <= 16, "shape");
};

// Registers holding one chunk's K (Q.K layout) and V (P.V layout).
template <int CT, int D, int GW>
struct ChunkRegs {
  using C = Cfg<CT, D, GW>;
  uint4 k[2][C::qk_loads];
  uint32_t v[C::pv_loads][C::pv_vec / 4];
  bool kok[2];  // this lane's key of each sub-step exists and sits in a valid block
};

struct SeqCtx {
  const uint8_t* kbase;  // cache + g * row_bytes
  const uint8_t* vbase;
  int64_t slot_stride;   // bytes between slots = num_kv_heads * row_bytes
  const int32_t* tbl;    // LDS: block ids of the split, first entry = block blk0
  int blk0;
  int log2bs;
  int bs_mask;
  int lk;
};

__device__ __forceinline__ int64_t slot_of_key(const SeqCtx& s, int key, bool& ok) {
  const int blk = s.tbl[(key >> s.log2bs) - s.blk0];
  ok = blk >= 0;
  return ((int64_t)blk << s.log2bs) + (key & s.bs_mask);
}

template <int CT, int D, int GW>
__device__ __forceinline__ void load_chunk(ChunkRegs<CT, D, GW>& r, const SeqCtx& s, int start,
                                           int lane) {
  using C = Cfg<CT, D, GW>;
  const int kq = lane >> 2, quarter = lane & 3;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int key = start + sb * 16 + kq;
    bool ok = key < s.lk;
    int64_t slot = 0;
    if (ok) slot = slot_of_key(s, key, ok);
    r.kok[sb] = ok;
    const uint8_t* row = s.kbase + slot * s.slot_stride + quarter * 16;
#pragma unroll
    for (int i = 0; i < C::qk_loads; ++i) {
      if (ok) {
        r.k[sb][i] = *reinterpret_cast<const uint4*>(row + i * 64);
      } else {
        r.k[sb][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  const int kp = lane / C::pv_lanes;
  const int off = (lane % C::pv_lanes) * C::pv_vec;
#pragma unroll
  for (int i = 0; i < C::pv_loads; ++i) {
    const int key = start + i * C::pv_kp + kp;
    bool ok = key < s.lk;
    int64_t slot = 0;
    if (ok) slot = slot_of_key(s, key, ok);
    const uint8_t* row = s.vbase + slot * s.slot_stride + off;
#pragma unroll
    for (int w = 0; w < C::pv_vec / 4; ++w) {
      r.v[i][w] = ok ? reinterpret_cast<const uint32_t*>(row)[w] : 0u;
    }
  }
}

// Partial dot product of one key's quarter row with head h's q words.
template <int CT, int D, int GW>
__device__ __forceinline__ float qk_partial(const uint4 (&k)[Cfg<CT, D, GW>::qk_loads],
                                            const uint32_t* qh) {
  using C = Cfg<CT, D, GW>;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < C::qk_loads; ++i) {
    const uint32_t kw[4] = {k[i].x, k[i].y, k[i].z, k[i].w};
    if constexpr (CT == kBF16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = dot2_bf16(qh[i * 4 + j], kw[j], acc);
    } else if constexpr (CT == kFP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = dot2_bf16(qh[i * 8 + 2 * j], e4m3x2_to_bf16x2<false>(kw[j]), acc);
        acc = dot2_bf16(qh[i * 8 + 2 * j + 1], e4m3x2_to_bf16x2<true>(kw[j]), acc);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(__uint_as_float(qh[i * 4 + j]), __uint_as_float(kw[j]), acc);
    }
  }
  return acc;
}

// The pv_nv fp32 values of one lane's V slice.
template <int CT, int D, int GW>
__device__ __forceinline__ void v_values(const uint32_t* w, float* out) {
  using C = Cfg<CT, D, GW>;
  if constexpr (CT == kBF16) {
#pragma unroll
    for (int j = 0; j < C::pv_vec / 4; ++j) {
      out[2 * j] = bf16_lo(w[j]);
      out[2 * j + 1] = bf16_hi(w[j]);
    }
  } else if constexpr (CT == kFP8) {
#pragma unroll
    for (int j = 0; j < C::pv_vec / 4; ++j) {
      const float2_t a = e4m3x2_to_f32x2<false>(w[j]);
      const float2_t b = e4m3x2_to_f32x2<true>(w[j]);
      out[4 * j] = a.x;
      out[4 * j + 1] = a.y;
      out[4 * j + 2] = b.x;
      out[4 * j + 3] = b.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::pv_vec / 4; ++j) out[j] = __uint_as_float(w[j]);
  }
}

template <int CT, int D, int GW>
struct WaveState {
  using C = Cfg<CT, D, GW>;
  float m[GW];                 // running max (log2 domain), uniform across the wave
  float l[GW];                 // per-lane partial sums of p (replicated within a quad)
  float o[GW][C::pv_nv];       // per-lane partial outputs (keys = kp mod pv_kp)
};

template <int CT, int D, int GW>
__device__ __forceinline__ void compute_chunk(WaveState<CT, D, GW>& st, const ChunkRegs<CT, D, GW>& r,
                                              const uint32_t (&q)[GW][Cfg<CT, D, GW>::q_words],
                                              float logit_scale, int lane,
                                              float* p_lds) {
  using C = Cfg<CT, D, GW>;
  const int kq = lane >> 2, quarter = lane & 3;
  float s[GW][2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      const float dot = quad_sum(qk_partial<CT, D, GW>(r.k[sb], q[h]));
      s[h][sb] = r.kok[sb] ? dot * logit_scale : -INFINITY;
    }
  }
  float alpha[GW];
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    const float cm = max_across_quads(fmaxf(s[h][0], s[h][1]));
    const float mn = fmaxf(st.m[h], cm);
    alpha[h] = fast_exp2(st.m[h] - mn);
    st.m[h] = mn;
    const float p0 = fast_exp2(s[h][0] - mn);
    const float p1 = fast_exp2(s[h][1] - mn);
    st.l[h] = st.l[h] * alpha[h] + p0 + p1;
    // lane (key, quarter) publishes heads h == quarter (mod 4)
    if ((h & 3) == quarter) {
      p_lds[kq * GW + h] = p0;
      p_lds[(16 + kq) * GW + h] = p1;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
  for (int h = 0; h < GW; ++h)
#pragma unroll
    for (int e = 0; e < C::pv_nv; ++e) st.o[h][e] *= alpha[h];

  const int kp = lane / C::pv_lanes;
#pragma unroll
  for (int i = 0; i < C::pv_loads; ++i) {
    const int key = i * C::pv_kp + kp;
    float vv[C::pv_nv];
    v_values<CT, D, GW>(r.v[i], vv);
    float p[GW];
    if constexpr (GW % 4 == 0) {
#pragma unroll
      for (int h4 = 0; h4 < GW; h4 += 4) {
        const float4 pp = *reinterpret_cast<const float4*>(p_lds + key * GW + h4);
        p[h4] = pp.x;
        p[h4 + 1] = pp.y;
        p[h4 + 2] = pp.z;
        p[h4 + 3] = pp.w;
      }
    } else {
#pragma unroll
      for (int h = 0; h < GW; ++h) p[h] = p_lds[key * GW + h];
    }
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
      for (int e = 0; e < C::pv_nv; ++e) st.o[h][e] = fmaf(p[h], vv[e], st.o[h][e]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int QT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (QT == kF32) {
    reinterpret_cast<float*>(out)[idx] = x;
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits(x);
  }
}

template <int CT, int D, int GW>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a, int split_keys, int num_splits,
                                                     int head_groups) {
  using C = Cfg<CT, D, GW>;
  constexpr int QT = (CT == kF32) ? kF32 : kBF16;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x;
  const int g = blockIdx.y / head_groups;
  const int h0 = g * (a.num_heads / a.num_kv_heads) + (blockIdx.y % head_groups) * GW;
  const int b = blockIdx.z;

  __shared__ int32_t tbl[kDecodeMaxSplitKeys / 8 + 2];
  __shared__ float p_lds[kWaves][kChunk * GW];
  __shared__ float red_o[kWaves][GW][D];
  __shared__ float red_m[kWaves][GW];
  __shared__ float red_l[kWaves][GW];

  const int log2bs = __builtin_ctz(a.block_size);
  int lk = a.cache_seqlens[b];
  const int cap = a.max_blocks_per_seq * a.block_size;
  lk = lk < 0 ? 0 : (lk > cap ? cap : lk);
  const int start = split * split_keys;
  if (split > 0 && start >= lk) return;  // nothing to do for this split
  const int end = min(lk, start + split_keys);
  const int nsplit_seq = lk > 0 ? (lk + split_keys - 1) / split_keys : 1;
  const bool final_out = nsplit_seq == 1;

  // the split's block ids, validated against the pool size
  const int blk0 = start >> log2bs;
  const int nblk = end > start ? ((end - 1) >> log2bs) - blk0 + 1 : 0;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) {
    const int id = a.block_table[(int64_t)b * a.max_blocks_per_seq + blk0 + i];
    tbl[i] = (id >= 0 && id < a.num_blocks) ? id : -1;
  }

  // this wave's q words
  uint32_t q[GW][C::q_words];
  {
    const int quarter = lane & 3;
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                            ((int64_t)b * a.num_heads + h0 + h) * D * Elt<QT>::bytes;
#pragma unroll
      for (int i = 0; i < C::qk_loads; ++i) {
        // this lane's elements of load i: [(i*64 + quarter*16)/elt, +16/elt)
        const int e0 = (i * 64 + quarter * 16) / C::elt;
        if constexpr (CT == kFP8) {
          const uint4 lo = *reinterpret_cast<const uint4*>(qrow + e0 * 2);
          const uint4 hi = *reinterpret_cast<const uint4*>(qrow + e0 * 2 + 16);
          q[h][i * 8 + 0] = lo.x; q[h][i * 8 + 1] = lo.y; q[h][i * 8 + 2] = lo.z; q[h][i * 8 + 3] = lo.w;
          q[h][i * 8 + 4] = hi.x; q[h][i * 8 + 5] = hi.y; q[h][i * 8 + 6] = hi.z; q[h][i * 8 + 7] = hi.w;
        } else {
          const uint4 x = *reinterpret_cast<const uint4*>(qrow + e0 * Elt<QT>::bytes);
          q[h][i * 4 + 0] = x.x; q[h][i * 4 + 1] = x.y; q[h][i * 4 + 2] = x.z; q[h][i * 4 + 3] = x.w;
        }
      }
    }
  }
  float logit_scale = a.softmax_scale * kLog2e;
  float out_scale = 1.0f;
  if constexpr (CT == kFP8) {
    logit_scale *= a.k_scale[g];
    out_scale = a.v_scale[g];
  }
  __syncthreads();

  SeqCtx sc;
  const int64_t row_bytes = C::row_bytes;
  sc.kbase = a.k_cache + g * row_bytes;
  sc.vbase = a.v_cache + g * row_bytes;
  sc.slot_stride = (int64_t)a.num_kv_heads * row_bytes;
  sc.tbl = tbl;
  sc.blk0 = blk0;
  sc.log2bs = log2bs;
  sc.bs_mask = a.block_size - 1;
  sc.lk = end;

  WaveState<CT, D, GW> st;
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    st.m[h] = kNegBig;
    st.l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < C::pv_nv; ++e) st.o[h][e] = 0.0f;
  }

  float* my_p = p_lds[wave];
  const int stride = kWaves * kChunk;
  int c = start + wave * kChunk;
  if (c < end) {
    ChunkRegs<CT, D, GW> A, B;
    load_chunk<CT, D, GW>(A, sc, c, lane);
    while (true) {
      const bool more = c + stride < end;
      if (more) load_chunk<CT, D, GW>(B, sc, c + stride, lane);
      compute_chunk<CT, D, GW>(st, A, q, logit_scale, lane, my_p);
      if (!more) break;
      c += stride;
      const bool more2 = c + stride < end;
      if (more2) load_chunk<CT, D, GW>(A, sc, c + stride, lane);
      compute_chunk<CT, D, GW>(st, B, q, logit_scale, lane, my_p);
      if (!more2) break;
      c += stride;
    }
  }

  // wave totals: l over the 16 key positions, o over the pv_kp key groups
  const int kp = lane / C::pv_lanes;
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    st.l[h] = sum_across_quads(st.l[h]);
#pragma unroll
    for (int e = 0; e < C::pv_nv; ++e) {
#pragma unroll
      for (int x = C::pv_lanes; x < 64; x <<= 1) st.o[h][e] += shfl_xor(st.o[h][e], x);
    }
  }
  if (kp == 0) {
    const int d0 = (lane % C::pv_lanes) * C::pv_nv;
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
      for (int e = 0; e < C::pv_nv; ++e) red_o[wave][h][d0 + e] = st.o[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      red_m[wave][h] = st.m[h];
      red_l[wave][h] = st.l[h];
    }
  }
  __syncthreads();

  // merge the four waves; write the final row or this split's partial triple
  const int hq = a.num_heads;
  for (int idx = threadIdx.x; idx < GW * D; idx += blockDim.x) {
    const int h = idx / D, d = idx % D;
    float mx = red_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, red_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(red_m[w][h] - mx);
      L = fmaf(red_l[w][h], f, L);
      O = fmaf(red_o[w][h][d], f, O);
    }
    const int64_t bh = (int64_t)b * hq + h0 + h;
    if (final_out) {
      const float val = L > 0.0f ? O / L * out_scale : 0.0f;
      store_out<QT>(a.out, bh * D + d, val);
    } else {
      float* ws_o = a.workspace;
      ws_o[(bh * num_splits + split) * D + d] = O * out_scale;
      if (d == 0) {
        float* ws_ml = a.workspace + (int64_t)a.batch * hq * num_splits * D;
        ws_ml[(bh * num_splits + split) * 2 + 0] = mx;
        ws_ml[(bh * num_splits + split) * 2 + 1] = L;
      }
    }
  }
}

// Merge the split partials of every (sequence, q head) with more than one split.
template <int QT, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int split_keys, int num_splits) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * kWaves + wave;
  const int hq = a.num_heads;
  if (bh >= (int64_t)a.batch * hq) return;
  const int b = (int)(bh / hq);
  int lk = a.cache_seqlens[b];
  const int cap = a.max_blocks_per_seq * a.block_size;
  lk = lk < 0 ? 0 : (lk > cap ? cap : lk);
  const int ns = (lk + split_keys - 1) / split_keys;
  if (ns <= 1) return;  // the decode kernel wrote this row already
  const float* ws_o = a.workspace + bh * num_splits * D;
  const float* ws_ml = a.workspace + (int64_t)a.batch * hq * num_splits * D + bh * num_splits * 2;
  float mx = kNegBig;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, ws_ml[2 * s]);
  for (int x = 1; x < 64; x <<= 1) mx = fmaxf(mx, shfl_xor(mx, x));
  constexpr int NV = D / 64;
  float O[NV] = {};
  float L = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float f = fast_exp2(ws_ml[2 * s] - mx);
    L = fmaf(ws_ml[2 * s + 1], f, L);
#pragma unroll
    for (int e = 0; e < NV; ++e) O[e] = fmaf(ws_o[s * D + lane * NV + e], f, O[e]);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int e = 0; e < NV; ++e) store_out<QT>(a.out, bh * D + lane * NV + e, O[e] * inv);
}

template <int CT, int D, int GW>
hipError_t launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  constexpr int QT = (CT == kF32) ? kF32 : kBF16;
  const dim3 grid(p.num_splits, a.num_kv_heads * p.head_groups, a.batch);
  hipLaunchKernelGGL((decode_kernel<CT, D, GW>), grid, dim3(256), 0, stream, a, p.split_keys,
                     p.num_splits, p.head_groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits == 1) return e;
  const int64_t rows = (int64_t)a.batch * a.num_heads;
  hipLaunchKernelGGL((merge_kernel<QT, D>), dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(256),
                     0, stream, a, p.split_keys, p.num_splits);
  return hipGetLastError();
}

template <int CT, int D>
hipError_t launch_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  const int gw = (a.num_heads / a.num_kv_heads) / p.head_groups;
  switch (gw) {
    case 1: return launch_t<CT, D, 1>(a, p, stream);
    case 2: return launch_t<CT, D, 2>(a, p, stream);
    case 4: return launch_t<CT, D, 4>(a, p, stream);
    case 8: return launch_t<CT, D, 8>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int CT>
hipError_t launch_c(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (a.head_dim == 64) return launch_d<CT, 64>(a, p, stream);
  if (a.head_dim == 128) return launch_d<CT, 128>(a, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (a.cache_dtype == kF32) return launch_c<kF32>(a, p, stream);
  if (a.cache_dtype == kBF16) return launch_c<kBF16>(a, p, stream);
  if (a.cache_dtype == kFP8) return launch_c<kFP8>(a, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
