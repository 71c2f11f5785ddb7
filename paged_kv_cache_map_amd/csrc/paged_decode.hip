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
// * Addressing is scalar: a 16-key sub-step lies in one cache block, so the
//   block's base address is formed once in SGPRs from the block table (staged
//   in LDS) and each lane adds a fixed offset.  Masking is confined to the one
//   chunk that crosses the end of the split.
// * Loads of the next chunk are issued before the current chunk is computed
//   (two register buffers), keeping 2 x 16 KiB per wave in flight.
// * fp8 caches are dequantised in registers (exact E4M3 -> bf16); the K scale
//   folds into the logit scale and the V scale into the output.

#include "pkv_device.hpp"
#include "pkv_internal.h"

#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 2
#endif
#ifndef PKV_DECODE_DEPTH_FP8
#define PKV_DECODE_DEPTH_FP8 2
#endif
#ifndef PKV_DECODE_OCC
#define PKV_DECODE_OCC 1
#endif
#ifndef PKV_DECODE_OCC_FP8
#define PKV_DECODE_OCC_FP8 2
#endif

namespace pkv {
namespace {

constexpr int kWaves = kDecodeWaves;
constexpr int kChunk = kDecodeChunk;  // keys per wave iteration (2 sub-steps of 16)

template <int CT, int D, int GW>
struct Cfg {
  static constexpr int elt = Elt<CT>::bytes;
  static constexpr int row_bytes = D * elt;        // one KV head's row of one slot
  // Q.K layout: lane = 4 * key + quarter, 16 keys per sub-step
  static constexpr int qk_loads = row_bytes / 64;  // 16-byte loads per lane per key
  static constexpr int qk_elems = D / 4;
  // q words per head: bf16 pairs (bf16/fp8 caches) or fp32 values (fp32 cache)
  static constexpr int q_words = (CT == kF32) ? qk_elems : qk_elems / 2;
  // P.V layout: lane = (key kp, slice of head_dim); pv_vec bytes per lane per key
  static constexpr int pv_vec = (row_bytes / 64 > 4) ? row_bytes / 64 : 4;
  static constexpr int pv_lanes = row_bytes / pv_vec;  // lanes per key row
  static constexpr int pv_kp = 64 / pv_lanes;          // keys per load instruction
  static constexpr int pv_nv = pv_vec / elt;           // elements per lane
  static constexpr int pv_loads = kChunk / pv_kp;      // load instructions per chunk
  static_assert(qk_loads >= 1 && pv_kp >= 1 && pv_kp <= 8, "shape");
};

// Registers holding one chunk's K (Q.K layout) and V (P.V layout).
template <int CT, int D, int GW>
struct ChunkRegs {
  using C = Cfg<CT, D, GW>;
  uint4 k[2][C::qk_loads];
  uint32_t v[C::pv_loads][C::pv_vec / 4];
  uint32_t kmask;  // uniform: bit k set iff key start + k exists and sits in a valid block
};

struct SeqCtx {
  const uint8_t* kbase;  // cache + g * row_bytes
  const uint8_t* vbase;
  int64_t block_bytes;   // block_size slots
  int slot_stride;       // bytes between slots = num_kv_heads * row_bytes
  const int32_t* tbl;    // LDS: block ids of the split (-1 = invalid), first = block blk0
  int blk0, log2bs, bs, end;
  uint32_t k_off;        // this lane's byte offset from its 8-key row group (Q.K)
  uint32_t v_off;        // this lane's byte offset from the instruction's first key (P.V)
};

constexpr int kBufferWord3 = 0x00020000;  // gfx9 raw buffer descriptor, dword 3

// Uniform byte offset of `key` (a uniform key) from the cache base; keys at or
// past the end and keys of invalid blocks map to slot 0 of block 0 (always
// present) and report valid = false.
__device__ __forceinline__ int64_t key_offset(const SeqCtx& s, int key, bool& valid) {
  const bool in_range = key < s.end;
  int blk = __builtin_amdgcn_readfirstlane(s.tbl[in_range ? (key >> s.log2bs) - s.blk0 : 0]);
  valid = in_range && blk >= 0;
  return valid ? (int64_t)blk * s.block_bytes + (int64_t)(key & (s.bs - 1)) * s.slot_stride : 0;
}

// Buffer resource over 8 consecutive slots starting at base + off.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows8(const uint8_t* base, int64_t off, int stride) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), 0, 8 * stride, kBufferWord3);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// A chunk's keys come as two 16-key sub-steps, each made of two 8-key row
// groups that lie in one block (block_size >= 8).  A row group is addressed by
// one buffer resource in SGPRs; every lane adds a fixed offset, so the loads
// need no per-key address arithmetic.  off[sb][0/1]: uniform byte offsets of
// the two row groups of sub-step sb (for block_size >= 16 the second is the
// first plus 8 slots).
template <int CT, int D, int GW, bool SMALL>
__device__ __forceinline__ void issue_chunk_loads(ChunkRegs<CT, D, GW>& r, const uint8_t* kbase,
                                                  const uint8_t* vbase, int stride, uint32_t k_off,
                                                  uint32_t v_off, const int64_t (&off)[2][2],
                                                  int lane) {
  using C = Cfg<CT, D, GW>;
  const bool hi_lane = (lane >> 2) >= 8;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    if constexpr (!SMALL) {
      // block_size >= 16: the sub-step's 16 rows are one run of one block
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(kbase + off[sb][0]), 0, 16 * stride, kBufferWord3);
#pragma unroll
      for (int i = 0; i < C::qk_loads; ++i) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
            kr, (int)(k_off + (hi_lane ? 8 * stride : 0)), i * 64, 0);
        r.k[sb][i] = make_uint4(x.x, x.y, x.z, x.w);
      }
    } else {
      // block_size 8: keys 0..7 and 8..15 sit in two blocks; both loads are
      // issued for every lane (lanes that share an address merge) and each
      // lane keeps its own
      const __amdgpu_buffer_rsrc_t ka = rows8(kbase, off[sb][0], stride);
      const __amdgpu_buffer_rsrc_t kb = rows8(kbase, off[sb][1], stride);
#pragma unroll
      for (int i = 0; i < C::qk_loads; ++i) {
        const u32x4_t xa = __builtin_amdgcn_raw_buffer_load_b128(ka, (int)k_off, i * 64, 0);
        const u32x4_t xb = __builtin_amdgcn_raw_buffer_load_b128(kb, (int)k_off, i * 64, 0);
        const u32x4_t x = hi_lane ? xb : xa;
        r.k[sb][i] = make_uint4(x.x, x.y, x.z, x.w);
      }
    }
    const __amdgpu_buffer_rsrc_t va_r = rows8(vbase, off[sb][0], stride);
    const __amdgpu_buffer_rsrc_t vb_r = rows8(vbase, off[sb][1], stride);
#pragma unroll
    for (int j = 0; j < 16 / C::pv_kp; ++j) {
      const int x = j * C::pv_kp;  // first key of the instruction within the sub-step
      const int soff = (x & 7) * stride;
      const int i = sb * (16 / C::pv_kp) + j;
      if constexpr (C::pv_vec == 4) {
        r.v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(x < 8 ? va_r : vb_r, (int)v_off, soff, 0);
      } else {
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(x < 8 ? va_r : vb_r, (int)v_off, soff, 0);
        r.v[i][0] = w.x;
        r.v[i][1] = w.y;
      }
    }
  }
}

// Validity mask of a chunk from its row groups' validity and the key count.
__device__ __forceinline__ uint32_t chunk_mask(const bool (&valid)[2][2], int keys_left) {
  uint32_t m = 0;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    m |= (valid[sb][0] ? 0xffu : 0u) << (16 * sb);
    m |= (valid[sb][1] ? 0xffu : 0u) << (16 * sb + 8);
  }
  return keys_left >= kChunk ? m : (keys_left <= 0 ? 0u : m & ((1u << keys_left) - 1u));
}

template <int CT, int D, int GW, bool SMALL>
__device__ __forceinline__ void load_chunk(ChunkRegs<CT, D, GW>& r, const SeqCtx& s, int start,
                                           int lane) {
  int64_t off[2][2];
  bool valid[2][2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int key0 = start + sb * 16;
    off[sb][0] = key_offset(s, key0, valid[sb][0]);
    if constexpr (!SMALL) {
      off[sb][1] = off[sb][0] + 8 * (int64_t)s.slot_stride;
      valid[sb][1] = valid[sb][0];
    } else {
      off[sb][1] = key_offset(s, key0 + 8, valid[sb][1]);
    }
  }
  issue_chunk_loads<CT, D, GW, SMALL>(r, s.kbase, s.vbase, s.slot_stride, s.k_off, s.v_off, off, lane);
  r.kmask = chunk_mask(valid, s.end - start);
}

// Partial dot product of one key's quarter row with head h's q (in LDS,
// q_h = that head's row; the four quarters of a quad read four 16-byte pieces).
template <int CT, int D, int GW>
__device__ __forceinline__ float qk_partial(const uint4 (&k)[Cfg<CT, D, GW>::qk_loads],
                                            const uint8_t* q_h, int quarter) {
  using C = Cfg<CT, D, GW>;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < C::qk_loads; ++i) {
    const uint32_t kw[4] = {k[i].x, k[i].y, k[i].z, k[i].w};
    if constexpr (CT == kBF16) {
      const uint4 qv = *reinterpret_cast<const uint4*>(q_h + i * 64 + quarter * 16);
      const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = dot2_bf16(qw[j], kw[j], acc);
    } else if constexpr (scaled8(CT)) {
      const uint4 q0 = *reinterpret_cast<const uint4*>(q_h + (i * 64 + quarter * 16) * 2);
      const uint4 q1 = *reinterpret_cast<const uint4*>(q_h + (i * 64 + quarter * 16) * 2 + 16);
      const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = dot2_bf16(qw[2 * j], code8x2_to_bf16x2<CT, false>(kw[j]), acc);
        acc = dot2_bf16(qw[2 * j + 1], code8x2_to_bf16x2<CT, true>(kw[j]), acc);
      }
    } else {
      const uint4 qv = *reinterpret_cast<const uint4*>(q_h + i * 64 + quarter * 16);
      const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(__uint_as_float(qw[j]), __uint_as_float(kw[j]), acc);
    }
  }
  return acc;
}

// The pv_nv fp32 values of one lane's V slice of one key.
template <int CT, int D, int GW>
__device__ __forceinline__ void v_values(const uint32_t* w, float* out) {
  using C = Cfg<CT, D, GW>;
  if constexpr (CT == kBF16) {
#pragma unroll
    for (int j = 0; j < C::pv_vec / 4; ++j) {
      out[2 * j] = bf16_lo(w[j]);
      out[2 * j + 1] = bf16_hi(w[j]);
    }
  } else if constexpr (scaled8(CT)) {
#pragma unroll
    for (int j = 0; j < C::pv_vec / 4; ++j) {
      const float2_t a = code8x2_to_f32x2<CT, false>(w[j]);
      const float2_t b = code8x2_to_f32x2<CT, true>(w[j]);
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

// Bytes of one q row as the kernel consumes it.
template <int CT, int D>
constexpr int kQRowBytes = D * (CT == kF32 ? 4 : 2);

template <int CT, int D, int GW>
struct WaveState {
  using C = Cfg<CT, D, GW>;
  float m[GW];               // running max (log2 domain), uniform across the wave
  float l[GW];               // per-lane partial sums of p (replicated within a quad)
  float o[GW][C::pv_nv];     // per-lane partial outputs (keys == kp mod pv_kp)
};

// One chunk of 32 keys.  MASKED: some key is past the end or in an invalid
// block (only the last chunk of a split, or a corrupt table).
template <int CT, int D, int GW, bool MASKED>
__device__ __forceinline__ void compute_chunk(WaveState<CT, D, GW>& st, const ChunkRegs<CT, D, GW>& r,
                                              const uint8_t* q_lds, float logit_scale, int start,
                                              const SeqCtx& sc, int lane, float* p_lds) {
  using C = Cfg<CT, D, GW>;
  const int kq = lane >> 2, quarter = lane & 3;
  float s[GW][2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    bool ok = true;
    if constexpr (MASKED) ok = (r.kmask >> (sb * 16 + kq)) & 1u;
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      const float dot = quad_sum(qk_partial<CT, D, GW>(r.k[sb], q_lds + h * kQRowBytes<CT, D>, quarter));
      s[h][sb] = ok ? dot * logit_scale : -INFINITY;
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
    uint32_t vw[C::pv_vec / 4];
#pragma unroll
    for (int w = 0; w < C::pv_vec / 4; ++w) vw[w] = r.v[i][w];
    if constexpr (MASKED) {
      const bool ok = (r.kmask >> key) & 1u;
#pragma unroll
      for (int w = 0; w < C::pv_vec / 4; ++w) vw[w] = ok ? vw[w] : 0u;
    }
    float vv[C::pv_nv];
    v_values<CT, D, GW>(vw, vv);
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
    // keep the scheduler from hoisting every key's p broadcast (GW registers
    // per key) to the top of the loop
    if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int CT, int D, int GW>
__device__ __forceinline__ void compute_any(WaveState<CT, D, GW>& st, const ChunkRegs<CT, D, GW>& r,
                                            const uint8_t* q_lds, float logit_scale, int start,
                                            const SeqCtx& sc, int lane, float* p_lds) {
  if (r.kmask == 0xffffffffu) {
    compute_chunk<CT, D, GW, false>(st, r, q_lds, logit_scale, start, sc, lane, p_lds);
  } else {
    compute_chunk<CT, D, GW, true>(st, r, q_lds, logit_scale, start, sc, lane, p_lds);
  }
}

template <int QT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (QT == kF32) {
    reinterpret_cast<float*>(out)[idx] = x;
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits(x);
  }
}

template <int CT, int D, int GW, bool SMALL>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a, int split_keys, int num_splits,
                                                     int head_groups) {
  using C = Cfg<CT, D, GW>;
  constexpr int QT = (CT == kF32) ? kF32 : kBF16;
  // wave index in a scalar register: the chunk loop is then uniform per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // x = KV head (group): the heads of one (sequence, split) are dispatched
  // together, so they read their slices of the same slot rows at the same time
  const int split = blockIdx.y;
  const int g = blockIdx.x / head_groups;
  const int h0 = g * (a.num_heads / a.num_kv_heads) + (blockIdx.x % head_groups) * GW;
  const int b = blockIdx.z;

  __shared__ int32_t tbl[kDecodeMaxSplitKeys / 8 + 2];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[GW * kQRowBytes<CT, D>];
  __shared__ __attribute__((aligned(16))) float p_lds[kWaves][kChunk * GW];
  __shared__ float red_o[kWaves][GW][D];
  __shared__ float red_m[kWaves][GW];
  __shared__ float red_l[kWaves][GW];

  const int log2bs = __builtin_ctz(a.block_size);
  const int cap = a.max_blocks_per_seq * a.block_size;
  const int lk = clamp_keys(a.cache_seqlens[b], a.len_bias, cap);
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
  if (threadIdx.x == 0 && nblk == 0) tbl[0] = -1;

  // the group's q rows, staged once in LDS (q dtype: fp32 with an fp32 cache, else bf16)
  {
    constexpr int qrow = kQRowBytes<CT, D>;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.q) + ((int64_t)b * a.num_heads + h0) * qrow;
    for (int i = threadIdx.x; i < GW * qrow / 16; i += blockDim.x)
      reinterpret_cast<uint4*>(q_lds)[i] = reinterpret_cast<const uint4*>(src)[i];
  }
  float logit_scale = a.softmax_scale * kLog2e;
  float out_scale = 1.0f;
  if constexpr (scaled8(CT)) {
    logit_scale *= a.k_scale[g];
    out_scale = a.v_scale[g];
  }
  __syncthreads();

  SeqCtx sc;
  const int row_bytes = C::row_bytes;
  sc.kbase = a.k_cache + g * row_bytes;
  sc.vbase = a.v_cache + g * row_bytes;
  sc.slot_stride = a.num_kv_heads * row_bytes;
  sc.block_bytes = (int64_t)a.block_size * sc.slot_stride;
  sc.tbl = tbl;
  sc.blk0 = blk0;
  sc.log2bs = log2bs;
  sc.bs = a.block_size;
  sc.end = end;
  {
    const int kq = lane >> 2, quarter = lane & 3;
    sc.k_off = (uint32_t)((kq & 7) * sc.slot_stride + quarter * 16);  // within an 8-row group
    sc.v_off = (uint32_t)((lane / C::pv_lanes) * sc.slot_stride + (lane % C::pv_lanes) * C::pv_vec);
  }

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
    // Two register buffers; the next chunk's loads are always issued (past
    // the end they read a safe row and are masked), so every wait is exact.
    ChunkRegs<CT, D, GW> A, B;
    load_chunk<CT, D, GW, SMALL>(A, sc, c, lane);
    for (;;) {
      load_chunk<CT, D, GW, SMALL>(B, sc, c + stride, lane);
      compute_any<CT, D, GW>(st, A, q_lds, logit_scale, c, sc, lane, my_p);
      c += stride;
      if (c >= end) break;
      load_chunk<CT, D, GW, SMALL>(A, sc, c + stride, lane);
      compute_any<CT, D, GW>(st, B, q_lds, logit_scale, c, sc, lane, my_p);
      c += stride;
      if (c >= end) break;
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
  const int cap = a.max_blocks_per_seq * a.block_size;
  const int lk = clamp_keys(a.cache_seqlens[b], a.len_bias, cap);
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

// ---------------------------------------------------------------------------
// Stream-K decode: every wave is an independent worker that takes an equal,
// contiguous share of the whole step's work, counted in 32-key chunks over
// all (sequence, KV head group) units in order.  A wave keeps streaming
// across unit boundaries; where a unit is split between waves each wave
// writes a partial (max, sum, output) triple and the stream merge kernel
// combines them.  This balances variable lengths exactly, and no workgroup
// waits for a start-up or a tail of its own.
// ---------------------------------------------------------------------------

// Chunk counts: pre[b] = chunks of all units of sequences before b.
__device__ __forceinline__ void build_prefix(int32_t* pre, int32_t* part, const DecodeArgs& a,
                                             int units_per_seq) {
  const int B = a.batch;
  const int cap = a.max_blocks_per_seq * a.block_size;
  const int per = (B + kStreamThreads - 1) / kStreamThreads;
  const int b0 = threadIdx.x * per;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < B) {
      const int lk = clamp_keys(a.cache_seqlens[b], a.len_bias, cap);
      sum += ((lk + kChunk - 1) / kChunk) * units_per_seq;
    }
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  // inclusive scan of the per-thread sums (Hillis-Steele, 8 steps)
  for (int d = 1; d < kStreamThreads; d <<= 1) {
    const int x = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
    __syncthreads();
    part[threadIdx.x] += x;
    __syncthreads();
  }
  int run = part[threadIdx.x] - sum;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < B) {
      pre[b] = run;
      const int lk = clamp_keys(a.cache_seqlens[b], a.len_bias, cap);
      run += ((lk + kChunk - 1) / kChunk) * units_per_seq;
    }
  }
  if (threadIdx.x == kStreamThreads - 1) pre[B] = part[kStreamThreads - 1];
  __syncthreads();
}

// Wave that owns global chunk x when T chunks are dealt to W waves
// (wave w owns [floor(T w / W), floor(T (w+1) / W))).
__device__ __forceinline__ int wave_of(int64_t x, int64_t T, int W) {
  return (int)(((x + 1) * W - 1) / T);
}

struct Pos {
  int b, gg;    // sequence, unit (KV head group) within the sequence
  int ch, nch;  // chunk within the unit, chunks per unit of this sequence
  int len;      // keys of the sequence (kept by the matrix-core kernel only)
};

__device__ __forceinline__ Pos locate(const int32_t* pre, int B, int ug, int x) {
  int lo = 0, hi = B;  // largest b with pre[b] <= x (and a non-empty sequence)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= x) lo = mid; else hi = mid;
  }
  while (pre[lo + 1] <= x) ++lo;  // skip empty sequences
  Pos p;
  p.b = lo;
  p.nch = (pre[lo + 1] - pre[lo]) / ug;
  const int r = x - pre[lo];
  p.gg = r / p.nch;
  p.ch = r % p.nch;
  return p;
}

__device__ __forceinline__ Pos advance(const int32_t* pre, int ug, Pos p) {
  if (p.ch + 1 < p.nch) {
    ++p.ch;
  } else if (p.gg + 1 < ug) {
    ++p.gg;
    p.ch = 0;
  } else {
    do { ++p.b; } while (pre[p.b + 1] == pre[p.b]);  // callers stay inside [0, T)
    p.gg = 0;
    p.ch = 0;
    p.nch = (pre[p.b + 1] - pre[p.b]) / ug;
  }
  return p;
}

struct StreamCtx {
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* seqlens;
  int64_t block_bytes;
  int slot_stride, row_bytes, max_blocks, num_blocks, log2bs, bs, cap, heads_per_kv, head_groups;
  int len_bias;  // added to cache_seqlens (1 when the call appends the step's token)
  uint32_t k_off, v_off;
};

__device__ __forceinline__ int seq_len(const StreamCtx& c, int b) {
  return clamp_keys(c.seqlens[b], c.len_bias, c.cap);
}

// Block ids of the four 8-key row groups of chunk p (lane j holds group j & 3).
__device__ __forceinline__ int fetch_table(const StreamCtx& c, const Pos& p, int lane) {
  const int key = p.ch * kChunk + 8 * (lane & 3);
  const int idx = min(key >> c.log2bs, c.max_blocks - 1);
  return c.block_table[(int64_t)p.b * c.max_blocks + idx];
}

template <int CT, int D, int GW, bool SMALL>
__device__ __forceinline__ void load_chunk_stream(ChunkRegs<CT, D, GW>& r, const StreamCtx& c,
                                                  const Pos& p, int tbl, int lane) {
  const int lk = seq_len(c, p.b);
  const int start = p.ch * kChunk;
  const int g = (p.gg / c.head_groups);
  int64_t off[2][2];
  bool valid[2][2];
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const int key = start + 8 * grp;
    const int id = __builtin_amdgcn_readlane(tbl, grp);
    const bool ok = key < lk && id >= 0 && id < c.num_blocks;
    off[grp >> 1][grp & 1] =
        ok ? (int64_t)id * c.block_bytes + (int64_t)(key & (c.bs - 1)) * c.slot_stride : 0;
    valid[grp >> 1][grp & 1] = ok;
  }
  const uint8_t* kbase = c.k_cache + g * c.row_bytes;
  const uint8_t* vbase = c.v_cache + g * c.row_bytes;
  issue_chunk_loads<CT, D, GW, SMALL>(r, kbase, vbase, c.slot_stride, c.k_off, c.v_off, off, lane);
  r.kmask = chunk_mask(valid, lk - start);
}

// Copy the q rows of unit (b, gg) into this wave's LDS region.
template <int CT, int D, int GW>
__device__ __forceinline__ void load_q(uint8_t* q_w, const DecodeArgs& a, const StreamCtx& c,
                                       const Pos& p, int lane) {
  constexpr int qrow = kQRowBytes<CT, D>;
  const int h0 = (p.gg / c.head_groups) * c.heads_per_kv + (p.gg % c.head_groups) * GW;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.q) + ((int64_t)p.b * a.num_heads + h0) * qrow;
  for (int i = lane; i < GW * qrow / 16; i += 64)
    reinterpret_cast<uint4*>(q_w)[i] = reinterpret_cast<const uint4*>(src)[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workspace layout of the stream plan: partial outputs [slots][GW][D], then
// (max, sum) pairs [slots][GW][2], then the chunk prefix [batch + 1].
__device__ __forceinline__ int32_t* stream_prefix(const DecodeArgs& a, int gw, int d) {
  return reinterpret_cast<int32_t*>(a.workspace + a.stream_slots * gw * (int64_t)(d + 2));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += shfl_xor(x, m);
  return x;
}

// End of a wave's segment of a unit: the final rows if the wave processed the
// whole unit, else a partial triple in slot (wave + unit).
template <int CT, int D, int GW>
__device__ __forceinline__ void flush_segment(WaveState<CT, D, GW>& st, const DecodeArgs& a,
                                              const StreamCtx& c, const Pos& p, bool whole, int slot,
                                              float out_scale, int lane) {
  using C = Cfg<CT, D, GW>;
  constexpr int QT = (CT == kF32) ? kF32 : kBF16;
  const int kp = lane / C::pv_lanes;
  const int d0 = (lane % C::pv_lanes) * C::pv_nv;
  const int h0 = (p.gg / c.head_groups) * c.heads_per_kv + (p.gg % c.head_groups) * GW;
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    const float l = sum_across_quads(st.l[h]);
#pragma unroll
    for (int e = 0; e < C::pv_nv; ++e) {
#pragma unroll
      for (int x = C::pv_lanes; x < 64; x <<= 1) st.o[h][e] += shfl_xor(st.o[h][e], x);
    }
    if (whole) {
      if (kp == 0) {
        const float inv = l > 0.0f ? out_scale / l : 0.0f;
        const int64_t base = ((int64_t)p.b * a.num_heads + h0 + h) * D + d0;
#pragma unroll
        for (int e = 0; e < C::pv_nv; ++e) store_out<QT>(a.out, base + e, st.o[h][e] * inv);
      }
    } else {
      float* ws_o = a.workspace + ((int64_t)slot * GW + h) * D;
      float* ws_ml = a.workspace + (int64_t)a.stream_slots * GW * D + ((int64_t)slot * GW + h) * 2;
      if (kp == 0) {
#pragma unroll
        for (int e = 0; e < C::pv_nv; ++e) ws_o[d0 + e] = st.o[h][e] * out_scale;
      }
      if (lane == 0) {
        ws_ml[0] = st.m[h];
        ws_ml[1] = l;
      }
    }
    st.m[h] = kNegBig;
    st.l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < C::pv_nv; ++e) st.o[h][e] = 0.0f;
  }
}

template <int CT, int D, int GW, bool SMALL>
__global__ __launch_bounds__(kStreamThreads) void decode_stream_kernel(DecodeArgs a, int head_groups) {
  using C = Cfg<CT, D, GW>;
  constexpr int qrow = kQRowBytes<CT, D>;
  __shared__ int32_t pre[kStreamMaxBatch + 1];
  __shared__ int32_t part[kStreamThreads];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kWaves][GW * qrow];
  __shared__ __attribute__((aligned(16))) float p_lds[kWaves][kChunk * GW];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ug = a.num_kv_heads * head_groups;  // units per sequence
  build_prefix(pre, part, a, ug);
  if (blockIdx.x == 0) {  // the merge kernel reads the prefix instead of rebuilding it
    int32_t* pre_g = stream_prefix(a, GW, D);
    for (int i = threadIdx.x; i <= a.batch; i += kStreamThreads) pre_g[i] = pre[i];
  }
  const int64_t T = pre[a.batch];
  const int W = gridDim.x * kWaves;
  const int w = blockIdx.x * kWaves + wave;
  const int c0 = (int)(T * w / W), c1 = (int)(T * (w + 1) / W);
  if (c0 >= c1) return;

  StreamCtx c;
  c.k_cache = a.k_cache;
  c.v_cache = a.v_cache;
  c.block_table = a.block_table;
  c.seqlens = a.cache_seqlens;
  c.len_bias = a.len_bias;
  c.row_bytes = C::row_bytes;
  c.slot_stride = a.num_kv_heads * C::row_bytes;
  c.block_bytes = (int64_t)a.block_size * c.slot_stride;
  c.max_blocks = a.max_blocks_per_seq;
  c.num_blocks = a.num_blocks;
  c.log2bs = __builtin_ctz(a.block_size);
  c.bs = a.block_size;
  c.cap = a.max_blocks_per_seq * a.block_size;
  c.heads_per_kv = a.num_heads / a.num_kv_heads;
  c.head_groups = head_groups;
  {
    const int kq = lane >> 2, quarter = lane & 3;
    c.k_off = (uint32_t)((kq & 7) * c.slot_stride + quarter * 16);  // within an 8-row group
    c.v_off = (uint32_t)((lane / C::pv_lanes) * c.slot_stride + (lane % C::pv_lanes) * C::pv_vec);
  }
  const float base_scale = a.softmax_scale * kLog2e;

  uint8_t* q_w = q_lds[wave];
  float* p_w = p_lds[wave];
  WaveState<CT, D, GW> st;
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    st.m[h] = kNegBig;
    st.l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < C::pv_nv; ++e) st.o[h][e] = 0.0f;
  }

  // cur: chunk being computed; nxt: chunk whose loads are in flight
  Pos cur = locate(pre, a.batch, ug, c0);
  Pos nxt = c0 + 1 < c1 ? advance(pre, ug, cur) : cur;
  int tbl_nxt = fetch_table(c, nxt, lane);
  {
    const int tbl_cur = fetch_table(c, cur, lane);
    load_q<CT, D, GW>(q_w, a, c, cur, lane);
    int x = c0;
    ChunkRegs<CT, D, GW> A, B;
    load_chunk_stream<CT, D, GW, SMALL>(A, c, cur, tbl_cur, lane);
    float logit_scale = base_scale, out_scale = 1.0f;
    const int g_cur = cur.gg / head_groups;
    if constexpr (scaled8(CT)) {
      logit_scale *= a.k_scale[g_cur];
      out_scale = a.v_scale[g_cur];
    }
    // One step: compute `cur` from R (while S loads `nxt`), then move on.
    auto step = [&](ChunkRegs<CT, D, GW>& R, ChunkRegs<CT, D, GW>& S) -> bool {
      const Pos nn = x + 2 < c1 ? advance(pre, ug, nxt) : nxt;
      const int tbl_nn = fetch_table(c, nn, lane);
      load_chunk_stream<CT, D, GW, SMALL>(S, c, nxt, tbl_nxt, lane);
      compute_any<CT, D, GW>(st, R, q_w, logit_scale, cur.ch * kChunk, SeqCtx{}, lane, p_w);
      const bool last = x + 1 == c1;
      if (last || cur.ch + 1 == cur.nch) {
        const int u = cur.b * ug + cur.gg;
        const int64_t ustart = pre[cur.b] + (int64_t)cur.gg * cur.nch;
        const bool whole = ustart >= c0 && ustart + cur.nch <= c1;
        flush_segment<CT, D, GW>(st, a, c, cur, whole, w + u, out_scale, lane);
      }
      if (last) return false;
      if (nxt.b != cur.b || nxt.gg != cur.gg) {
        load_q<CT, D, GW>(q_w, a, c, nxt, lane);
        if constexpr (scaled8(CT)) {
          const int g = nxt.gg / head_groups;
          logit_scale = base_scale * a.k_scale[g];
          out_scale = a.v_scale[g];
        }
      }
      cur = nxt;
      nxt = nn;
      tbl_nxt = tbl_nn;
      ++x;
      return true;
    };
    for (;;) {
      if (!step(A, B)) break;
      if (!step(B, A)) break;
    }
  }
}

// Combine the partial triples of units split between waves and write zero
// rows for empty sequences.  One wave per (sequence, q head): one round trip
// for the prefix, one for every part's (max, sum) (a lane per part), then the
// parts' outputs, up to 32 in flight per lane:
//   out = sum_w o_w 2^(m_w - m) / sum_w l_w 2^(m_w - m),  m = max_w m_w.
// Units of at most KB parts (the common case) take one pass with all their
// parts' rows in flight at once.
template <int QT, int D, int GW, int KB>
__device__ __forceinline__ void merge_parts_once(const DecodeArgs& a, int64_t bh, int lane, int64_t T, int W,
                                                 int wf, int n, int u, int hh) {
  constexpr int NV = D / 64;
  const float* ws_o = a.workspace;
  const float* ws_ml = a.workspace + (int64_t)a.stream_slots * GW * D;
  const int wj = wf + min(lane, n - 1);
  const bool has = lane < n && (T * wj / W < T * (wj + 1) / W);
  const int64_t slot = (int64_t)(wj + u) * GW + hh;
  const float2 ml = *reinterpret_cast<const float2*>(ws_ml + slot * 2);  // (max, sum), one load
  const float m_raw = ml.x, l_raw = ml.y;
  float ov[KB][NV];
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    const int64_t si = (int64_t)(wf + min(i, n - 1) + u) * GW + hh;
#pragma unroll
    for (int e = 0; e < NV; ++e) ov[i][e] = ws_o[si * D + lane * NV + e];
  }
  const float mj = has ? m_raw : kNegBig;
  const float mn = wave_max(mj);
  const float f = has ? fast_exp2(mj - mn) : 0.0f;
  const float Ls = wave_sum(has ? l_raw * f : 0.0f);
  float Of[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) Of[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    const float fi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), i));
    const bool use = i < n && fi > 0.0f;
#pragma unroll
    for (int e = 0; e < NV; ++e) Of[e] = use ? fmaf(ov[i][e], fi, Of[e]) : Of[e];
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
#pragma unroll
  for (int e = 0; e < NV; ++e) store_out<QT>(a.out, bh * D + lane * NV + e, Of[e] * inv);
}

// The running combination of parts [jb, je) of a unit (wave-wide: a lane per
// part for the (max, sum) pairs, then the parts' rows kBatch at a time).
template <int D, int GW, int kBatch>
__device__ __forceinline__ void merge_range(const DecodeArgs& a, int lane, int64_t T, int W, int wf, int jb,
                                            int je, int u, int hh, float& mx, float& L, float (&O)[D / 64]) {
  constexpr int NV = D / 64;
  const float* ws_o = a.workspace;
  const float* ws_ml = a.workspace + (int64_t)a.stream_slots * GW * D;
  mx = kNegBig;
  L = 0.0f;
#pragma unroll
  for (int e = 0; e < NV; ++e) O[e] = 0.0f;
  for (int j0 = jb; j0 < je; j0 += 64) {
    // lane i: wave wf + j0 + i; waves that own no chunk at all wrote nothing
    const int j = min(j0 + lane, je - 1);
    const int wj = wf + j;
    const bool has = j0 + lane < je && (T * wj / W < T * (wj + 1) / W);
    const int64_t slot = (int64_t)(wj + u) * GW + hh;
    const float m_raw = ws_ml[slot * 2];
    const float l_raw = ws_ml[slot * 2 + 1];
    const float mj = has ? m_raw : kNegBig;
    const float mn = fmaxf(mx, wave_max(mj));
    const float alpha = fast_exp2(mx - mn);
    const float f = has ? fast_exp2(mj - mn) : 0.0f;
    L = L * alpha + wave_sum(has ? l_raw * f : 0.0f);
#pragma unroll
    for (int e = 0; e < NV; ++e) O[e] *= alpha;
    mx = mn;
    const int cnt = min(64, je - j0);
    for (int i0 = 0; i0 < cnt; i0 += kBatch) {
      float ov[kBatch][NV];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t si = (int64_t)(wf + j0 + min(i0 + i, cnt - 1) + u) * GW + hh;
#pragma unroll
        for (int e = 0; e < NV; ++e) ov[i][e] = ws_o[si * D + lane * NV + e];
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        // f is 0 for lanes past cnt and for waves without a part: skip those rows
        const float fi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), min(i0 + i, 63)));
        const bool use = i0 + i < cnt && fi > 0.0f;
#pragma unroll
        for (int e = 0; e < NV; ++e) O[e] = use ? fmaf(ov[i][e], fi, O[e]) : O[e];
      }
    }
  }
}

// MODE 0: one wave per (sequence, q head) row, parts eight at a time (few
// parts per unit; the fewest registers, for the most rows in flight).
// MODE 1: the same with up to 32 parts in flight.  MODE 2 (units split into
// many parts, few rows): one workgroup per row, its four waves taking a
// quarter of the parts each and combining their results through LDS in a
// fixed order.
template <int QT, int D, int GW, int MODE>
__global__ __launch_bounds__(kStreamThreads) void stream_merge_kernel(DecodeArgs a, int head_groups, int W) {
  constexpr int NV = D / 64;
  constexpr bool wide = MODE == 2;
  constexpr int kB = MODE == 0 ? 8 : 32;
  __shared__ float sm_ml[wide ? kWaves : 1][2];
  __shared__ float sm_o[wide ? kWaves : 1][wide ? D : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // (in the wide form every exit below is taken by the whole workgroup)
  const int64_t bh = wide ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * kWaves + wave;
  if (bh >= (int64_t)a.batch * a.num_heads) return;
  const bool writer = !wide || wave == 0;
  const int b = (int)(bh / a.num_heads), h = (int)(bh % a.num_heads);
  const int32_t* pre = stream_prefix(a, GW, D);
  const int64_t T = pre[a.batch];
  const int ug = a.num_kv_heads * head_groups;
  const int G = a.num_heads / a.num_kv_heads;
  const int gg = (h / G) * head_groups + (h % G) / GW;
  const int hh = (h % G) % GW;
  const int nch = (pre[b + 1] - pre[b]) / ug;
  // (T == 0 implies nch == 0; testing it keeps T's load next to the others)
  if (nch == 0 || T == 0) {
    if (writer) {
#pragma unroll
      for (int e = 0; e < NV; ++e) store_out<QT>(a.out, bh * D + lane * NV + e, 0.0f);
    }
    return;
  }
  const int64_t ustart = pre[b] + (int64_t)gg * nch;
  const int wf = wave_of(ustart, T, W), wl = wave_of(ustart + nch - 1, T, W);
  if (wf == wl) return;  // one wave processed the whole unit and wrote the row
  const int u = b * ug + gg;
  const int n = wl - wf + 1;
  if (n <= 8) {
    if (writer) merge_parts_once<QT, D, GW, 8>(a, bh, lane, T, W, wf, n, u, hh);
    return;
  }
  float mx, L, O[NV];
  if constexpr (!wide) {
    if (MODE == 1 && n <= 32) return merge_parts_once<QT, D, GW, 32>(a, bh, lane, T, W, wf, n, u, hh);
    merge_range<D, GW, kB>(a, lane, T, W, wf, 0, n, u, hh, mx, L, O);
  } else {
    merge_range<D, GW, kB>(a, lane, T, W, wf, n * wave / kWaves, n * (wave + 1) / kWaves, u, hh, mx, L, O);
    if (lane == 0) {
      sm_ml[wave][0] = mx;
      sm_ml[wave][1] = L;
    }
#pragma unroll
    for (int e = 0; e < NV; ++e) sm_o[wave][lane * NV + e] = O[e];
    __syncthreads();
    if (wave != 0) return;
    mx = fmaxf(fmaxf(sm_ml[0][0], sm_ml[1][0]), fmaxf(sm_ml[2][0], sm_ml[3][0]));
    L = 0.0f;
#pragma unroll
    for (int e = 0; e < NV; ++e) O[e] = 0.0f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      const float f = fast_exp2(sm_ml[q][0] - mx);
      L = fmaf(sm_ml[q][1], f, L);
#pragma unroll
      for (int e = 0; e < NV; ++e) O[e] = fmaf(sm_o[q][lane * NV + e], f, O[e]);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int e = 0; e < NV; ++e) store_out<QT>(a.out, bh * D + lane * NV + e, O[e] * inv);
}

// Launches the merge of a stream-K decode whose W waves covered `units`
// units, in the form for the parts per unit: at most 8 on average (MODE 0),
// at most 16 (MODE 1), more (MODE 2, a workgroup per row).
template <int QT, int D, int GW>
hipError_t launch_stream_merge(const DecodeArgs& a, int head_groups, int W, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.num_heads;
  const int64_t units = (int64_t)a.batch * a.num_kv_heads * head_groups;
  const dim3 narrow_grid((unsigned)((rows + kWaves - 1) / kWaves));
  if ((int64_t)W <= 8 * units)
    hipLaunchKernelGGL((stream_merge_kernel<QT, D, GW, 0>), narrow_grid, dim3(kStreamThreads), 0, stream, a,
                       head_groups, W);
  else if ((int64_t)W <= 16 * units)
    hipLaunchKernelGGL((stream_merge_kernel<QT, D, GW, 1>), narrow_grid, dim3(kStreamThreads), 0, stream, a,
                       head_groups, W);
  else
    hipLaunchKernelGGL((stream_merge_kernel<QT, D, GW, 2>), dim3((unsigned)rows), dim3(kStreamThreads), 0, stream,
                       a, head_groups, W);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Appending decode.  [paged-doc] section デコードパス (キャッシュの動作): the
// decode kernel indexes the paged cache through the block table and updates
// it in place; the worked example stores the new token of a sequence with
// cache_seqlens[b] cached keys at position cache_seqlens[b].  The append call
// takes the step's new K/V rows, stores each at that position (slot
// block_table[b][pos / bs] * bs + pos % bs) and attends cache_seqlens[b] + 1
// keys, so the write needs no launch of its own.
// ---------------------------------------------------------------------------

// One lane's share of the new K and V rows of KV head g of sequence b: lanes
// [0, P) move the 16-byte source pieces of K, lanes [P, 2 P) those of V (P
// pieces per head row, at most 32).  fetch_new issues the source load and
// the length load without waiting for either; store_new finds the slot and
// stores (nothing for idle lanes, or for a position past the block table or
// in an invalid block: bad metadata, memory-safe).
struct NewPiece {
  uint4 x;  // the lane's source bytes
  int b, g;
  int pos;  // cache_seqlens[b]: the new token's position
};

typedef const __attribute__((address_space(4))) int32_t* cptr_i32;
typedef const __attribute__((address_space(4))) float* cptr_f32;

template <int SRC, int D>
__device__ __forceinline__ NewPiece fetch_new(const DecodeArgs& a, int b, int g, int lane) {
  constexpr int src_row = D * Elt<SRC>::bytes;
  constexpr int P = src_row / 16;
  static_assert(2 * P <= 64, "one wave moves a head's K and V rows");
  const int l = lane < 2 * P ? lane : 2 * P - 1;
  const bool is_v = l >= P;
  const uint8_t* src = (is_v ? a.v_new + (int64_t)b * a.v_new_stride : a.k_new + (int64_t)b * a.k_new_stride) +
                       g * src_row + (is_v ? l - P : l) * 16;
  NewPiece n;
  n.x = *reinterpret_cast<const uint4*>(src);
  n.b = b;
  n.g = g;
  n.pos = ((cptr_i32)a.cache_seqlens)[b];  // metadata is not written while a kernel runs
  return n;
}

template <int SRC, int DST, int D>
__device__ __forceinline__ void store_new(const DecodeArgs& a, const NewPiece& n, int lane) {
  constexpr int src_row = D * Elt<SRC>::bytes;
  constexpr int dst_row = D * Elt<DST>::bytes;
  constexpr int P = src_row / 16;
  constexpr int dst_piece = 16 * Elt<DST>::bytes / Elt<SRC>::bytes;  // cache bytes per source piece
  const int cap = a.max_blocks_per_seq * a.block_size;
  if (n.pos < 0 || n.pos >= cap) return;
  const int blk = ((cptr_i32)a.block_table)[(int64_t)n.b * a.max_blocks_per_seq +
                                            (n.pos >> __builtin_ctz(a.block_size))];
  if (blk < 0 || blk >= a.num_blocks || lane >= 2 * P) return;
  const bool is_v = lane >= P;
  float sc = 1.0f;
  if constexpr (scaled8(DST)) sc = ((cptr_f32)(is_v ? a.v_scale : a.k_scale))[n.g];
  const int64_t slot = (int64_t)blk * a.block_size + (n.pos & (a.block_size - 1));
  // the caches are the caller's writable buffers (the decode kernels only read them)
  uint8_t* dst = const_cast<uint8_t*>(is_v ? a.v_cache : a.k_cache) + slot * ((int64_t)a.num_kv_heads * dst_row) +
                 n.g * dst_row + (is_v ? lane - P : lane) * dst_piece;
  const u32x4_t v = convert_piece<SRC, DST>(n.x, sc);
  if constexpr (dst_piece == 16) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(v.x, v.y, v.z, v.w);
  } else if constexpr (dst_piece == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = v.x;
  }
}

// Store the new K and V rows of KV head g of sequence b.
template <int SRC, int DST, int D>
__device__ __forceinline__ void append_head(const DecodeArgs& a, int b, int g, int lane) {
  store_new<SRC, DST, D>(a, fetch_new<SRC, D>(a, b, g, lane), lane);
}

// The append on its own (plans other than the matrix-core stream-K kernel):
// one wave per (sequence, KV head); the decode kernels run after it on the
// same stream.
template <int SRC, int DST, int D>
__global__ __launch_bounds__(256) void append_kernel(DecodeArgs a) {
  const int64_t w = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w >= (int64_t)a.batch * a.num_kv_heads) return;
  append_head<SRC, DST, D>(a, (int)(w / a.num_kv_heads), (int)(w % a.num_kv_heads), threadIdx.x & 63);
}

template <int SRC, int DST>
hipError_t launch_append_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.batch * a.num_kv_heads;
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
  if (a.head_dim == 64) hipLaunchKernelGGL((append_kernel<SRC, DST, 64>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((append_kernel<SRC, DST, 128>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_append(const DecodeArgs& a, hipStream_t stream) {
  if (a.q_dtype == kF32 && a.cache_dtype == kF32) return launch_append_t<kF32, kF32>(a, stream);
  if (a.q_dtype == kBF16 && a.cache_dtype == kBF16) return launch_append_t<kBF16, kBF16>(a, stream);
  if (a.q_dtype == kBF16 && a.cache_dtype == kFP8) return launch_append_t<kBF16, kFP8>(a, stream);
  if (a.q_dtype == kBF16 && a.cache_dtype == kI8) return launch_append_t<kBF16, kI8>(a, stream);
  return hipErrorInvalidValue;
}

// Workgroups of a persistent launch: every CU filled to the kernel's
// occupancy, and never more waves than the workspace has slots for.
template <typename K>
int persistent_grid(K kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kStreamThreads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    cus = 256;
    per_cu = 1;
  }
  int64_t wgs = (int64_t)cus * per_cu;
  if (wgs > kStreamMaxWaves / kWaves) wgs = kStreamMaxWaves / kWaves;
  return (int)(wgs < 1 ? 1 : wgs);
}

// ---------------------------------------------------------------------------
// Stream-K decode on the matrix cores (bf16 cache).
//
// The G q heads that share a KV head form a [G x D] by [D x keys] product, so
// a wave computes each 32-key chunk as S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_16x16x32_bf16 with the G heads as the 16 columns (q rows of
// absent heads are zero when G < 16).  The vector ALUs only run the softmax
// (8 exponentials per lane and chunk instead of 2 G), so the wave's time goes
// to waiting for HBM, as it should in a memory-bound kernel.
// * K reaches the A operand straight from HBM: lane l loads 16 bytes of key
//   l mod 16 at head_dim 32 ks + 8 (l / 16) (a 64-byte run per key).
// * V rows are copied to the wave's LDS region (row-major, 16-byte pieces
//   permuted by vswz) and read back with ds_read_b64_tr_b16, which hands each
//   lane four consecutive keys of one head_dim element: the A operand of V^T.
//   P^T comes straight from the lane's own S^T registers once the product's
//   key order is permuted to match (the same permutation on both operands
//   leaves the sum unchanged).
// * the stream-K schedule, partial triples and merge kernel are those of the
//   vector kernel; units are whole KV heads (no head groups).
// ---------------------------------------------------------------------------
namespace mfd {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8_t, x); }

// Geometry for cache type CT (bf16 or fp8) and head_dim D.  V always sits in
// LDS as bf16 rows; fp8 K and V are dequantised on the way (exactly).
template <int CT, int D>
struct Geo {
  static constexpr int elt = Elt<CT>::bytes;
  static constexpr int row_bytes = D * elt;           // cache row of one KV head
  static constexpr int lds_row = D * 2;               // bf16 V row in LDS
  static constexpr int KS = D / 32;                   // QK k-steps
  static constexpr int DB = D / 16;                   // 16-element blocks of head_dim
  static constexpr int pieces = row_bytes / 16;       // 16-byte pieces per cache row
  // V rows per load instruction: at most 8, so that an instruction stays in
  // one 8-key group (with fp8 and D = 64 half of the lanes then idle)
  static constexpr int vkeys = 64 / pieces < 8 ? 64 / pieces : 8;
  static constexpr int vlanes = vkeys * pieces;       // lanes that move V
  static constexpr int vloads = kChunk / vkeys;       // V load instructions per chunk
  static constexpr int vbytes = kChunk * lds_row;     // one chunk of K or V in LDS
  static constexpr int qrow = D * 2;                  // bf16 q row
};

// LDS piece permutation of V row r: keeps both the row writes and the
// transposed reads (16 consecutive rows x 2 pieces) free of bank conflicts.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? ((r & 7) << 1) : ((r & 3) << 1);
}

// LDS piece permutation of K row r: the A-operand reads (16 consecutive rows,
// one piece) and the row writes are free of bank conflicts.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : (r & 7);
}

__device__ __forceinline__ uint2 read_tr(const uint8_t* p) {
  const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
  return __builtin_bit_cast(uint2, x);
}

__device__ __forceinline__ float max_quarters(float x) {  // over lanes l, l^16, l^32, l^48
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_halves(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

__device__ __forceinline__ float sum_quarters(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return sum_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// Sixteen one-byte codes (E4M3 or int8) -> sixteen bf16 (exact), as two
// 8-element operands.
template <int CT>
__device__ __forceinline__ void code8x16_to_bf16(const uint4& x, uint4& lo, uint4& hi) {
  lo = make_uint4(code8x2_to_bf16x2<CT, false>(x.x), code8x2_to_bf16x2<CT, true>(x.x),
                  code8x2_to_bf16x2<CT, false>(x.y), code8x2_to_bf16x2<CT, true>(x.y));
  hi = make_uint4(code8x2_to_bf16x2<CT, false>(x.z), code8x2_to_bf16x2<CT, true>(x.z),
                  code8x2_to_bf16x2<CT, false>(x.w), code8x2_to_bf16x2<CT, true>(x.w));
}

// Values every lane of a wave needs (lengths, block-table entries, scales)
// are read with scalar loads through the constant address space: none of
// them is written while a kernel runs.  Scalar loads wait on their own
// counter (shared with LDS), so they never make a wave wait for the K and V
// loads in flight, as a vector load would (vector loads complete in order).
typedef const __attribute__((address_space(4))) int32_t* sptr_i32;
typedef const __attribute__((address_space(4))) float* sptr_f32;

__device__ __forceinline__ int seq_len_s(const StreamCtx& c, int b) {
  return clamp_keys(((sptr_i32)c.seqlens)[b], c.len_bias, c.cap);
}

// Block ids of the four 8-key groups of a chunk.
struct Tbl {
  int32_t e[4];
};

__device__ __forceinline__ Tbl fetch_tbl(const StreamCtx& c, const Pos& p) {
  const sptr_i32 row = (sptr_i32)c.block_table + (int64_t)p.b * c.max_blocks;
  Tbl t;
#pragma unroll
  for (int g = 0; g < 4; ++g) t.e[g] = row[min((p.ch * kChunk + 8 * g) >> c.log2bs, c.max_blocks - 1)];
  return t;
}

// One chunk in flight: its K and V registers (row pieces, as loaded), where
// its keys live, and its unit's scales.  K and V go through LDS (as bf16):
// every load instruction then reads whole 128-byte lines of a few rows, and
// the MFMA operands come from LDS reads.
template <int CT, int D>
struct Chunk {
  uint4 k[Geo<CT, D>::vloads];  // K: piece lane % pieces of row vkeys * i + lane / pieces
  uint4 v[Geo<CT, D>::vloads];  // V: the same pieces
  uint32_t kmask;               // bit k: key k of the chunk exists and sits in a valid block
  int64_t off[4];               // byte offsets of the chunk's four 8-key groups (uniform)
  float ls;                     // |softmax scale x K scale| x log2 e of the chunk's unit
  float vs;                     // V scale of the chunk's unit
  uint32_t qs;                  // sign flip applied to q (negative scale)
};

// Per-lane byte offsets: row lane / pieces of a load instruction (K and V),
// q row lane % 16 (past the unit's rows for absent heads, which read 0).
struct Offs {
  uint32_t row, q;
};

// Loads of chunk p's K and V rows.  Each 8-key group of the chunk lies in
// one block (block_size >= 8) and one load instruction covers at most 8 rows
// of one group, addressed through a buffer descriptor; keys past the end or
// in invalid blocks read row 0 of block 0 and are masked.
template <int CT, int D>
__device__ __forceinline__ void load_kv(Chunk<CT, D>& r, const StreamCtx& c, const Pos& p, const Tbl& tbl,
                                        const Offs& o) {
  using G = Geo<CT, D>;
  const int lk = p.len;
  const int start = p.ch * kChunk;
  uint32_t mask = 0;
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const int key = start + 8 * grp;
    const int id = tbl.e[grp];
    const bool ok = key < lk && id >= 0 && id < c.num_blocks;
    r.off[grp] = ok ? (int64_t)id * c.block_bytes + (int64_t)(key & (c.bs - 1)) * c.slot_stride : 0;
    const int n = min(max(lk - key, 0), 8);
    mask |= (ok ? ((1u << n) - 1u) : 0u) << (8 * grp);
  }
  r.kmask = mask;
  const uint8_t* kbase = c.k_cache + p.gg * c.row_bytes;
  const uint8_t* vbase = c.v_cache + p.gg * c.row_bytes;
#pragma unroll
  for (int i = 0; i < G::vloads; ++i) {
    const int row0 = G::vkeys * i;  // first key of the instruction (within one 8-key group)
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + r.off[row0 >> 3]), 0, 8 * c.slot_stride, kBufferWord3);
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)o.row, (row0 & 7) * c.slot_stride, 0);
    r.k[i] = make_uint4(x.x, x.y, x.z, x.w);
  }
#pragma unroll
  for (int i = 0; i < G::vloads; ++i) {
    const int row0 = G::vkeys * i;
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + r.off[row0 >> 3]), 0, 8 * c.slot_stride, kBufferWord3);
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)o.row, (row0 & 7) * c.slot_stride, 0);
    r.v[i] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

// q rows of unit p (G heads) as the B operand: head lane % 16 (zero for
// absent heads), 8 elements per k-step.
template <int CT, int D, int G>
__device__ __forceinline__ void load_q(uint4 (&q)[D / 32], const DecodeArgs& a, const Pos& p,
                                       const Offs& o) {
  using Ge = Geo<CT, D>;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.q) + ((int64_t)p.b * a.num_heads + p.gg * G) * Ge::qrow;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, G * Ge::qrow, kBufferWord3);
#pragma unroll
  for (int ks = 0; ks < Ge::KS; ++ks) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)o.q, 64 * ks, 0);
    q[ks] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

// The scales of unit p.
template <int CT, int D>
__device__ __forceinline__ void unit_scales(Chunk<CT, D>& r, const DecodeArgs& a, const Pos& p) {
  // The chunk max is taken over unscaled scores, which needs a scale > 0: a
  // negative scale is applied as |scale| to -q (bf16 negation is exact), a
  // zero scale as 1e-30 (every logit then rounds to 0 in the exponent, while
  // masked keys stay at -inf instead of -inf * 0).
  float sc = a.softmax_scale;
  r.vs = 1.0f;
  if constexpr (scaled8(CT)) {
    sc *= ((sptr_f32)a.k_scale)[p.gg];
    r.vs = ((sptr_f32)a.v_scale)[p.gg];
  }
  r.qs = sc < 0.0f ? 0x80008000u : 0u;
  r.ls = fmaxf(fabsf(sc) * kLog2e, 1e-30f);
}

// K and V rows of the chunk (registers) -> this wave's LDS regions as bf16.
// V rows of keys that do not exist are stored as zeros: their p is 0, but the
// cache may hold anything there (NaN included) and 0 * NaN would leak (their
// scores are masked, so K rows need no such care).
template <int CT, int D, int SW>
__device__ __forceinline__ void store_rows(const uint4& x, uint8_t* w, int row, int piece) {
  using G = Geo<CT, D>;
  const int sw = SW == 0 ? kswz<D>(row) : vswz<D>(row);
  if constexpr (scaled8(CT)) {
    uint4 lo, hi;
    code8x16_to_bf16<CT>(x, lo, hi);
    *reinterpret_cast<uint4*>(w + row * G::lds_row + (((2 * piece) ^ sw) << 4)) = lo;
    *reinterpret_cast<uint4*>(w + row * G::lds_row + (((2 * piece + 1) ^ sw) << 4)) = hi;
  } else {
    *reinterpret_cast<uint4*>(w + row * G::lds_row + ((piece ^ sw) << 4)) = x;
  }
}

template <int CT, int D>
__device__ __forceinline__ void store_kv(const Chunk<CT, D>& r, uint8_t* k_w, uint8_t* v_w, int lane) {
  using G = Geo<CT, D>;
  const bool full = r.kmask == 0xffffffffu;
  if (G::vlanes < 64 && lane >= G::vlanes) return;
  const int piece = lane % G::pieces;
#pragma unroll
  for (int i = 0; i < G::vloads; ++i) {
    const int row = G::vkeys * i + lane / G::pieces;
    const bool ok = full || ((r.kmask >> row) & 1u);
    store_rows<CT, D, 0>(r.k[i], k_w, row, piece);
    store_rows<CT, D, 1>(ok ? r.v[i] : make_uint4(0u, 0u, 0u, 0u), v_w, row, piece);
  }
}

template <int D>
struct MState {
  f32x4_t o[D / 16];  // O^T: rows 16 db + 4 (lane / 16) + i, column (head) lane % 16
  float m;            // running max of this lane's head (log2 domain)
  float l;            // this lane's share of the running sum
};

constexpr float kRescaleBits = 8.0f;  // lazy running max (log2 domain)

// S^T = K Q^T for the chunk (K in LDS, q in r): register i of block kb holds
// the score of key 16 kb + 4 (lane / 16) + i for head lane % 16.  k_off[ks]:
// this lane's A-operand piece (row lane % 16, elements 32 ks + 8 (lane / 16)).
template <int CT, int D>
__device__ __forceinline__ void chunk_scores(f32x4_t (&s)[2], const uint4 (&qf)[D / 32], uint32_t qs,
                                             const uint8_t* k_w, const uint32_t (&k_off)[D / 32]) {
  using G = Geo<CT, D>;
  s[0] = f32x4_t{};
  s[1] = f32x4_t{};
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const uint4 q = make_uint4(qf[ks].x ^ qs, qf[ks].y ^ qs, qf[ks].z ^ qs, qf[ks].w ^ qs);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 kf = *reinterpret_cast<const uint4*>(k_w + kb * 16 * G::lds_row + k_off[ks]);
      s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(q), s[kb], 0, 0, 0);
    }
  }
}

// Softmax update and O^T += V^T P^T for one chunk's scores (V in LDS).
template <int D>
__device__ __forceinline__ void chunk_update(MState<D>& st, f32x4_t (&s)[2], uint32_t kmask, const uint8_t* v_w,
                                             const uint32_t (&v_off)[D / 16], float logit_scale, int lane) {
  constexpr int DB = D / 16;
  const int g4 = 4 * (lane >> 4);
  if (kmask != 0xffffffffu) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kb][i] = ((kmask >> (16 * kb + g4 + i)) & 1u) ? s[kb][i] : -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  mx = max_quarters(mx) * logit_scale;
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kRescaleBits) != 0) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.o[db] *= alpha;
  }
  // P^T operand: k-slots 8 (lane / 16) + j hold keys 4 (lane / 16) + j (j < 4)
  // and 16 + 4 (lane / 16) + j - 4 (j >= 4): the lane's own scores
  f32x8_t pv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pv[i] = fast_exp2(fmaf(s[0][i], logit_scale, -st.m));
    pv[4 + i] = fast_exp2(fmaf(s[1][i], logit_scale, -st.m));
  }
  const uint4 pb = __builtin_bit_cast(uint4, __builtin_convertvector(pv, bf16x8_t));
  float ps = dot2_bf16(pb.x, 0x3f803f80u, 0.0f);
  ps = dot2_bf16(pb.y, 0x3f803f80u, ps);
  ps = dot2_bf16(pb.z, 0x3f803f80u, ps);
  ps = dot2_bf16(pb.w, 0x3f803f80u, ps);
  st.l += ps;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const uint2 lo = read_tr(v_w + v_off[db]);
    const uint2 hi = read_tr(v_w + v_off[db] + 16 * D * 2);
    st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                                      as_bf16x8(pb), st.o[db], 0, 0, 0);
  }
}

// End of a wave's segment of a unit: the final rows if the wave processed the
// whole unit, else a partial triple in slot (wave + unit).  Lanes l, l^16,
// l^32, l^48 hold head l % 16's 4 x DB output rows and shares of its sum.
template <int D, int G>
__device__ __forceinline__ void flush(MState<D>& st, const DecodeArgs& a, const Pos& p, bool whole, int slot,
                                      float out_scale, int lane) {
  constexpr int DB = D / 16;
  const int hc = lane & 15, g4 = 4 * (lane >> 4);
  const float l = sum_quarters(st.l);
  if (hc < G) {
    if (whole) {
      const float inv = l > 0.0f ? out_scale / l : 0.0f;
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)p.b * a.num_heads + p.gg * G + hc) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t w0 = pack_bf16x2(st.o[db][0] * inv, st.o[db][1] * inv);
        const uint32_t w1 = pack_bf16x2(st.o[db][2] * inv, st.o[db][3] * inv);
        *reinterpret_cast<uint2*>(out + 16 * db + g4) = make_uint2(w0, w1);
      }
    } else {
      float* ws_o = a.workspace + ((int64_t)slot * G + hc) * D;
      float* ws_ml = a.workspace + (int64_t)a.stream_slots * G * D + ((int64_t)slot * G + hc) * 2;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(ws_o + 16 * db + g4) =
            make_float4(st.o[db][0] * out_scale, st.o[db][1] * out_scale, st.o[db][2] * out_scale,
                        st.o[db][3] * out_scale);
      if (g4 == 0) {
        ws_ml[0] = st.m;
        ws_ml[1] = l;
      }
    }
  }
  st.m = kNegBig;
  st.l = 0.0f;
#pragma unroll
  for (int db = 0; db < DB; ++db) st.o[db] = f32x4_t{};
}

// N chunks in flight per wave, held in registers, OCC waves per SIMD (up to
// 512 / OCC registers per lane).
// The appending form (APPEND): the wave that owns the last chunk of a unit
// (the chunk holding key cache_seqlens[b], the new token) stores that unit's
// new K and V rows before it issues the load of that chunk.  A wave's memory
// operations reach the caches in issue order, so its own later load returns
// the stored rows; no other wave reads the rows of that KV head at that
// position.  The rows of the first unit that ends past the wave's first N
// chunks are fetched before those chunks' loads and stored after them, so
// waiting for them holds up nothing; units ending inside the first N chunks
// (before their loads) and the further ones are stored directly.

// First chunk >= lo that ends a unit, and that unit; -1 if none below hi.
// p0: the position of chunk c0.
__device__ __forceinline__ int first_unit_end(const int32_t* pre, int ug, const Pos& p0, int c0, int lo, int hi,
                                              Pos& p) {
  if (lo >= hi) return -1;
  p = p0;
  int x = c0 - p.ch + p.nch - 1;  // last chunk of p's unit
  while (x < lo) {
    if (x + 1 >= hi) return -1;
    p.ch = p.nch - 1;
    p = advance(pre, ug, p);  // the next unit with chunks (one exists: x + 1 < hi <= T)
    x += p.nch;
  }
  return x < hi ? x : -1;
}

// Store the rows of every unit whose last chunk lies in [lo, hi).
template <int CT, int D>
__device__ __forceinline__ void append_range(const DecodeArgs& a, const int32_t* pre, int ug, const Pos& p0, int c0,
                                             int lo, int hi, int lane) {
  Pos p;
  int x = first_unit_end(pre, ug, p0, c0, lo, hi, p);
  if (x < 0) return;
  for (;;) {
    append_head<kBF16, CT, D>(a, p.b, p.gg, lane);
    if (x + 1 >= hi) break;
    p.ch = p.nch - 1;
    p = advance(pre, ug, p);
    x += p.nch;
    if (x >= hi) break;
  }
}

// The workgroup body of the stream-K decode: workgroup wg of num_wgs, with
// its LDS passed in (the chunk prefix, the scan scratch and each wave's K and
// V chunk), so that a launch that serves other work too can run it.
template <int CT, int D, int G, int N, bool APPEND>
__device__ __forceinline__ void decode_mfma_body(const DecodeArgs& a, int wg, int num_wgs, int32_t* pre,
                                                 int32_t* part, uint8_t* k_lds, uint8_t* v_lds) {
  using Ge = Geo<CT, D>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ug = a.num_kv_heads;  // units per sequence: one per KV head
  build_prefix(pre, part, a, ug);
  if (wg == 0) {  // the merge kernel reads the prefix instead of rebuilding it
    int32_t* pre_g = stream_prefix(a, G, D);
    for (int i = threadIdx.x; i <= a.batch; i += kStreamThreads) pre_g[i] = pre[i];
  }
  const int64_t T = pre[a.batch];
  const int W = num_wgs * kWaves;
  const int w = wg * kWaves + wave;
  const int c0 = (int)(T * w / W), c1 = (int)(T * (w + 1) / W);
  if (c0 >= c1) return;
  const Pos p0 = locate(pre, a.batch, ug, c0);
  NewPiece pend;  // APPEND: the rows of the first unit ending past the first N chunks
  int pend_x = -1;
  if constexpr (APPEND) {
    Pos pe;
    pend_x = first_unit_end(pre, ug, p0, c0, c0 + N, c1, pe);
    if (pend_x >= 0) pend = fetch_new<kBF16, D>(a, pe.b, pe.gg, lane);
    append_range<CT, D>(a, pre, ug, p0, c0, c0, min(c1, c0 + N), lane);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no load of the caches moves above these stores
  }

  StreamCtx c;
  c.k_cache = a.k_cache;
  c.v_cache = a.v_cache;
  c.block_table = a.block_table;
  c.seqlens = a.cache_seqlens;
  c.len_bias = a.len_bias;
  c.row_bytes = Ge::row_bytes;
  c.slot_stride = a.num_kv_heads * Ge::row_bytes;
  c.block_bytes = (int64_t)a.block_size * c.slot_stride;
  c.max_blocks = a.max_blocks_per_seq;
  c.num_blocks = a.num_blocks;
  c.log2bs = __builtin_ctz(a.block_size);
  c.bs = a.block_size;
  c.cap = a.max_blocks_per_seq * a.block_size;
  c.heads_per_kv = G;
  c.head_groups = 1;
  Offs o;
  o.row = lane < Ge::vlanes ? (uint32_t)((lane / Ge::pieces) * c.slot_stride + (lane % Ge::pieces) * 16)
                           : 0x7ffffff0u;  // idle lanes read nothing
  o.q = (lane & 15) < G ? (uint32_t)((lane & 15) * Ge::qrow + (lane >> 4) * 16) : 0x7ffffff0u;

  uint8_t* k_w = k_lds + wave * Ge::vbytes;
  uint8_t* v_w = v_lds + wave * Ge::vbytes;
  uint32_t k_off[Ge::KS];
#pragma unroll
  for (int ks = 0; ks < Ge::KS; ++ks)
    k_off[ks] = (lane & 15) * Ge::lds_row + (((4 * ks + (lane >> 4)) ^ kswz<D>(lane & 15)) << 4);
  // transposed-read offsets: group lane / 16 reads keys 4 (lane / 16) + 16 x + (lane % 16) / 4,
  // elements 16 db + 4 (lane % 4) .. + 3 (vswz does not depend on the 16 x)
  uint32_t v_off[Ge::DB];
  {
    const int r = lane & 15, g = lane >> 4;
    const int key = 4 * g + r / 4;
#pragma unroll
    for (int db = 0; db < Ge::DB; ++db) {
      const int dd = 16 * db + 4 * (r & 3);
      v_off[db] = key * Ge::lds_row + (((dd >> 3) ^ vswz<D>(key)) << 4) + (dd & 7) * 2;
    }
  }
  MState<D> st;
  st.m = kNegBig;
  st.l = 0.0f;
#pragma unroll
  for (int db = 0; db < Ge::DB; ++db) st.o[db] = f32x4_t{};

  // N chunks in flight: at the step of chunk x ring slot x % N holds x and
  // the other slots x + 1 .. x + N - 1 (loading).  Once x's K and V are in
  // LDS and its scores are taken, the slot is refilled with x + N.  q of a
  // chunk's unit is loaded before the loads of the chunk after it (N - 1
  // buffers: q of x + N - 1 goes into x's buffer once its scores are taken).
  // Vector loads complete in order, so every wait is for the oldest chunk
  // only.  Positions past the wave's last chunk repeat it (loaded, never
  // used), so every step issues the same loads.
  constexpr int NQ = N > 1 ? N - 1 : 1;
  auto next_pos = [&](const Pos& p, int xp) __attribute__((always_inline)) {
    if (xp + 1 >= c1) return p;
    Pos n = advance(pre, ug, p);
    n.len = n.b == p.b ? p.len : seq_len_s(c, n.b);
    return n;
  };
  auto issue = [&](Chunk<CT, D>& r, const Pos& p, const Tbl& t) __attribute__((always_inline)) {
    load_kv<CT, D>(r, c, p, t, o);
    unit_scales<CT, D>(r, a, p);
  };
  Chunk<CT, D> ring[N];
  uint4 qbuf[NQ][Ge::KS];
  Pos cur = p0;
  cur.len = seq_len_s(c, cur.b);
  Pos ip = cur, lp = cur;  // next chunk to load, last chunk loaded
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (j < NQ) load_q<CT, D, G>(qbuf[j], a, ip, o);
    issue(ring[j], ip, fetch_tbl(c, ip));
    lp = ip;
    ip = next_pos(ip, c0 + j);
  }
  if constexpr (APPEND) {
    if (pend_x >= 0) {
      store_new<kBF16, CT, D>(a, pend, lane);
      append_range<CT, D>(a, pre, ug, p0, c0, pend_x + 1, c1, lane);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  Tbl tb = fetch_tbl(c, ip);
  int x = c0;
  auto step = [&](Chunk<CT, D>& R, uint4 (&Q)[Ge::KS]) __attribute__((always_inline)) -> bool {
    const Pos ipn = next_pos(ip, x + N);
    const Tbl tbn = fetch_tbl(c, ipn);
    store_kv<CT, D>(R, k_w, v_w, lane);
    const uint32_t kmask = R.kmask;
    const float ls = R.ls, vs = R.vs;
    const uint32_t qs = R.qs;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4_t s[2];
    chunk_scores<CT, D>(s, Q, qs, k_w, k_off);
    load_q<CT, D, G>(Q, a, lp, o);
    issue(R, ip, tb);
    lp = ip;
    ip = ipn;
    tb = tbn;
    chunk_update<D>(st, s, kmask, v_w, v_off, ls, lane);
    const bool last = x + 1 == c1;
    if (last || cur.ch + 1 == cur.nch) {
      const int u = cur.b * ug + cur.gg;
      const int64_t ustart = pre[cur.b] + (int64_t)cur.gg * cur.nch;
      const bool whole = ustart >= c0 && ustart + cur.nch <= c1;
      flush<D, G>(st, a, cur, whole, w + u, vs, lane);
    }
    if (last) return false;
    cur = next_pos(cur, x);
    ++x;
    // the next step overwrites this chunk's K and V in LDS: their reads are
    // done (they fed this chunk's MFMAs)
    return true;
  };
  // rounds of lcm(N, NQ) steps (every ring and q index a compile-time
  // constant, so all stay in registers).  Each step that ends the wave's
  // range leaves the loop directly: no path from such a step reaches the
  // loop head, whose waits would otherwise be sized for it.
  constexpr int R = N * NQ / (N % NQ == 0 ? NQ : 1);
  static_assert(R <= 6, "ring depth");
  for (;;) {
    if (!step(ring[0], qbuf[0])) break;
    if (!step(ring[1 % N], qbuf[1 % NQ])) break;
    if constexpr (R > 2) {
      if (!step(ring[2 % N], qbuf[2 % NQ])) break;
      if (!step(ring[3 % N], qbuf[3 % NQ])) break;
    }
    if constexpr (R > 4) {
      if (!step(ring[4 % N], qbuf[4 % NQ])) break;
      if (!step(ring[5 % N], qbuf[5 % NQ])) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // loads past the last chunk land before the wave ends
}

template <int CT, int D>
struct DecodeLds {  // LDS of decode_mfma_body, in bytes
  static constexpr int pre = ((kStreamMaxBatch + 1) * 4 + 15) / 16 * 16;
  static constexpr int part = kStreamThreads * 4;
  static constexpr int chunk = kWaves * Geo<CT, D>::vbytes;  // K (or V) chunks of all waves
  static constexpr int bytes = pre + part + 2 * chunk;
};

template <int CT, int D, int G, int N, int OCC, bool APPEND>
__global__ __launch_bounds__(kStreamThreads, OCC) void decode_mfma_kernel(DecodeArgs a) {
  using Ge = Geo<CT, D>;
  __shared__ int32_t pre[kStreamMaxBatch + 1];
  __shared__ int32_t part[kStreamThreads];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kWaves * Ge::vbytes];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[kWaves * Ge::vbytes];
  decode_mfma_body<CT, D, G, N, APPEND>(a, blockIdx.x, gridDim.x, pre, part, k_lds, v_lds);
}

// Chunks in flight per wave and waves per SIMD: bf16 chunks (16 KiB of K and
// V at head_dim 128) take 64 registers a lane, so two of them fit one wave
// per SIMD; fp8 chunks take half that, and two of them fit two waves.
template <int CT>
constexpr int depth() {
  return scaled8(CT) ? PKV_DECODE_DEPTH_FP8 : PKV_DECODE_DEPTH;
}

// Waves per SIMD the kernel is compiled for.
template <int CT>
constexpr int occupancy() {
  return scaled8(CT) ? PKV_DECODE_OCC_FP8 : PKV_DECODE_OCC;
}

template <int CT, int D, int G, bool APPEND>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  constexpr int N = depth<CT>();
  static int cached_grid = 0;  // per instantiation; the CU count of one process's GPUs is fixed
  if (cached_grid == 0) cached_grid = persistent_grid(decode_mfma_kernel<CT, D, G, N, occupancy<CT>(), APPEND>);
  const int64_t max_chunks = (int64_t)a.batch * a.num_kv_heads *
                             (((int64_t)a.max_blocks_per_seq * a.block_size + kChunk - 1) / kChunk);
  int64_t grid = cached_grid;
  if (grid * kWaves > max_chunks) grid = (max_chunks + kWaves - 1) / kWaves;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((decode_mfma_kernel<CT, D, G, N, occupancy<CT>(), APPEND>), dim3((unsigned)grid),
                     dim3(kStreamThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_stream_merge<kBF16, D, G>(a, 1, (int)(grid * kWaves), stream);
}

template <int CT, int D, bool APPEND>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_g<CT, D, 1, APPEND>(a, stream);
    case 2: return launch_g<CT, D, 2, APPEND>(a, stream);
    case 4: return launch_g<CT, D, 4, APPEND>(a, stream);
    case 8: return launch_g<CT, D, 8, APPEND>(a, stream);
    case 16: return launch_g<CT, D, 16, APPEND>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int CT, bool APPEND>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return launch_d<CT, 64, APPEND>(a, stream);
  if (a.head_dim == 128) return launch_d<CT, 128, APPEND>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mfd

template <int CT, int D, int GW, bool SMALL>
hipError_t launch_stream_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  constexpr int QT = (CT == kF32) ? kF32 : kBF16;
  static int cached_grid = 0;  // per instantiation; the CU count of one process's GPUs is fixed
  const int64_t max_chunks = (int64_t)a.batch * a.num_kv_heads * p.head_groups *
                             (((int64_t)a.max_blocks_per_seq * a.block_size + kChunk - 1) / kChunk);
  if (cached_grid == 0) cached_grid = persistent_grid(decode_stream_kernel<CT, D, GW, SMALL>);
  int64_t grid = cached_grid;
  if (grid * kWaves > max_chunks) grid = (max_chunks + kWaves - 1) / kWaves;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((decode_stream_kernel<CT, D, GW, SMALL>), dim3((unsigned)grid), dim3(kStreamThreads),
                     0, stream, a, p.head_groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_stream_merge<QT, D, GW>(a, p.head_groups, (int)(grid * kWaves), stream);
}

template <int CT, int D, int GW>
hipError_t launch_stream(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (a.block_size < 16) return launch_stream_t<CT, D, GW, true>(a, p, stream);
  return launch_stream_t<CT, D, GW, false>(a, p, stream);
}

template <int CT, int D, int GW>
hipError_t launch_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (p.stream) return launch_stream<CT, D, GW>(a, p, stream);
  constexpr int QT = (CT == kF32) ? kF32 : kBF16;
  const dim3 grid(a.num_kv_heads * p.head_groups, p.num_splits, a.batch);
  if (a.block_size < 16) {
    hipLaunchKernelGGL((decode_kernel<CT, D, GW, true>), grid, dim3(256), 0, stream, a, p.split_keys,
                       p.num_splits, p.head_groups);
  } else {
    hipLaunchKernelGGL((decode_kernel<CT, D, GW, false>), grid, dim3(256), 0, stream, a, p.split_keys,
                       p.num_splits, p.head_groups);
  }
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
    default: return hipErrorInvalidValue;
  }
}

template <int CT>
hipError_t launch_c(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (a.head_dim == 64) return launch_d<CT, 64>(a, p, stream);
  if (a.head_dim == 128) return launch_d<CT, 128>(a, p, stream);
  return hipErrorInvalidValue;
}

// One launch sequence (decode, then merge) over the batch of `a`.
hipError_t launch_whole(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  const bool append = a.k_new != nullptr;
  if (p.stream && p.mfma) {
    if (a.cache_dtype == kBF16) return append ? mfd::launch<kBF16, true>(a, stream) : mfd::launch<kBF16, false>(a, stream);
    if (a.cache_dtype == kFP8) return append ? mfd::launch<kFP8, true>(a, stream) : mfd::launch<kFP8, false>(a, stream);
    if (a.cache_dtype == kI8) return append ? mfd::launch<kI8, true>(a, stream) : mfd::launch<kI8, false>(a, stream);
    return hipErrorInvalidValue;
  }
  if (append) {  // the other plans: the append kernel, then the decode as usual
    const hipError_t e = launch_append(a, stream);
    if (e != hipSuccess) return e;
  }
  if (a.cache_dtype == kF32) return launch_c<kF32>(a, p, stream);
  if (a.cache_dtype == kBF16) return launch_c<kBF16>(a, p, stream);
  if (a.cache_dtype == kFP8) return launch_c<kFP8>(a, p, stream);
  if (a.cache_dtype == kI8) return launch_c<kI8>(a, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (!p.stream || p.slice >= a.batch) return launch_whole(a, p, stream);
  // Slices of the batch, in stream order: each slice's merge has read the
  // workspace before the next slice's decode writes it.
  const int64_t row_bytes = (int64_t)a.num_heads * a.head_dim * (a.q_dtype == kF32 ? 4 : 2);
  for (int32_t b0 = 0; b0 < a.batch; b0 += p.slice) {
    DecodeArgs s = a;
    s.batch = a.batch - b0 < p.slice ? a.batch - b0 : p.slice;
    s.out = static_cast<uint8_t*>(a.out) + b0 * row_bytes;
    s.q = static_cast<const uint8_t*>(a.q) + b0 * row_bytes;
    s.block_table = a.block_table + (int64_t)b0 * a.max_blocks_per_seq;
    s.cache_seqlens = a.cache_seqlens + b0;
    if (a.k_new != nullptr) {
      s.k_new = a.k_new + b0 * a.k_new_stride;
      s.v_new = a.v_new + b0 * a.v_new_stride;
    }
    const hipError_t e = launch_whole(s, p, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pkv
