// Varlen causal prefill over a packed batch, K/V contiguous or paged.
//
// [paged-doc] "ページド・アテンション", section "Varlen パス": request b owns query
// rows [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]).  [KV-mgmt]
// "効率的な KV キャッシュ管理と Attention 計算", section "Attention モジュールの実装":
// with block tables the paged caches replace k and v, so a chunk attends its
// cached prefix and itself.  Causal masking is aligned to the end: row i of a
// request with Lq queries and Lk keys sees keys j <= i + Lk - Lq.  [ch15]
// "KV cache / batching / paged attention", section "FlashAttention：注意計算そのも
// のを速く": tiles stay on chip and the result equals plain attention.
//
// Main kernel (prefill16_kernel; bf16 caches, and paged fp8 caches at
// head_dim 128): 128 query rows of one (request, q head) per workgroup, 4
// waves x 32 rows (two 16-column blocks) on v_mfma_f32_16x16x32_bf16, two
// waves per SIMD; K and V tiles copied HBM -> LDS by DMA (buffer loads with
// the lds bit, 1 KiB per wave instruction, no registers), two stages.
// Details at the kernel.
//
// Register-staged kernel (prefill_kernel; fp8 caches at head_dim 64), on
// v_mfma_f32_32x32x16_bf16:
// * workgroup = 128 query rows of one (request, q head); 4 waves x 32 rows.
// * per 64-key tile: S^T = K Q^T on MFMA (keys x queries), so each lane owns
//   one query column and 16 of its 32 scores per 32-key block; the row max and
//   row sum need one cross-lane exchange (lane ^ 32).  P^T, packed to bf16,
//   is used directly as the B operand of O^T += V^T P^T.
// * K tiles are staged in LDS row-major; V tiles are transposed in registers
//   (8 x 8 bf16 blocks with v_perm) and staged as V^T, so both MFMA A operands
//   are plain LDS reads.  Two LDS buffers: the next tile's global loads are in
//   flight while the current tile is computed.  fp8 caches are dequantised to
//   bf16 (exact) while staging; the K scale folds into the logit scale, the V
//   scale into the output.
//
// Both renumber workgroups (work_item) so that the tiles of one (request,
// KV head) run on the same XCD and share its L2, with the pairs balanced
// over the XCDs and the longest query tiles first.
//
// fp32 kernel: a plain per-row wave kernel (lanes over head_dim), kept for
// fp32 accuracy checks; it is not tuned.

#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_internal.h"

#ifndef PKV_PREFILL_CB
#define PKV_PREFILL_CB 2  // 16-row column blocks per wave (1 or 2)
#endif
#ifndef PKV_PREFILL_QK_SCHED
#define PKV_PREFILL_QK_SCHED 1
#endif

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int kThreads = 256;
constexpr int kWaitVmcnt0 = 0x0f70;  // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15)

template <int D>
struct Lds {
  static constexpr int k_row = D + 8;    // bf16 elements per K row (16-byte pad)
  static constexpr int vt_row = BN + 4;  // bf16 elements per V^T row (8-byte pad)
  static constexpr int k_elems = BN * k_row;
  static constexpr int vt_elems = D * vt_row;
  static constexpr int buf_elems = k_elems + vt_elems;
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Eight one-byte cache codes (E4M3 or int8; two words) -> eight bf16 (four
// words), exact.
template <int KVT>
__device__ __forceinline__ uint4 code8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(code8x2_to_bf16x2<KVT, false>(w0), code8x2_to_bf16x2<KVT, true>(w0),
                    code8x2_to_bf16x2<KVT, false>(w1), code8x2_to_bf16x2<KVT, true>(w1));
}

__device__ __forceinline__ uint32_t word_of(const uint4& x, int i) {
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

// bf16 element e (0..7) of rows a and b packed as (a[e], b[e]).
__device__ __forceinline__ uint32_t pair_elem(const uint4& a, const uint4& b, int e) {
  return perm(word_of(b, e >> 1), word_of(a, e >> 1), (e & 1) ? 0x07060302u : 0x05040100u);
}

struct KeyAddr {
  const uint8_t* base;  // k or v + g * row_bytes (+ k_start rows when contiguous)
  int64_t row_stride;   // bytes between consecutive slots / rows
  const int32_t* table; // paged: block_table row of the request, else nullptr
  int log2bs, bs_mask, num_blocks, lk, max_blocks;
};

// Address of key j's row (nullptr if the key does not exist).  Used by the
// fp32 kernel only.
__device__ __forceinline__ const uint8_t* key_row(const KeyAddr& ka, int j) {
  if (j >= ka.lk) return nullptr;
  if (ka.table == nullptr) return ka.base + (int64_t)j * ka.row_stride;
  const int blk = ka.table[j >> ka.log2bs];
  if (blk < 0 || blk >= ka.num_blocks) return nullptr;
  return ka.base + (((int64_t)blk << ka.log2bs) + (j & ka.bs_mask)) * ka.row_stride;
}

// Work item of hardware workgroup `hw`: (request b, q head h, query tile qt).
// Workgroup i runs on XCD i % 8.  Each (request, KV head) pair lives on one
// XCD (pair p on XCD p % 8), so the q heads and query tiles that share its
// K/V share that XCD's L2, and the pairs are dealt round-robin so every XCD
// gets the same share however the lengths vary.  Within an XCD the query
// tiles run from last to first: under the causal mask the last tiles carry
// the most keys, so the longest work starts first.  Returns false for the
// padding workgroups of XCDs with fewer pairs.
struct WorkItem {
  int b, h, g, qt;
};

__device__ __forceinline__ bool work_item(int hw, int q_tiles, int batch, int num_heads,
                                          int num_kv_heads, WorkItem& w) {
  const int G = num_heads / num_kv_heads;
  const int pairs = batch * num_kv_heads;
  const int x = hw & 7, j = hw >> 3;
  const int px = (pairs - x + 7) >> 3;  // pairs on XCD x
  const int per_tile = px * G;          // items per query tile on XCD x
  if (j >= q_tiles * per_tile) return false;
  w.qt = q_tiles - 1 - j / per_tile;
  const int rem = j % per_tile;
  const int pidx = x + 8 * (rem / G);
  w.b = pidx / num_kv_heads;
  w.g = pidx % num_kv_heads;
  w.h = w.g * G + rem % G;
  return true;
}

// Grid for work_item(): 8 XCDs x the largest per-XCD share.
__host__ __forceinline__ int64_t work_grid(int q_tiles, int batch, int num_heads, int num_kv_heads) {
  const int64_t pairs = (int64_t)batch * num_kv_heads;
  return 8 * (int64_t)q_tiles * ((pairs + 7) / 8) * (num_heads / num_kv_heads);
}

// How the 256 threads of a workgroup move one 64-key tile from HBM to LDS.
// K: each thread copies `kp` 16-byte pieces (consecutive threads cover a row
// contiguously).  V: each thread owns a block of `kr` keys x 8 head-dim
// elements, transposes it in registers and writes it into V^T; threads that
// share an 8-element group are adjacent so their LDS writes hit distinct banks.
template <int KVT, int D>
struct Loader {
  static constexpr int elt = Elt<KVT>::bytes;
  static constexpr int ppr = D * elt / 16;          // 16-byte pieces per K row
  static constexpr int kp = BN * ppr / kThreads;    // K pieces per thread
  static constexpr int kstep = kThreads / ppr;      // rows between a thread's K pieces
  static constexpr int dg = D / 8;                  // 8-element groups per V row
  static constexpr int kr = BN * dg / kThreads;     // V rows per thread
  static constexpr int kgroups = BN / kr;           // key groups per 8-element group
  static_assert(kp >= 1 && (kr == 2 || kr == 4), "tile shape");

  // per tile in flight
  uint4 kd[kp];
  uint4 vd[kr];
  uint32_t ok;        // validity bit per K piece (bits 0..kp-1) and V row (bits 8..)
  int32_t tk[kp];     // block ids (paged) of the next tile to load
  int32_t tv;

  __device__ __forceinline__ int k_row(int tid, int i) const { return tid / ppr + kstep * i; }
  __device__ __forceinline__ int k_piece(int tid) const { return tid % ppr; }
  __device__ __forceinline__ int v_group(int tid) const { return tid / kgroups; }   // 8-element group
  __device__ __forceinline__ int v_key0(int tid) const { return (tid % kgroups) * kr; }

  // Block-table entries of tile `key0` (global loads, consumed one tile later).
  __device__ __forceinline__ void fetch_table(const KeyAddr& a, int key0, int tid) {
    if (a.table == nullptr) return;
#pragma unroll
    for (int i = 0; i < kp; ++i) {
      const int j = key0 + k_row(tid, i);
      tk[i] = a.table[min(j >> a.log2bs, a.max_blocks - 1)];
    }
    const int j = key0 + v_key0(tid);
    tv = a.table[min(j >> a.log2bs, a.max_blocks - 1)];
  }

  // Offset of key j given its block id; `valid` false -> offset 0 (a safe row).
  __device__ __forceinline__ int64_t offset(const KeyAddr& a, int j, int blk, bool& valid) const {
    if (a.table == nullptr) {
      valid = j < a.lk;
      return valid ? (int64_t)j * a.row_stride : 0;
    }
    valid = j < a.lk && blk >= 0 && blk < a.num_blocks;
    return valid ? ((((int64_t)blk) << a.log2bs) + (j & a.bs_mask)) * a.row_stride : 0;
  }

  // Issue the global loads of tile `key0` with the table entries fetched earlier.
  __device__ __forceinline__ void load(const KeyAddr& ka, const KeyAddr& va, int key0, int tid) {
    ok = 0;
#pragma unroll
    for (int i = 0; i < kp; ++i) {
      bool valid;
      const int64_t off = offset(ka, key0 + k_row(tid, i), tk[i], valid);
      kd[i] = *reinterpret_cast<const uint4*>(ka.base + off + k_piece(tid) * 16);
      ok |= (uint32_t)valid << i;
    }
    const int j0 = key0 + v_key0(tid);
#pragma unroll
    for (int r = 0; r < kr; ++r) {
      bool valid;
      const int64_t off = offset(va, j0 + r, tv, valid);
      const uint8_t* src = va.base + off + v_group(tid) * 8 * elt;
      if constexpr (KVT == kBF16) {
        vd[r] = *reinterpret_cast<const uint4*>(src);
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(src);
        vd[r] = make_uint4(x.x, x.y, 0u, 0u);
      }
      ok |= (uint32_t)valid << (8 + r);
    }
  }

  // Zero invalid rows, dequantise fp8, transpose V, write the tile to LDS.
  __device__ __forceinline__ void store(uint16_t* buf, int tid) const {
    using L = Lds<D>;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kp; ++i) {
      const uint4 x = ((ok >> i) & 1) ? kd[i] : zero;
      uint16_t* dst = buf + k_row(tid, i) * L::k_row + k_piece(tid) * (16 / elt);
      if constexpr (KVT == kBF16) {
        *reinterpret_cast<uint4*>(dst) = x;
      } else {
        *reinterpret_cast<uint4*>(dst) = code8x8_to_bf16x8<KVT>(x.x, x.y);
        *reinterpret_cast<uint4*>(dst + 8) = code8x8_to_bf16x8<KVT>(x.z, x.w);
      }
    }
    uint4 rows[kr];
#pragma unroll
    for (int r = 0; r < kr; ++r) {
      const uint4 x = ((ok >> (8 + r)) & 1) ? vd[r] : zero;
      if constexpr (KVT == kBF16) {
        rows[r] = x;
      } else {
        rows[r] = code8x8_to_bf16x8<KVT>(x.x, x.y);
      }
    }
    uint16_t* vt = buf + L::k_elems + v_group(tid) * 8 * L::vt_row + v_key0(tid);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (kr == 4) {
        *reinterpret_cast<uint2*>(vt + e * L::vt_row) =
            make_uint2(pair_elem(rows[0], rows[1], e), pair_elem(rows[2], rows[3], e));
      } else {
        *reinterpret_cast<uint32_t*>(vt + e * L::vt_row) = pair_elem(rows[0], rows[1], e);
      }
    }
  }
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8_t, x); }

template <int KVT, int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a, int q_tiles) {
  using L = Lds<D>;
  constexpr int KS = D / 16;   // MFMA k-steps over head_dim
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * L::buf_elems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;

  WorkItem w;
  if (!work_item(blockIdx.x, q_tiles, a.batch, a.num_heads, a.num_kv_heads, w)) return;
  const int qt = w.qt, h = w.h, b = w.b, g = w.g;

  const int q_start = a.cu_seqlens_q[b];
  int lq = a.cu_seqlens_q[b + 1] - q_start;
  if (lq > a.max_seqlen_q) lq = a.max_seqlen_q;
  if (q_start < 0 || q_start >= a.total_q) lq = 0;
  else if (lq > a.total_q - q_start) lq = a.total_q - q_start;
  const int q0 = qt * BM;
  if (q0 >= lq) return;
  const int k_start = a.cu_seqlens_k[b];
  int lk = a.cu_seqlens_k[b + 1] - k_start;
  if (lk < 0) lk = 0;
  const bool paged = a.block_table != nullptr;
  if (paged) {
    const int cap = a.max_blocks_per_seq * a.block_size;
    if (lk > cap) lk = cap;
  } else {
    if (k_start < 0 || k_start > a.total_k) lk = 0;
    else if (lk > a.total_k - k_start) lk = a.total_k - k_start;
  }
  const int offset = lk - lq;  // bottom-right causal alignment
  const int last_row = min(q0 + BM, lq) - 1;
  int key_end = a.causal ? min(lk, last_row + offset + 1) : lk;
  if (key_end < 0) key_end = 0;
  const int n_tiles = (key_end + BN - 1) / BN;

  constexpr int elt = Elt<KVT>::bytes;
  const int64_t row_bytes = (int64_t)D * elt;
  KeyAddr ka, va;
  ka.row_stride = va.row_stride = (int64_t)a.num_kv_heads * row_bytes;
  ka.base = a.k + g * row_bytes + (paged ? 0 : (int64_t)k_start * ka.row_stride);
  va.base = a.v + g * row_bytes + (paged ? 0 : (int64_t)k_start * va.row_stride);
  ka.table = va.table = paged ? a.block_table + (int64_t)b * a.max_blocks_per_seq : nullptr;
  ka.log2bs = va.log2bs = paged ? __builtin_ctz(a.block_size) : 0;
  ka.bs_mask = va.bs_mask = paged ? a.block_size - 1 : 0;
  ka.num_blocks = va.num_blocks = a.num_blocks;
  ka.max_blocks = va.max_blocks = a.max_blocks_per_seq;
  ka.lk = va.lk = lk;

  // this wave's query column: row q0 + 32 * wave + col
  const int qrow = q0 + wave * 32 + col;
  const bool qvalid = qrow < lq;
  uint4 qf[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)(q_start + (qvalid ? qrow : 0)) * a.num_heads + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 x = *reinterpret_cast<const uint4*>(qp + ks * 16);
      qf[ks] = qvalid ? x : make_uint4(0u, 0u, 0u, 0u);
    }
    // Resolve the q loads here: otherwise the wait for them lands inside the
    // tile loop, where it also waits for the next tile's prefetch.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  float scale = a.softmax_scale * kLog2e;
  float out_scale = 1.0f;
  if constexpr (scaled8(KVT)) {
    scale *= a.k_scale[g];
    out_scale = a.v_scale[g];
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
  float m = kNegBig, l = 0.0f;

  Loader<KVT, D> ld;
  if (n_tiles > 0) {
    ld.fetch_table(ka, 0, tid);
    ld.load(ka, va, 0, tid);
    if (n_tiles > 1) ld.fetch_table(ka, BN, tid);
    ld.store(lds, tid);
  }
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();
    const int key0 = t * BN;
    if (t + 1 < n_tiles) {
      ld.load(ka, va, key0 + BN, tid);
      if (t + 2 < n_tiles) ld.fetch_table(ka, key0 + 2 * BN, tid);
    }
    const uint16_t* kb_lds = lds + (t & 1) * L::buf_elems;
    const uint16_t* vt_lds = kb_lds + L::k_elems;

    // S^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const uint16_t* krow = kb_lds + (kb * 32 + col) * L::k_row + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kf = *reinterpret_cast<const uint4*>(krow + ks * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), s[kb], 0, 0, 0);
      }
    }
    // scale, mask, row max
    const bool need_mask = (key0 + BN > lk) || (a.causal && key0 + BN - 1 > q0 + wave * 32 + offset);
    float mx = kNegBig;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key < lk && (!a.causal || key <= qrow + offset);
          const float x = vis ? s[kb][r] * scale : -INFINITY;
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = s[kb][r] * scale;
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
    }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    float psum = 0.0f;
    uint4 pb[2][2];  // [key block][16-key half] bf16 B operands
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        f32x8_t pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(s[kb][hs * 8 + e] - mn);
          pv[e] = p;
          psum += p;
        }
        pb[kb][hs] = __builtin_bit_cast(uint4, __builtin_convertvector(pv, bf16x8_t));
      }
    l = l * alpha + psum;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* vrow = vt_lds + (db * 32 + col) * L::vt_row + 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const int k0 = kb * 32 + hs * 16;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + k0);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + k0 + 8);
          const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pb[kb][hs]), o[db], 0, 0, 0);
        }
    }
    if (t + 1 < n_tiles) ld.store(lds + ((t + 1) & 1) * L::buf_elems, tid);
  }

  // normalise and store: lane holds O^T rows 8*(r/4) + 4*half + r%4 of each 32-row block
  l += shfl_xor(l, 32);
  if (!qvalid) return;
  const float inv = l > 0.0f ? out_scale / l : 0.0f;
  uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)(q_start + qrow) * a.num_heads + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + rg * 8 + half * 4;
      const uint32_t w0 = pack_bf16x2(o[db][rg * 4 + 0] * inv, o[db][rg * 4 + 1] * inv);
      const uint32_t w1 = pack_bf16x2(o[db][rg * 4 + 2] * inv, o[db][rg * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
    }
}

// fp32: one wave per (query row, q head); lanes hold head_dim / 64 elements.
template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int NV = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;  // (row of the packed q, head)
  if (item >= (int64_t)a.total_q * a.num_heads) return;
  const int row = (int)(item / a.num_heads), h = (int)(item % a.num_heads);
  // request owning this row: binary search over cu_seqlens_q
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_seqlens_q[mid] <= row) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int q_start = a.cu_seqlens_q[b];
  const int lq = a.cu_seqlens_q[b + 1] - q_start;
  if (row < q_start || row - q_start >= lq) return;
  const int i = row - q_start;
  const int g = h / (a.num_heads / a.num_kv_heads);
  const int k_start = a.cu_seqlens_k[b];
  int lk = a.cu_seqlens_k[b + 1] - k_start;
  if (lk < 0) lk = 0;
  const bool paged = a.block_table != nullptr;
  if (paged) lk = min(lk, a.max_blocks_per_seq * a.block_size);
  else if (k_start < 0 || k_start > a.total_k) lk = 0;
  else lk = min(lk, a.total_k - k_start);
  const int kend = a.causal ? max(0, min(lk, i + lk - lq + 1)) : lk;
  const int64_t row_bytes = (int64_t)D * 4;
  KeyAddr ka, va;
  ka.row_stride = va.row_stride = (int64_t)a.num_kv_heads * row_bytes;
  ka.base = a.k + g * row_bytes + (paged ? 0 : (int64_t)k_start * ka.row_stride);
  va.base = a.v + g * row_bytes + (paged ? 0 : (int64_t)k_start * va.row_stride);
  ka.table = va.table = paged ? a.block_table + (int64_t)b * a.max_blocks_per_seq : nullptr;
  ka.log2bs = va.log2bs = paged ? __builtin_ctz(a.block_size) : 0;
  ka.bs_mask = va.bs_mask = paged ? a.block_size - 1 : 0;
  ka.num_blocks = va.num_blocks = a.num_blocks;
  ka.lk = va.lk = lk;
  const float* qp = reinterpret_cast<const float*>(a.q) + ((int64_t)row * a.num_heads + h) * D;
  float qv[NV], o[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    qv[e] = qp[lane * NV + e];
    o[e] = 0.0f;
  }
  const float scale = a.softmax_scale * kLog2e;
  float m = kNegBig, l = 0.0f;
  for (int j = 0; j < kend; ++j) {
    const float* kr = reinterpret_cast<const float*>(key_row(ka, j));
    const float* vr = reinterpret_cast<const float*>(key_row(va, j));
    if (kr == nullptr) continue;
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < NV; ++e) dot = fmaf(qv[e], kr[lane * NV + e], dot);
    for (int x = 1; x < 64; x <<= 1) dot += shfl_xor(dot, x);
    const float s = dot * scale;
    const float mn = fmaxf(m, s);
    const float alpha = fast_exp2(m - mn);
    const float p = fast_exp2(s - mn);
    m = mn;
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < NV; ++e) o[e] = fmaf(p, vr[lane * NV + e], o[e] * alpha);
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* op = reinterpret_cast<float*>(a.out) + ((int64_t)row * a.num_heads + h) * D;
#pragma unroll
  for (int e = 0; e < NV; ++e) op[lane * NV + e] = o[e] * inv;
}

// ---------------------------------------------------------------------------
// DMA-fed kernel: K/V tiles move HBM -> LDS by DMA, V is read transposed
// ---------------------------------------------------------------------------
//
// * a 64-key tile of K and of V is copied straight from HBM into LDS (1 KiB
//   per wave instruction; no registers).  The DMA writes each KiB
//   contiguously, so bank conflicts are avoided by permuting what each lane
//   fetches: LDS piece position i of row r holds the row's 16-byte piece
//   i ^ swz(r).  fp8 tiles are copied as they are and dequantised by the wave
//   that copied them into bf16 tiles with the same permutations.
// * online softmax in the log2 domain with a lazy running max: the output is
//   rescaled only when a row's max grows by more than 2^8, so most tiles skip
//   the rescale; the result is the same exact algebra (numerator and
//   denominator always share one reference max).  Row sums accumulate the
//   bf16-rounded p that the MFMA consumes.
// * keys past the sequence end or in invalid blocks are masked, and their V
//   rows are zeroed in LDS so that stale cache contents never reach the
//   output.
namespace dma {

constexpr int kBN = 64;
constexpr float kRescaleBits = 8.0f;  // lazy-max threshold (log2 domain)
constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor, dword 3

// Tile geometry for head_dim D and W waves per workgroup (32 query rows per
// wave): one DMA instruction fills 1 KiB of a K or V tile.
template <int D, int W, int E = 2>
struct Tile {
  static constexpr int row_bytes = D * E;  // E: bytes per element
  static constexpr int pieces = row_bytes / 16;          // 16-byte pieces per row
  static constexpr int bytes = kBN * row_bytes;          // one K or V tile
  static constexpr int rows_per_dma = 1024 / row_bytes;  // rows one DMA instruction fills
  static constexpr int dma_per_wave = bytes / 1024 / W;  // per K (or V) tile
  static constexpr int rows_per_wave = kBN / W;
  static constexpr int groups_per_wave = rows_per_wave / 8;  // 8-key groups
  static_assert(dma_per_wave >= 1 && groups_per_wave >= 1, "tile shape");
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

__device__ __forceinline__ uint2 read_tr(const uint8_t* p) {
  const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
  return __builtin_bit_cast(uint2, x);
}

// Where the keys of one tile live, in 8-key groups (block_size >= 8, so a
// group never straddles a block): the byte offsets of the first rows of this
// wave's groups, and which of the tile's keys exist.  Block-table entries are
// read with scalar loads through the constant address space (the table is
// not written while a kernel runs), issued after a tile's LDS reads are done:
// scalar loads share their wait counter with LDS reads, and an outstanding
// one would hold up every LDS wait of the next tile.
template <int GPW>
struct TileMap {
  int64_t off[GPW];  // uniform
  uint64_t valid;    // bit k: key k of the tile exists and sits in a valid block
  bool blocks_ok;    // every block of the tile is valid (valid is then a prefix mask)
};

struct Entries {
  int32_t e[8];  // block id of each 8-key group of a tile (uniform)
};

template <bool PAGED>
__device__ __forceinline__ void fetch_entries(Entries& en, const PrefillArgs& a, const int32_t* table,
                                              int key0, int log2bs) {
  if constexpr (PAGED) {
    const_i32_ptr t = (const_i32_ptr)table;
#pragma unroll
    for (int g = 0; g < 8; ++g) en.e[g] = t[min((key0 + 8 * g) >> log2bs, a.max_blocks_per_seq - 1)];
  }
}

template <bool PAGED, int GPW>
__device__ __forceinline__ void resolve(TileMap<GPW>& m, const PrefillArgs& a, const Entries& en,
                                        int64_t row_stride, int key0, int lk, int log2bs, int wave) {
  const int n = lk - key0;  // keys of the tile that exist (clamped below)
  const uint64_t len_mask = n >= 64 ? ~0ull : (n <= 0 ? 0ull : ((1ull << n) - 1));
  if constexpr (PAGED) {
    uint64_t blk_mask = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      blk_mask |= ((uint32_t)en.e[g] < (uint32_t)a.num_blocks ? 0xffull : 0ull) << (8 * g);
    m.valid = len_mask & blk_mask;
    m.blocks_ok = blk_mask == ~0ull;
#pragma unroll
    for (int x = 0; x < GPW; ++x) {
      const int grp = wave * GPW + x;
      int blk = en.e[0];
#pragma unroll
      for (int g = 1; g < 8; ++g) blk = grp == g ? en.e[g] : blk;
      const int key = key0 + 8 * grp;
      const bool ok = (uint32_t)blk < (uint32_t)a.num_blocks;
      m.off[x] = ok ? (((int64_t)blk << log2bs) + (key & ((1 << log2bs) - 1))) * row_stride : 0;
    }
  } else {
    m.valid = len_mask;
    m.blocks_ok = true;
#pragma unroll
    for (int x = 0; x < GPW; ++x) m.off[x] = 0;  // packed rows are addressed per lane
  }
}

// Zero this wave's V rows of keys that do not exist (after its DMA landed).
template <int D, int W>
__device__ __forceinline__ void zero_rows(uint64_t valid, uint8_t* vbuf, int wave, int lane) {
  using T = Tile<D, W>;
  const int r0 = wave * T::rows_per_wave;
  const uint32_t bad = ~(uint32_t)(valid >> r0) & ((1u << T::rows_per_wave) - 1);
  if (bad == 0) return;
  constexpr int per_pass = 64 * 16 / T::row_bytes;  // rows per pass
#pragma unroll
  for (int i = 0; i < T::rows_per_wave; i += per_pass) {
    const int r = i + lane / T::pieces;
    if (r < T::rows_per_wave && ((bad >> r) & 1u))
      *reinterpret_cast<uint4*>(vbuf + (r0 + r) * T::row_bytes + (lane % T::pieces) * 16) =
          make_uint4(0u, 0u, 0u, 0u);
  }
}

// Piece permutations of the 16-query-row kernel (K read as 16 consecutive
// rows x one piece for the A operand; V read transposed, 16 consecutive rows
// x 2 pieces): both free of bank conflicts.
template <int D>
__device__ __forceinline__ int kswz16(int r) {
  return D == 128 ? (r & 15) : (r & 7);
}
template <int D>
__device__ __forceinline__ int vswz16(int r) {
  return D == 128 ? ((r & 7) << 1) : ((r & 3) << 1);
}

// An LDS address whose object the compiler cannot see.  The pipelined
// kernel waits for its copies itself (s_waitcnt before a barrier); the
// compiler does not track copies made through such an address, where it
// would otherwise make some LDS reads wait for every copy in flight (its
// record of which copy feeds which buffer does not survive the loop).
__device__ __forceinline__ lds_void_t* lds_opaque(uint8_t* p) {
  uint32_t x = (uint32_t)(uintptr_t)(lds_void_t*)p;
  asm volatile("" : "+s"(x));
  return (lds_void_t*)(uintptr_t)x;
}

// DMA of this wave's rows of one K or V tile into buf, through buffer
// descriptors: paged rows by the 8-key group's block, packed rows from the
// tile's first key with the descriptor ending at the request's last key, so
// rows past it read zeros.  SW picks the piece permutation (0: none, 1: the
// K operand's, 2: the transposed V reads'); E is the element size.
template <int D, int W, bool PAGED, int SW, int E = 2>
__device__ __forceinline__ void issue_rows(const TileMap<Tile<D, W, E>::groups_per_wave>& m, const uint8_t* base,
                                           int64_t row_stride, int key0, int lk, uint8_t* buf, int wave,
                                           int lane) {
  using T = Tile<D, W, E>;
  const int rr = lane / T::pieces;
  const int pos = lane % T::pieces;
  __amdgpu_buffer_rsrc_t rs[PAGED ? T::groups_per_wave : 1];
  if constexpr (PAGED) {
#pragma unroll
    for (int x = 0; x < T::groups_per_wave; ++x)
      rs[x] = __builtin_amdgcn_make_buffer_rsrc((void*)(base + m.off[x]), 0, (int)(8 * row_stride), kBufferWord3);
  } else {
    const int rows = min(lk - key0, kBN);  // >= 1: only tiles that hold a key are copied
    rs[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)key0 * row_stride), 0,
                                              (int)((rows - 1) * row_stride + T::row_bytes), kBufferWord3);
  }
#pragma unroll
  for (int j = 0; j < T::dma_per_wave; ++j) {
    const int chunk = wave * T::dma_per_wave + j;
    const int r = chunk * T::rows_per_dma + rr;
    const int piece = pos ^ (SW == 0 ? 0 : (SW == 1 ? kswz16<D>(r) : vswz16<D>(r)));
    if constexpr (PAGED) {
      const int voff = (int)((r & 7) * row_stride) + piece * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[(j * T::rows_per_dma) >> 3], lds_opaque(buf + chunk * 1024), 16,
                                               voff, 0, 0, 0);
    } else {
      const int voff = (int)(r * row_stride) + piece * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[0], lds_opaque(buf + chunk * 1024), 16, voff, 0, 0, 0);
    }
  }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float max_quarters(float x) {  // over lanes l, l^16, l^32, l^48
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_halves(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

__device__ __forceinline__ float sum_quarters(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return sum_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// 16 or 32 query rows per wave (CB = 1 or 2 column blocks of 16), 128 rows
// per workgroup, on v_mfma_f32_16x16x32_bf16.  With CB = 1 a wave's
// registers (about a hundred) allow four waves per SIMD; with CB = 2 each K
// and V fragment read from LDS feeds two MFMAs (one per column block), which
// halves the LDS reads per flop, at two waves per SIMD.  Per 64-key tile and
// column block: S^T = K Q^T as four 16-key blocks (lane l holds keys
// 16 kb + 4 (l / 16) + i of query column l % 16), online softmax per column
// (max and sum over the lane's 16 scores, then over lanes l ^ 16, l ^ 32),
// O^T += V^T P^T per 32-key half with P^T's k-slot 8 (l / 16) + j holding
// key 4 (l / 16) + j (j < 4) or 16 + 4 (l / 16) + j - 4 (j >= 4) of the
// half: the lane's own scores, so P^T needs no exchange; the transposed V
// reads put the same keys in the same k-slots.  Two LDS stages of K and V
// tiles copied by DMA through buffer descriptors.
// The workgroup body: work item hw (see work_item), with its LDS passed in
// (two stages of K and V tiles as copied, and for one-byte caches the bf16
// tiles dequantised from them), so that a launch that serves other work too
// can run it.  Buffers are 1 KiB-aligned.
template <int KVT, int D, bool PAGED, int CB>
__device__ __forceinline__ void prefill16_body(const PrefillArgs& a, int q_tiles, int hw, uint8_t* k0b,
                                               uint8_t* v0b, uint8_t* k1b, uint8_t* v1b, uint8_t* kxb,
                                               uint8_t* vxb) {
  constexpr int W = 8 / CB;
  constexpr bool F8 = KVT == kFP8 || KVT == kI8;  // one-byte cache, dequantised in LDS
  static_assert(CB == 1 || CB == 2, "one or two column blocks per wave");
  static_assert(!F8 || (PAGED && D == 128), "one-byte caches: paged, head_dim 128");
  using T = Tile<D, W>;              // bf16 tiles the MFMAs read
  using TC = Tile<D, W, F8 ? 1 : 2>;  // tiles as copied from the cache
  constexpr int BM = 16 * CB * W;
  constexpr int KS = D / 32;  // MFMA k-steps over head_dim
  constexpr int DB = D / 16;  // 16-row blocks of O^T
  constexpr int GPW = T::groups_per_wave;
  constexpr int kDma = TC::dma_per_wave;
  constexpr int kWaitLgkm0 = 0xc07f;
  static_assert(BM == 128 && GPW == CB && TC::groups_per_wave == GPW, "8-key groups per wave");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 15, grp4 = lane >> 4;

  WorkItem w;
  if (!work_item(hw, q_tiles, a.batch, a.num_heads, a.num_kv_heads, w)) return;
  const int qt = w.qt, h = w.h, b = w.b, g = w.g;

  const int q_start = a.cu_seqlens_q[b];
  int lq = a.cu_seqlens_q[b + 1] - q_start;
  if (lq > a.max_seqlen_q) lq = a.max_seqlen_q;
  if (q_start < 0 || q_start >= a.total_q) lq = 0;
  else if (lq > a.total_q - q_start) lq = a.total_q - q_start;
  const int q0 = qt * BM;
  if (q0 >= lq) return;
  const int k_start = a.cu_seqlens_k[b];
  int lk = a.cu_seqlens_k[b + 1] - k_start;
  if (lk < 0) lk = 0;
  if constexpr (PAGED) {
    lk = min(lk, a.max_blocks_per_seq * a.block_size);
  } else {
    if (k_start < 0 || k_start > a.total_k) lk = 0;
    else if (lk > a.total_k - k_start) lk = a.total_k - k_start;
  }
  const int offset = lk - lq;  // bottom-right causal alignment
  const int last_row = min(q0 + BM, lq) - 1;
  int key_end = a.causal ? min(lk, last_row + offset + 1) : lk;
  if (key_end < 0) key_end = 0;
  const int n_tiles = (key_end + kBN - 1) / kBN;

  const int64_t row_stride = (int64_t)a.num_kv_heads * TC::row_bytes;
  const uint8_t* kbase = a.k + g * TC::row_bytes + (PAGED ? 0 : (int64_t)k_start * row_stride);
  const uint8_t* vbase = a.v + g * TC::row_bytes + (PAGED ? 0 : (int64_t)k_start * row_stride);
  const int32_t* table = PAGED ? a.block_table + (int64_t)b * a.max_blocks_per_seq : nullptr;
  const int log2bs = PAGED ? __builtin_ctz(a.block_size) : 0;

  // this lane's query column in column block cb: row q0 + 16 (CB wave + cb) + col
  const int wrow0 = q0 + 16 * CB * wave;  // the wave's first row
  int qrow[CB];
  bool qvalid[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    qrow[cb] = wrow0 + 16 * cb + col;
    qvalid[cb] = qrow[cb] < lq;
  }
  const bool wave_rows = wrow0 < lq;
  // The row max is taken over unscaled scores, which needs scale > 0: a
  // negative scale is applied as |scale| to -q (bf16 negation is exact), and
  // a zero scale as 1e-30 (every logit then rounds to exactly 0 in the
  // exponent, as with scale 0, while masked keys stay at -inf instead of
  // -inf * 0).
  // With fp8 caches the K scale folds into the logit scale and the V scale
  // into the output.
  const float sc = F8 ? a.softmax_scale * a.k_scale[g] : a.softmax_scale;
  const uint32_t q_sign = sc < 0.0f ? 0x80008000u : 0u;
  const float scale = fmaxf(fabsf(sc) * kLog2e, 1e-30f);
  // q[qrow][32 ks + 8 (lane / 16) .. + 8], as loaded (rows past the request
  // read row 0); the sign and the zeroing of those rows are applied once the
  // first tile has landed, so that the q loads and the first copy are in
  // flight together
  uint4 qf[CB][KS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)(q_start + (qvalid[cb] ? qrow[cb] : 0)) * a.num_heads + h) * D + grp4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[cb][ks] = *reinterpret_cast<const uint4*>(qp + ks * 32);
  }

  // K A operand: row 16 kb + col, piece 4 ks + lane / 16
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = col * T::row_bytes + (((4 * ks + grp4) ^ kswz16<D>(col)) << 4);
  // V transposed reads: lane group lane / 16 reads keys 4 (lane / 16) + (lane % 16) / 4 (and + 16),
  // elements 16 db + 4 (lane % 4) .. + 3
  int v_off[DB];
  {
    const int key = 4 * grp4 + col / 4;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dd = 16 * db + 4 * (col & 3);
      v_off[db] = key * T::row_bytes + (((dd >> 3) ^ vswz16<D>(key)) << 4) + (dd & 7) * 2;
    }
  }

  f32x4_t o[CB][DB];
  float m[CB], l[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[cb][db] = f32x4_t{};
    m[cb] = kNegBig;
    l[cb] = 0.0f;
  }

  auto compute = [&](const uint8_t* kb_lds, const uint8_t* vb_lds, int key0, uint64_t valid, bool blocks_ok)
                     __attribute__((always_inline)) {
    const int lim_first = min(a.causal ? wrow0 + offset - key0 + 1 : kBN, lk - key0);
    const int lim_last = min(a.causal ? wrow0 + 16 * CB + offset - key0 : kBN, lk - key0);
    if (!wave_rows || lim_last <= 0) return;  // nothing of this tile reaches the wave's rows
    f32x4_t s[CB][4];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[cb][kb] = f32x4_t{};
    // K fragments one k-step ahead: the four reads of step ks + 1 are in
    // flight during the 4 CB MFMAs of step ks
    uint4 kf[2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      kf[0][kb] = *reinterpret_cast<const uint4*>(kb_lds + kb * 16 * T::row_bytes + k_off[0]);
#if PKV_PREFILL_QK_SCHED
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the first step's reads
#endif
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          kf[(ks + 1) & 1][kb] = *reinterpret_cast<const uint4*>(kb_lds + kb * 16 * T::row_bytes + k_off[ks + 1]);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          s[cb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[ks & 1][kb]), as_bf16x8(qf[cb][ks]),
                                                              s[cb][kb], 0, 0, 0);
#if PKV_PREFILL_QK_SCHED
      if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the next step's reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * CB, 0);             // then this step's MFMAs
#endif
    }
    // mask (register i of block kb holds key 16 kb + 4 (lane / 16) + i)
    if (lim_first < kBN) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int lim = min(a.causal ? qrow[cb] + offset - key0 + 1 : kBN, lk - key0);
        const int lim_g = lim - 4 * grp4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[cb][kb][i] = 16 * kb + i < lim_g ? s[cb][kb][i] : -INFINITY;
      }
    }
    if (!blocks_ok) {  // corrupt block table: skip the keys of invalid blocks
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bool ok = ((valid >> (16 * kb + 4 * grp4)) & 0xfull) != 0;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[cb][kb][i] = ok ? s[cb][kb][i] : -INFINITY;
      }
    }
    float mx[CB];
    bool grow = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float x = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, s[cb][kb][i]);
      mx[cb] = max_quarters(x) * scale;
      grow = grow || mx[cb] > m[cb] + kRescaleBits;
    }
    // lazy running max: move it (and rescale) only when it grows by > 2^8
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float mn = fmaxf(m[cb], mx[cb]);
        const float alpha = fast_exp2(m[cb] - mn);
        m[cb] = mn;
        l[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[cb][db] *= alpha;
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint4 pb[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float neg_m = -m[cb];
        f32x8_t pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = fast_exp2(fmaf(s[cb][2 * hf][i], scale, neg_m));
          pv[4 + i] = fast_exp2(fmaf(s[cb][2 * hf + 1][i], scale, neg_m));
        }
        pb[cb] = __builtin_bit_cast(uint4, __builtin_convertvector(pv, bf16x8_t));
        float ps = l[cb];
        ps = dot2_bf16(pb[cb].x, 0x3f803f80u, ps);
        ps = dot2_bf16(pb[cb].y, 0x3f803f80u, ps);
        ps = dot2_bf16(pb[cb].z, 0x3f803f80u, ps);
        l[cb] = dot2_bf16(pb[cb].w, 0x3f803f80u, ps);
      }
      const uint8_t* vh = vb_lds + hf * 32 * T::row_bytes;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint2 lo = read_tr(vh + v_off[db]);
        const uint2 hi = read_tr(vh + 16 * T::row_bytes + v_off[db]);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          o[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                                              as_bf16x8(pb[cb]), o[cb][db], 0, 0, 0);
      }
    }
  };

  // Two stages: the copy of tile t + 1 is in flight while tile t is computed.
  // Copies are issued for tile indices clamped to the last tile, so every
  // step issues the same memory operations and the wait counts stay exact.
  if (n_tiles > 0) {
    const int last = n_tiles - 1;
    TileMap<GPW> mc, mn;  // maps of tiles t and t + 1
    Entries ent;          // block-table entries of tile t + 2
    {
      Entries e;
      fetch_entries<PAGED>(e, a, table, 0, log2bs);
      resolve<PAGED, GPW>(mc, a, e, row_stride, 0, lk, log2bs, wave);
      fetch_entries<PAGED>(e, a, table, min(1, last) * kBN, log2bs);
      resolve<PAGED, GPW>(mn, a, e, row_stride, min(1, last) * kBN, lk, log2bs, wave);
      fetch_entries<PAGED>(ent, a, table, min(2, last) * kBN, log2bs);
    }
    constexpr int kSwK = F8 ? 0 : 1, kSwV = F8 ? 0 : 2, kE = F8 ? 1 : 2;
    issue_rows<D, W, PAGED, kSwK, kE>(mc, kbase, row_stride, 0, lk, k0b, wave, lane);
    issue_rows<D, W, PAGED, kSwV, kE>(mc, vbase, row_stride, 0, lk, v0b, wave, lane);
    bool q_fresh = true;
    auto step = [&](uint8_t* kc, uint8_t* vc, uint8_t* kn, uint8_t* vn, int t) __attribute__((always_inline)) {
      // the copy of t + 1 into the other buffers (freed by the previous step's closing barrier)
      issue_rows<D, W, PAGED, kSwK, kE>(mn, kbase, row_stride, min(t + 1, last) * kBN, lk, kn, wave, lane);
      issue_rows<D, W, PAGED, kSwV, kE>(mn, vbase, row_stride, min(t + 1, last) * kBN, lk, vn, wave, lane);
      __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * kDma));  // tile t (and the q rows) have landed
      __builtin_amdgcn_sched_barrier(0);  // the compiler does not see the copies: keep LDS accesses below
      if constexpr (F8) {
        // this wave's copied rows (8 per pass, one 16-code piece per lane)
        // -> bf16 tiles in the layouts the MFMA reads; V rows of keys that
        // do not exist become zeros
#pragma unroll
        for (int x = 0; x < GPW; ++x) {
          const int r = (wave * GPW + x) * 8 + (lane >> 3), pc = lane & 7;
          const uint4 k8 = *reinterpret_cast<const uint4*>(kc + r * TC::row_bytes + pc * 16);
          const uint4 v8 = *reinterpret_cast<const uint4*>(vc + r * TC::row_bytes + pc * 16);
          const bool ok = (mc.valid >> r) & 1ull;
          const uint4 z = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(kxb + r * T::row_bytes + (((2 * pc) ^ kswz16<D>(r)) << 4)) =
              code8x8_to_bf16x8<KVT>(k8.x, k8.y);
          *reinterpret_cast<uint4*>(kxb + r * T::row_bytes + (((2 * pc + 1) ^ kswz16<D>(r)) << 4)) =
              code8x8_to_bf16x8<KVT>(k8.z, k8.w);
          *reinterpret_cast<uint4*>(vxb + r * T::row_bytes + (((2 * pc) ^ vswz16<D>(r)) << 4)) =
              ok ? code8x8_to_bf16x8<KVT>(v8.x, v8.y) : z;
          *reinterpret_cast<uint4*>(vxb + r * T::row_bytes + (((2 * pc + 1) ^ vswz16<D>(r)) << 4)) =
              ok ? code8x8_to_bf16x8<KVT>(v8.z, v8.w) : z;
        }
      } else {
        zero_rows<D, W>(mc.valid, vc, wave, lane);
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      if (q_fresh) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            qf[cb][ks] = qvalid[cb] ? make_uint4(qf[cb][ks].x ^ q_sign, qf[cb][ks].y ^ q_sign,
                                                 qf[cb][ks].z ^ q_sign, qf[cb][ks].w ^ q_sign)
                                    : make_uint4(0u, 0u, 0u, 0u);
        q_fresh = false;
      }
      if constexpr (F8) compute(kxb, vxb, t * kBN, mc.valid, mc.blocks_ok);
      else compute(kc, vc, t * kBN, mc.valid, mc.blocks_ok);
      mc = mn;
      resolve<PAGED, GPW>(mn, a, ent, row_stride, min(t + 2, last) * kBN, lk, log2bs, wave);
      fetch_entries<PAGED>(ent, a, table, min(t + 3, last) * kBN, log2bs);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();  // every wave is done with tile t's buffers
      return t < last;
    };
    for (int t = 0;; t += 2) {
      if (!step(k0b, v0b, k1b, v1b, t)) break;
      if (!step(k1b, v1b, k0b, v0b, t + 1)) break;
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // copies past the last tile land before LDS is released
  }

  // normalise and store: lane holds O^T rows 16 db + 4 (lane / 16) + i of its column
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = sum_quarters(l[cb]);
    if (!qvalid[cb]) continue;
    const float inv = lt > 0.0f ? (F8 ? a.v_scale[g] : 1.0f) / lt : 0.0f;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)(q_start + qrow[cb]) * a.num_heads + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint32_t w0 = pack_bf16x2(o[cb][db][0] * inv, o[cb][db][1] * inv);
      const uint32_t w1 = pack_bf16x2(o[cb][db][2] * inv, o[cb][db][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * db + 4 * grp4) = make_uint2(w0, w1);
    }
  }
}

template <int KVT, int D>
struct PrefillLds {  // LDS of prefill16_body, in bytes (each buffer 1 KiB-aligned)
  static constexpr bool F8 = scaled8(KVT);
  static constexpr int copied = Tile<D, 4, F8 ? 1 : 2>::bytes;  // one K or V tile as copied
  static constexpr int bf16 = F8 ? Tile<D, 4>::bytes : 1024;    // one dequantised tile
  static constexpr int bytes = 4 * copied + 2 * bf16;
};

template <int KVT, int D, bool PAGED, int CB>
__global__ __launch_bounds__(512 / CB, 4 / CB) void prefill16_kernel(PrefillArgs a, int q_tiles) {
  // The body is device code only: the host pass of the compiler, which
  // needs no more than the kernel's signature, rejects some of its template
  // instantiations when both one-byte cache types are built in one file.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool F8 = scaled8(KVT);
  using TC = Tile<D, 8 / CB, F8 ? 1 : 2>;
  using T = Tile<D, 8 / CB>;
  // copy targets (two stages); with one-byte caches, bf16 tiles dequantised from them
  __shared__ __attribute__((aligned(1024))) uint8_t k0b[TC::bytes], v0b[TC::bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k1b[TC::bytes], v1b[TC::bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t kxb[F8 ? T::bytes : 16], vxb[F8 ? T::bytes : 16];
  prefill16_body<KVT, D, PAGED, CB>(a, q_tiles, blockIdx.x, k0b, v0b, k1b, v1b, kxb, vxb);
#endif
}

template <int KVT, int D>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  const int q_tiles = (a.max_seqlen_q + 127) / 128;
  const int64_t grid = work_grid(q_tiles, a.batch, a.num_heads, a.num_kv_heads);
  if (grid > 0x7fffffff / 2) return hipErrorInvalidValue;
  constexpr int CB = PKV_PREFILL_CB;
  const dim3 block(512 / CB);
  if constexpr (scaled8(KVT)) {
    hipLaunchKernelGGL((prefill16_kernel<KVT, D, true, CB>), dim3((unsigned)grid), block, 0, stream, a, q_tiles);
  } else if (a.block_table != nullptr) {
    hipLaunchKernelGGL((prefill16_kernel<kBF16, D, true, CB>), dim3((unsigned)grid), block, 0, stream, a, q_tiles);
  } else {
    hipLaunchKernelGGL((prefill16_kernel<kBF16, D, false, CB>), dim3((unsigned)grid), block, 0, stream, a, q_tiles);
  }
  return hipGetLastError();
}

}  // namespace dma

template <int KVT, int D>
hipError_t launch_mfma(const PrefillArgs& a, hipStream_t stream) {
  const int q_tiles = (a.max_seqlen_q + BM - 1) / BM;
  const int64_t grid = work_grid(q_tiles, a.batch, a.num_heads, a.num_kv_heads);
  if (grid > 0x7fffffff / 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<KVT, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a, q_tiles);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const PrefillArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.total_q * a.num_heads;
  hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_varlen_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.q_dtype == kF32) {
    if (a.head_dim == 64) return launch_f32<64>(a, stream);
    return launch_f32<128>(a, stream);
  }
  if (a.kv_dtype == kBF16) {
    if (a.head_dim == 64) return dma::launch<kBF16, 64>(a, stream);
    return dma::launch<kBF16, 128>(a, stream);
  }
  // one-byte caches are paged (the entry point requires a block table)
  if (a.kv_dtype == kI8) {
    if (a.head_dim == 64) return launch_mfma<kI8, 64>(a, stream);
    return dma::launch<kI8, 128>(a, stream);
  }
  if (a.head_dim == 64) return launch_mfma<kFP8, 64>(a, stream);
  return dma::launch<kFP8, 128>(a, stream);
}

}  // namespace pkv
