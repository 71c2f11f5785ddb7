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
// Matrix-core kernel (prefill_kernel: bf16 queries over bf16, fp8 or int8
// caches, head_dim 64 or 128), designed around three gfx950 facts measured
// on the part: a v_mfma_f32_32x32x16_bf16 keeps the matrix core busy 32
// clocks and leaves the issuing wave about half of them for vector work (the
// 16x16x32 form leaves none); v_exp_f32 issues at half rate; and LDS serves
// about 130-165 bytes a clock to a CU.
// * Columns.  The 32 columns of a wave's matrix products are (query row,
//   q head) pairs: the G q heads that share a KV head sit side by side
//   (column c = row c / G, head c % G), so one K/V tile serves all of them,
//   a workgroup (4 waves, 128 columns) covers 128 / G query rows, and the
//   causal diagonal crosses fewer rows per tile.  At head_dim 64 with bf16
//   caches a wave takes two such 32-column blocks (256 columns a
//   workgroup), and each K and V operand it reads from LDS feeds both:
//   the LDS reads per flop, which limit the kernel, are halved.
// * Per 64-key tile and wave: S^T = K Q^T (keys x columns, 16 MFMAs at
//   head_dim 128), so each lane holds 16 scores of one column per 32-key
//   block and its partner lane (l ^ 32) the other 16: the row max needs one
//   v_permlane32_swap.  P^T, packed to bf16 in place, is the B operand of
//   O^T += V^T P^T as it stands: the transposed V reads
//   (ds_read_b64_tr_b16) put the same keys in the same k-slots.
// * Online softmax in the log2 domain with a lazy running max (moved, and
//   the output rescaled, only when a column's max grows by more than 2^8);
//   row sums accumulate the bf16-rounded p the MFMA consumes.  Masks are
//   applied only on tiles that cross the causal diagonal, the sequence end
//   or an invalid block.
// * K and V tiles go HBM -> LDS by DMA (buffer loads with the lds bit, no
//   registers), each wave copying its 16 keys through one buffer
//   descriptor per copy instruction whose range ends at the last key that
//   exists, so rows past the sequence (and blocks outside the pool) land as
//   zeros.  XOR permutations of 16-byte pieces keep the K operand reads and
//   the transposed V reads free of bank conflicts.  Two stages: the copy of
//   tile t + 1 is in flight while tile t is computed, one barrier per tile.
//   One-byte caches are copied as codes and each wave dequantises its own
//   rows (exact: every E4M3 and int8 value is a bf16) into bf16 tiles; the
//   K scale folds into the logit scale, the V scale into the output.
// * Work items are (request, KV head, query tile), tiles numbered from the
//   end of the request (tile 0 = the last rows, which see the most keys), and
//   dealt so that the pairs (request, KV head) go round-robin over the 8
//   XCDs: the tiles sharing a pair's K/V share one L2, and the longest tiles
//   of every request run first.  A persistent grid (two workgroups a CU)
//   takes the items at run time from one counter per XCD, then from the
//   other XCDs' counters once its own runs dry: CUs and XCDs run at
//   different speeds under this load, and a fixed deal of the items leaves
//   the fast ones idle at the end.  The counters are a small static array,
//   one set per stream, cleared by a fill kernel before each launch.
//
// fp32 kernel: a plain per-row wave kernel (lanes over head_dim), kept for
// fp32 accuracy checks; it is not tuned.

#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_internal.h"
#include "work_queue.hpp"


namespace pkv {
namespace {

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

}  // namespace

namespace pf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

constexpr int kBN = 64;      // keys per tile
constexpr int kWaves = 4;    // waves per workgroup
constexpr int kCols = 32;    // matrix columns per wave: (query row, q head) pairs
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerWave = kBN / kWaves;  // rows of each tile one wave copies
constexpr float kRescaleBits = 8.0f;        // lazy-max threshold (log2 domain)
constexpr int kBufferWord3 = 0x00020000;    // raw buffer descriptor, dword 3
constexpr int kWaitVm0 = 0x0f70;            // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xc07f;          // s_waitcnt lgkmcnt(0)

// One 64-key tile of K or V with E bytes per element, and how the copy
// instructions cover it: each lane moves dma_bytes, so one instruction
// fills rows_per_dma whole rows (never more than 8, so never more than a
// block: block sizes are at least 8).
template <int D, int E>
struct TileGeo {
  static constexpr int row_bytes = D * E;
  static constexpr int bytes = kBN * row_bytes;
  static constexpr int dma_bytes = row_bytes >= 128 ? 16 : 4;
  static constexpr int lanes_per_row = row_bytes / dma_bytes;
  static constexpr int rows_per_dma = 64 / lanes_per_row;
  static constexpr int dma_per_wave = kKeysPerWave / rows_per_dma;
  static_assert(rows_per_dma <= 8 && dma_per_wave >= 1, "copy geometry");
};

// LDS of one workgroup: two stages of K and V tiles as copied, and for
// one-byte caches the bf16 tiles dequantised from them.
template <int KVT, int D>
struct Lds {
  static constexpr bool one_byte = scaled8(KVT);
  using C = TileGeo<D, one_byte ? 1 : 2>;
  using B = TileGeo<D, 2>;
  static constexpr int stage = 2 * C::bytes;
  static constexpr int bf16 = one_byte ? 2 * B::bytes : 0;
  static constexpr int bytes = 2 * stage + bf16;
};

// 16-byte piece permutations of the bf16 tiles (piece i of row r is stored
// at position i ^ swz(r)).  K is read as 32 consecutive rows x one piece per
// 16 lanes, V transposed as 4 consecutive rows x 32 bytes per 16 lanes: with
// these each group of lanes the LDS serves together touches distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Work item of hardware workgroup hw: request b, KV head g, query tile qt
// (counted from the end of the request).  Workgroup i runs on XCD i % 8;
// pair p = b * Hkv + g lives on XCD p % 8.  Returns false for the padding
// workgroups of XCDs with fewer pairs.
struct Item {
  int b, g, qt;
};

__device__ __forceinline__ bool item_of(int hw, int q_tiles, int pairs, int num_kv_heads, Item& it) {
  const int x = hw & 7, j = hw >> 3;
  const int px = (pairs - x + 7) >> 3;  // pairs on XCD x
  if (j >= q_tiles * px) return false;
  it.qt = j / px;
  const int p = x + 8 * (j - it.qt * px);
  it.b = p / num_kv_heads;
  it.g = p - it.b * num_kv_heads;
  return true;
}

// 32-column blocks per wave.  With two, each K and V operand read from LDS
// serves two MFMAs, half the LDS reads per flop: bf16 caches at head_dim 64
// (240 VGPRs, still two workgroups a CU).  Head_dim 128 (two blocks would
// need about 300 registers a lane) and one-byte caches (their dequantised
// tiles, and the mixed-step kernel's decode workers beside them) keep one.
template <int KVT, int D>
__host__ __device__ constexpr int col_blocks() {
  return (scaled8(KVT) || D != 64) ? 1 : 2;
}

__host__ __forceinline__ int rows_per_item(int group, int cb) { return kWaves * kCols * cb / group; }

__host__ __forceinline__ int tiles_of(int max_seqlen_q, int group, int cb) {
  const int r = rows_per_item(group, cb);
  return (max_seqlen_q + r - 1) / r;
}

// Grid for item_of(): 8 XCDs x the largest per-XCD share.
__host__ __forceinline__ int64_t grid_of(int q_tiles, int batch, int num_kv_heads) {
  const int64_t pairs = (int64_t)batch * num_kv_heads;
  return 8 * (int64_t)q_tiles * ((pairs + 7) / 8);
}

// Query and key rows of request b as the kernel uses them (the clamps keep
// every access inside the buffers whatever the device metadata holds):
// query rows [q_start, q_start + lq) of q/out, lk keys.
struct Request {
  int q_start, lq, k_start, lk;
};

template <bool PAGED>
__device__ __forceinline__ Request request(const PrefillArgs& a, int b) {
  const const_i32_ptr cq = (const_i32_ptr)a.cu_seqlens_q, ck = (const_i32_ptr)a.cu_seqlens_k;
  Request r;
  r.q_start = cq[b];
  r.lq = cq[b + 1] - r.q_start;
  if (r.lq > a.max_seqlen_q) r.lq = a.max_seqlen_q;
  if (r.q_start < 0 || r.q_start >= a.total_q) r.lq = 0;
  else if (r.lq > a.total_q - r.q_start) r.lq = a.total_q - r.q_start;
  if (r.lq < 0) r.lq = 0;
  r.k_start = ck[b];
  r.lk = ck[b + 1] - r.k_start;
  if (r.lk < 0) r.lk = 0;
  if constexpr (PAGED) {
    r.lk = min(r.lk, a.max_blocks_per_seq * a.block_size);
  } else {
    if (r.k_start < 0 || r.k_start > a.total_k) r.lk = 0;
    else if (r.lk > a.total_k - r.k_start) r.lk = a.total_k - r.k_start;
  }
  return r;
}

// Work items are handed out at run time: a persistent grid (the
// workgroups that fit on the GPU) takes them from one counter per XCD, in
// item_of() order on that XCD (the last query tiles of every request
// first, so the longest items start first); a workgroup whose XCD has none
// left takes the other XCDs' items.  Workgroups on slower CUs or XCDs simply
// take fewer items, and no workgroup slot waits for the dispatcher.  The
// counters are the stream's prefill set of the work-queue array, cleared on
// that stream just before each launch.

// The next work item (item_of() number: item j of XCD xx is 8 j + xx) for a
// workgroup on XCD x, or -1 when every counter is past its XCD's items.
// `dry` marks the counters this workgroup found empty.  One lane calls it.
__device__ __forceinline__ int next_item(uint32_t* queues, int x, int q_tiles, int pairs, uint32_t& dry) {
#pragma unroll 1
  for (int d = 0; d < 8; ++d) {
    const int xx = (x + d) & 7;
    if ((dry >> xx) & 1u) continue;
    const uint32_t n = (uint32_t)q_tiles * (uint32_t)((pairs - xx + 7) >> 3);  // items on XCD xx
    const uint32_t j = atomicAdd(queues + xx * wq::kStride, 1u);
    if (j < n) return (int)(8 * j + xx);
    dry |= 1u << xx;
  }
  return -1;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ uint2 read_tr(const uint8_t* p) {
  const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
  return __builtin_bit_cast(uint2, x);
}

// Two fp32 -> two bf16 (round to nearest even) in one word.
__device__ __forceinline__ uint32_t cvt2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2v_t));
}

// Eight one-byte cache codes (E4M3 or int8; two words) -> eight bf16 (four
// words), exact.
template <int KVT>
__device__ __forceinline__ uint4 code8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(code8x2_to_bf16x2<KVT, false>(w0), code8x2_to_bf16x2<KVT, true>(w0),
                    code8x2_to_bf16x2<KVT, false>(w1), code8x2_to_bf16x2<KVT, true>(w1));
}

// An LDS address whose object the compiler cannot see.  The kernel waits
// for its copies itself (s_waitcnt, then a barrier); the compiler does not
// track copies made through such an address, where it would otherwise make
// LDS reads wait for every copy in flight.
__device__ __forceinline__ lds_void_t* lds_opaque(uint8_t* p) {
  uint32_t x = (uint32_t)(uintptr_t)(lds_void_t*)p;
  asm volatile("" : "+s"(x));
  return (lds_void_t*)(uintptr_t)x;
}

// Where this wave's 16 rows of a tile come from, per 8-row half (block
// sizes are at least 8, so a half never straddles a block): the cache row
// of the half's first key and the bytes its copy descriptor covers, ending
// at the last key that exists (0 when none does or the block is outside the
// pool), and which halves hold keys in a block outside the pool.
struct Halves {
  int64_t row0[2];
  int range[2];
  uint32_t bad;
};

// Block-table entries of this wave's two halves of a tile (scalar loads
// through the constant address space: the table is not written while a
// kernel runs), fetched a tile ahead of their use.
struct Entries {
  int32_t e[2];
};

template <bool PAGED>
__device__ __forceinline__ void fetch_entries(Entries& en, const int32_t* table, int key0, int log2bs, int max_blocks,
                                              int wave) {
  if constexpr (PAGED) {
    const const_i32_ptr t = (const_i32_ptr)table;
    const int k = key0 + kKeysPerWave * wave;
    en.e[0] = t[min(k >> log2bs, max_blocks - 1)];
    en.e[1] = t[min((k + 8) >> log2bs, max_blocks - 1)];
  }
}

template <bool PAGED>
__device__ __forceinline__ void locate(Halves& hv, const Entries& en, int key0, int lk, int log2bs, int num_blocks,
                                       int wave, int row_stride, int row_bytes) {
  hv.bad = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = key0 + kKeysPerWave * wave + 8 * h;
    int n = lk - key;  // keys of the half that exist
    n = n < 0 ? 0 : (n > 8 ? 8 : n);
    bool ok = n > 0;
    if constexpr (PAGED) {
      const int e = en.e[h];
      const bool in_pool = (uint32_t)e < (uint32_t)num_blocks;
      hv.bad |= (ok && !in_pool) ? (1u << h) : 0u;
      ok = ok && in_pool;
      hv.row0[h] = ok ? (((int64_t)e) << log2bs) + (key & ((1 << log2bs) - 1)) : 0;
    } else {
      hv.row0[h] = ok ? key : 0;
    }
    hv.range[h] = __builtin_amdgcn_readfirstlane(ok ? (n - 1) * row_stride + row_bytes : 0);
  }
}

// A buffer descriptor for the bytes [p, p + range).  Every input is uniform;
// readfirstlane keeps the descriptor in scalar registers (no waterfall loop
// around the copy).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* p, int range) {
  const uint64_t addr = (uint64_t)(uintptr_t)p;
  const uint64_t ua = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)ua, 0, range, kBufferWord3);
}

// Copy this wave's 16 rows of the K or V tile (from base, the tensor's
// first row of this KV head) into dst, a tile of the layout C.  voff: per
// copy instruction, this lane's byte offset from its half's first row.
template <typename C>
__device__ __forceinline__ void copy_rows(const uint8_t* base, int64_t row_stride, const Halves& hv, int wave,
                                          uint8_t* dst, const int (&voff)[C::dma_per_wave]) {
  const __amdgpu_buffer_rsrc_t r0 = rsrc(base + hv.row0[0] * row_stride, hv.range[0]);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(base + hv.row0[1] * row_stride, hv.range[1]);
#pragma unroll
  for (int i = 0; i < C::dma_per_wave; ++i) {
    const int r = kKeysPerWave * wave + i * C::rows_per_dma;  // the instruction's first row in the tile
    __builtin_amdgcn_raw_ptr_buffer_load_lds((i * C::rows_per_dma) < 8 ? r0 : r1, lds_opaque(dst + r * C::row_bytes),
                                             C::dma_bytes, voff[i], 0, 0, 0);
  }
}

// The workgroup body for work item hw, with its LDS passed in (two stages
// of K and V tiles as copied, s0 and s1, each Lds<KVT, D>::stage bytes; for
// one-byte caches the bf16 tiles, bf; all 1 KiB-aligned; and two flag words,
// one per stage, in which each wave marks the 8-key groups of its rows that
// lie in blocks outside the pool), so that a launch that serves other work
// too can run it.  Separate LDS objects let
// the compiler see that the copy into one stage does not touch the other.
template <int KVT, int D, bool PAGED>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, const Item& it, uint8_t* s0, uint8_t* s1,
                                             uint8_t* bf, uint32_t* flags) {
  constexpr bool ONE = scaled8(KVT);
  static_assert(!ONE || PAGED, "one-byte caches are paged");
  constexpr int CB = col_blocks<KVT, D>();  // 32-column blocks per wave
  using L = Lds<KVT, D>;
  using C = typename L::C;  // tiles as copied
  using B = typename L::B;  // bf16 tiles the matrix cores read
  constexpr int KS = D / 16;  // k-steps of S^T = K Q^T over head_dim
  constexpr int DB = D / 32;  // 32-dim blocks of O^T
  constexpr int RB = B::row_bytes;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;

  const int G = a.num_heads / a.num_kv_heads;  // a power of two (checked on the host)
  const int lg = __builtin_ctz(G);
  const int rpw = (kCols * CB) >> lg;  // query rows per wave
  const int rwg = rpw * kWaves;  // per workgroup

  const int b = it.b, g = it.g;
  const Request rq = request<PAGED>(a, b);
  const int q_start = rq.q_start, lq = rq.lq, k_start = rq.k_start, lk = rq.lk;
  const int row_end = lq - it.qt * rwg;  // one past the item's last row
  if (row_end <= 0) return;
  const int r0 = row_end - rwg;          // the item's first row (negative: rows that do not exist)
  const int offset = lk - lq;  // bottom-right causal alignment
  int key_end = a.causal ? min(lk, row_end + offset) : lk;
  if (key_end < 0) key_end = 0;
  const int n_tiles = (key_end + kBN - 1) / kBN;

  // this lane's column in column block cb: query row qrow[cb], q head
  // `head` (column 32 cb + col of the wave)
  const int wr0 = r0 + rpw * wave;  // the wave's first row
  int qrow[CB];
  bool qvalid[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    qrow[cb] = wr0 + ((kCols * cb + col) >> lg);
    qvalid[cb] = qrow[cb] >= 0;
  }
  const int head = g * G + (col & (G - 1));
  const bool wave_rows = wr0 + rpw > 0;  // the wave has a row that exists
  // keys [0, full_end) are visible to every column of the wave, keys past
  // any_end to none; lim: this column's visible keys
  const int lo_row = max(wr0, 0);
  const int full_end = a.causal ? min(lk, lo_row + offset + 1) : lk;
  const int any_end = a.causal ? min(lk, wr0 + rpw + offset) : lk;
  int lim[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) lim[cb] = a.causal ? min(lk, qrow[cb] + offset + 1) : lk;

  // The row max is taken over unscaled scores, which needs scale > 0: a
  // negative scale is applied as |scale| to -q (bf16 negation is exact), a
  // zero scale as 1e-30 (every logit then rounds to exactly 0 in the
  // exponent, as with scale 0, while masked keys stay at -inf).  With
  // one-byte caches the K scale folds into the logit scale and the V scale
  // into the output.
  const float sc = ONE ? a.softmax_scale * ((const __attribute__((address_space(4))) float*)a.k_scale)[g]
                       : a.softmax_scale;
  const uint32_t q_sign = sc < 0.0f ? 0x80008000u : 0u;
  const float scale = fmaxf(fabsf(sc) * kLog2e, 1e-30f);

  // q as the B operand of S^T = K Q^T: lane holds column `col`, head_dim
  // elements 16 ks + 8 half .. + 7 (rows that do not exist read row 0 and
  // are zeroed once the first tile has landed, so that the q loads and the
  // first copy are in flight together)
  uint4 qf[CB][KS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)(q_start + (qvalid[cb] ? qrow[cb] : 0)) * a.num_heads + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[cb][ks] = *reinterpret_cast<const uint4*>(qp + ks * 16);
  }

  // LDS read offsets.  K (A operand of S^T): row 32 kb + col, piece 2 ks + half.
  // V^T (A operand of O^T, transposed reads): within each 16-lane group,
  // lane c supplies key 4 half + c / 4 (+ 16 ks + 8 x) and head_dim elements
  // 32 db + 16 ((lane / 16) & 1) + 4 (c % 4) .. + 3, and receives element
  // 32 db + lane % 32 of those 4 keys.
  // (piece (2 ks + half) ^ swz = (2 ks) ^ (swz & ~1) plus bit 0 (half ^
  // swz & 1), so the offset of k-step ks is kl ^ (ks << 5): one register)
  const int kl = col * RB + (((swz_k<D>(col) & ~1) | (half ^ (swz_k<D>(col) & 1))) << 4);
  int voff[DB];
  {
    const int c = lane & 15, gi = (lane >> 4) & 1;
    const int key = 4 * half + (c >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int byte = 64 * db + 32 * gi + 8 * (c & 3);
      voff[db] = key * RB + ((((byte >> 4) ^ swz_v<D>(key))) << 4) + (byte & 15);
    }
  }

  // copy geometry: per lane and copy instruction, the byte offset from the
  // first row of the instruction's 8-row half (bf16 tiles: with the piece
  // permutations)
  const int64_t row_stride = (int64_t)a.num_kv_heads * C::row_bytes;
  int dk[C::dma_per_wave], dv[C::dma_per_wave];
  {
    const int lrow = lane / C::lanes_per_row, slot = lane % C::lanes_per_row;
#pragma unroll
    for (int i = 0; i < C::dma_per_wave; ++i) {
      const int r = kKeysPerWave * wave + i * C::rows_per_dma + lrow;
      const int pk = ONE ? slot : (slot ^ swz_k<D>(r));
      const int pv = ONE ? slot : (slot ^ swz_v<D>(r));
      const int hr = (i * C::rows_per_dma) % 8 + lrow;  // row within the 8-row half
      dk[i] = hr * (int)row_stride + pk * C::dma_bytes;
      dv[i] = hr * (int)row_stride + pv * C::dma_bytes;
    }
  }
  const uint8_t* kbase = a.k + g * C::row_bytes + (PAGED ? 0 : (int64_t)k_start * row_stride);
  const uint8_t* vbase = a.v + g * C::row_bytes + (PAGED ? 0 : (int64_t)k_start * row_stride);
  const int32_t* table = PAGED ? a.block_table + (int64_t)b * a.max_blocks_per_seq : nullptr;
  const int log2bs = PAGED ? __builtin_ctz(a.block_size) : 0;

  f32x16_t o[CB][DB];
  float m[CB], l[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[cb][db] = f32x16_t{};
    m[cb] = kNegBig;
    l[cb] = 0.0f;
  }

  // One tile: S^T = K Q^T (two 32-key blocks), after_k() (the caller's
  // work once the K operands are read), mask (only on tiles that cross the
  // causal diagonal or the sequence end, or hold keys in blocks outside the
  // pool: `bad` bit 8 w + x for wave w's half x), the column max, lazy
  // running max, p = exp2(s scale - m) packed to bf16 as the B operands of
  // O^T += V^T P^T, row sums of the packed p.
  auto compute = [&](const uint8_t* kt, const uint8_t* vt, int key0, uint32_t bad,
                     auto&& after_k) __attribute__((always_inline)) {
    // each K (and V) operand read serves the CB column blocks
    f32x16_t sv[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) sv[cb][0] = sv[cb][1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 kf = *reinterpret_cast<const uint4*>(kt + (kl ^ (ks << 5)) + kb * 32 * RB);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          sv[cb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[cb][ks]), sv[cb][kb], 0, 0, 0);
      }
    after_k();  // the next tile's copies
    // register i of block kb holds key 32 kb + 8 (i / 4) + 4 half + i % 4
    if (key0 + kBN > full_end || bad != 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int lim_rel = lim[cb] - key0 - 4 * half;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int grp = 4 * kb + (i >> 2);  // 8-key group, copied by wave grp / 2
            const bool skip =
                32 * kb + 8 * (i >> 2) + (i & 3) >= lim_rel || ((bad >> (8 * (grp >> 1) + (grp & 1))) & 1u);
            sv[cb][kb][i] = skip ? -INFINITY : sv[cb][kb][i];
          }
      }
    }
    // P^T as bf16 B operands, one per 16-key k-step: the lane's own scores
    uint4 pb[CB][4];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float x = fmaxf(sv[cb][0][0], sv[cb][0][1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) x = fmaxf(x, sv[cb][0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) x = fmaxf(x, sv[cb][1][i]);
      const float mx = max_halves(x) * scale;
      // lazy running max: move it (and rescale) only when it grows by > 2^8
      if (__builtin_amdgcn_ballot_w64(mx > m[cb] + kRescaleBits) != 0) {
        const float mn = fmaxf(m[cb], mx);
        const float alpha = fast_exp2(m[cb] - mn);
        m[cb] = mn;
        l[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[cb][db] *= alpha;
      }
      const float neg_m = -m[cb];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1, i0 = 8 * (ks & 1);
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(sv[cb][kb][i0 + j], scale, neg_m));
        pb[cb][ks] = make_uint4(cvt2_bf16(p[0], p[1]), cvt2_bf16(p[2], p[3]), cvt2_bf16(p[4], p[5]),
                                cvt2_bf16(p[6], p[7]));
        l[cb] = dot2_bf16(pb[cb][ks].x, 0x3f803f80u, l[cb]);
        l[cb] = dot2_bf16(pb[cb][ks].y, 0x3f803f80u, l[cb]);
        l[cb] = dot2_bf16(pb[cb][ks].z, 0x3f803f80u, l[cb]);
        l[cb] = dot2_bf16(pb[cb][ks].w, 0x3f803f80u, l[cb]);
      }
    }
    // O^T += V^T P^T; V^T operands by transposed reads (keys 16 ks + 8 x +
    // 4 half + c / 4 of each 16-lane group)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint2 lo = read_tr(vt + voff[db] + 16 * ks * RB);
        const uint2 hi = read_tr(vt + voff[db] + (16 * ks + 8) * RB);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          o[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                                              as_bf16x8(pb[cb][ks]), o[cb][db], 0, 0, 0);
      }
  };

  uint8_t* const bk = bf;  // dequantised tiles (one-byte caches)
  uint8_t* const bv = ONE ? bf + B::bytes : nullptr;
  if (n_tiles > 0) {
    const int rs32 = (int)row_stride;
    Entries en;  // block-table entries of tile t + 1 (fetched a tile ahead)
    Halves hv;
    fetch_entries<PAGED>(en, table, 0, log2bs, a.max_blocks_per_seq, wave);
    locate<PAGED>(hv, en, 0, lk, log2bs, a.num_blocks, wave, rs32, C::row_bytes);
    copy_rows<C>(kbase, row_stride, hv, wave, s0, dk);
    copy_rows<C>(vbase, row_stride, hv, wave, s0 + C::bytes, dv);
    if constexpr (PAGED) reinterpret_cast<uint8_t*>(flags)[wave] = (uint8_t)hv.bad;
    fetch_entries<PAGED>(en, table, kBN, log2bs, a.max_blocks_per_seq, wave);
    // the q rows were loaded before the copies: wait for them alone
    __builtin_amdgcn_s_waitcnt(kWaitVm0 | (2 * C::dma_per_wave));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[cb][ks] = qvalid[cb] ? make_uint4(qf[cb][ks].x ^ q_sign, qf[cb][ks].y ^ q_sign, qf[cb][ks].z ^ q_sign,
                                             qf[cb][ks].w ^ q_sign)
                                : make_uint4(0u, 0u, 0u, 0u);
    // Each step: wait for tile t, (one-byte caches: dequantise this wave's
    // rows of tile t), compute tile t if the wave has keys in it, locating
    // and copying tile t + 1 after the score products, fetch the block-table
    // entries of tile t + 2.
    auto step = [&](int t, bool work, uint8_t* cur, uint8_t* nxt, uint32_t* fcur, uint32_t* fnxt)
                    __attribute__((always_inline)) {
      // this wave's copies of tile t and its flag byte have landed
      __builtin_amdgcn_s_waitcnt(0x0070);
      __builtin_amdgcn_sched_barrier(0);
      // every wave's copies of tile t landed (bf16) / every wave is done
      // with tile t - 1, whose buffers receive tile t + 1 (and, one-byte,
      // tile t's dequantised rows) next
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // bit 8 w + x: wave w's half x of tile t lies in a block outside the
      // pool (read now, used after the copies are issued)
      const uint32_t bad_raw = (PAGED && work) ? *fcur : 0u;
      // Locating and copying tile t + 1: a wave with keys in tile t does it
      // from inside compute(), once its score products have read their K
      // operands, so that the products start sooner and the copies' writes
      // into LDS meet the softmax and the P.V reads rather than the K reads
      // (a wave without keys here does it now).
      auto copies = [&]() __attribute__((always_inline)) {
        if (t + 1 < n_tiles) {
          locate<PAGED>(hv, en, (t + 1) * kBN, lk, log2bs, a.num_blocks, wave, rs32, C::row_bytes);
          copy_rows<C>(kbase, row_stride, hv, wave, nxt, dk);
          copy_rows<C>(vbase, row_stride, hv, wave, nxt + C::bytes, dv);
          if constexpr (PAGED) reinterpret_cast<uint8_t*>(fnxt)[wave] = (uint8_t)hv.bad;
        }
      };
      if (!work) copies();
      if constexpr (ONE) {
        // this wave's 16 copied rows of K and V -> bf16 tiles (16 codes per
        // lane and pass; rows that were not copied hold zeros)
        constexpr int PPR = D / 16;  // 16-code pieces per row
#pragma unroll
        for (int x = 0; x < kKeysPerWave * PPR / 64; ++x) {
          const int idx = lane + 64 * x;
          const int r = kKeysPerWave * wave + idx / PPR, pc = idx % PPR;
          const uint4 k8 = *reinterpret_cast<const uint4*>(cur + r * C::row_bytes + pc * 16);
          const uint4 v8 = *reinterpret_cast<const uint4*>(cur + C::bytes + r * C::row_bytes + pc * 16);
          *reinterpret_cast<uint4*>(bk + r * RB + (((2 * pc) ^ swz_k<D>(r)) << 4)) = code8x8_to_bf16x8<KVT>(k8.x, k8.y);
          *reinterpret_cast<uint4*>(bk + r * RB + (((2 * pc + 1) ^ swz_k<D>(r)) << 4)) =
              code8x8_to_bf16x8<KVT>(k8.z, k8.w);
          *reinterpret_cast<uint4*>(bv + r * RB + (((2 * pc) ^ swz_v<D>(r)) << 4)) = code8x8_to_bf16x8<KVT>(v8.x, v8.y);
          *reinterpret_cast<uint4*>(bv + r * RB + (((2 * pc + 1) ^ swz_v<D>(r)) << 4)) =
              code8x8_to_bf16x8<KVT>(v8.z, v8.w);
          __builtin_amdgcn_sched_barrier(0);  // one piece at a time: few registers next to the tile state
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();  // every wave's rows of tile t are in the bf16 tiles
        __builtin_amdgcn_sched_barrier(0);
      }
      if (work) {
        const uint8_t* kt = ONE ? bk : cur;
        const uint8_t* vt = ONE ? bv : cur + C::bytes;
        const uint32_t bad = (uint32_t)__builtin_amdgcn_readfirstlane((int)bad_raw);
        compute(kt, vt, t * kBN, bad, copies);
      }
      // the entries of tile t + 2, after this tile's LDS reads (scalar loads
      // share a wait counter with LDS reads)
      __builtin_amdgcn_sched_barrier(0);
      fetch_entries<PAGED>(en, table, (t + 2) * kBN, log2bs, a.max_blocks_per_seq, wave);
    };
    // tiles [0, n_work) hold keys of this wave's rows; the rest it only
    // copies (two tiles per pass: the stage each tile uses is fixed in the
    // code)
    const int n_work = wave_rows ? min(n_tiles, (max(any_end, 0) + kBN - 1) / kBN) : 0;
    uint32_t* const f0 = flags;
    uint32_t* const f1 = flags + 1;
    int t = 0;
    for (; t + 1 < n_work; t += 2) {
      step(t, true, s0, s1, f0, f1);
      step(t + 1, true, s1, s0, f1, f0);
    }
    if (t < n_work) {
      step(t, true, s0, s1, f0, f1);
      ++t;
      if (t < n_tiles) {
        step(t, false, s1, s0, f1, f0);
        ++t;
      }
    }
    for (; t + 1 < n_tiles; t += 2) {
      step(t, false, s0, s1, f0, f1);
      step(t + 1, false, s1, s0, f1, f0);
    }
    if (t < n_tiles) step(t, false, s0, s1, f0, f1);
  }

  // normalise and store: lane holds O^T elements 32 db + 8 j + 4 half + i of
  // its column (register 4 j + i)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = sum_halves(l[cb]);
    if (qvalid[cb]) {
      const float inv = lt > 0.0f ? (ONE ? ((const __attribute__((address_space(4))) float*)a.v_scale)[g] : 1.0f) / lt
                                  : 0.0f;
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)(q_start + qrow[cb]) * a.num_heads + head) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(op + 32 * db + 8 * j + 4 * half) =
              make_uint2(cvt2_bf16(o[cb][db][4 * j] * inv, o[cb][db][4 * j + 1] * inv),
                         cvt2_bf16(o[cb][db][4 * j + 2] * inv, o[cb][db][4 * j + 3] * inv));
    }
  }
}

// The work items of one workgroup: with a counter set (slot >= 0), items
// from the queues until they are empty; else work item `hw` alone.  `item`:
// an int of LDS to share the next item through.
template <int KVT, int D, bool PAGED>
__device__ __forceinline__ void prefill_items(const PrefillArgs& a, int q_tiles, int slot, int hw, uint8_t* s0,
                                              uint8_t* s1, uint8_t* bf, uint32_t* flags, int* item) {
  const int pairs = a.batch * a.num_kv_heads;
  if (slot < 0) {
    Item it;
    if (item_of(hw, q_tiles, pairs, a.num_kv_heads, it)) prefill_body<KVT, D, PAGED>(a, it, s0, s1, bf, flags);
    return;
  }
  uint32_t* const queues = wq::counters(slot);
  const int x = blockIdx.x & 7;  // this workgroup's XCD
  uint32_t dry = 0;
  for (;;) {  // ends once every counter is past its XCD's items
    if (threadIdx.x == 0) *item = next_item(queues, x, q_tiles, pairs, dry);
    __syncthreads();
    const int next = *item;
    __syncthreads();  // every wave has read it before lane 0 writes the next
    if (next < 0) break;
    Item it;
    if (item_of(next, q_tiles, pairs, a.num_kv_heads, it)) {
      prefill_body<KVT, D, PAGED>(a, it, s0, s1, bf, flags);
      __syncthreads();  // the next item's copies reuse the buffers
    }
  }
}

template <int KVT, int D, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a, int q_tiles, int slot) {
  // The body is device code only: the host pass of the compiler, which
  // needs no more than the kernel's signature, rejects some of its template
  // instantiations when both one-byte cache types are built in one file.
#if defined(__HIP_DEVICE_COMPILE__)
  using L = Lds<KVT, D>;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[L::stage], s1[L::stage];
  __shared__ __attribute__((aligned(1024))) uint8_t bf[L::bf16 > 0 ? L::bf16 : 16];
  __shared__ uint32_t flags[2];
  __shared__ int item;
  prefill_items<KVT, D, PAGED>(a, q_tiles, slot, blockIdx.x, s0, s1, bf, flags, &item);
#endif
}

// Persistent workgroups: as many as fit on the GPU at once (occupancy x
// CUs), never more than the items.
__host__ inline int64_t workers_for(int64_t items, int per_cu) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    cus = (hipGetDevice(&dev) == hipSuccess &&
           hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
              ? n
              : 256;
  }
  const int64_t w = (int64_t)cus * per_cu;
  return items < w ? items : w;
}

template <int KVT, int D, bool PAGED>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  const int q_tiles = tiles_of(a.max_seqlen_q, a.num_heads / a.num_kv_heads, col_blocks<KVT, D>());
  const int64_t items = grid_of(q_tiles, a.batch, a.num_kv_heads);
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  const int slot = wq::slot_of(stream);
  if (slot >= 0) {
    const hipError_t e = wq::reset(slot, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = slot >= 0 ? workers_for(items, 2) : items;
  hipLaunchKernelGGL((prefill_kernel<KVT, D, PAGED>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a, q_tiles,
                     slot);
  return hipGetLastError();
}

}  // namespace pf

namespace {

template <int D>
hipError_t launch_f32(const PrefillArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.total_q * a.num_heads;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int KVT>
hipError_t launch_mfma(const PrefillArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return a.block_table ? pf::launch<KVT, 64, true>(a, stream) : pf::launch<KVT, 64, false>(a, stream);
  return a.block_table ? pf::launch<KVT, 128, true>(a, stream) : pf::launch<KVT, 128, false>(a, stream);
}

}  // namespace

hipError_t launch_varlen_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.q_dtype == kF32) {
    if (a.head_dim == 64) return launch_f32<64>(a, stream);
    return launch_f32<128>(a, stream);
  }
  if (a.kv_dtype == kBF16) return launch_mfma<kBF16>(a, stream);
  // one-byte caches are paged (the entry point requires a block table)
  if (a.block_table == nullptr) return hipErrorInvalidValue;
  if (a.kv_dtype == kI8) {
    if (a.head_dim == 64) return pf::launch<kI8, 64, true>(a, stream);
    return pf::launch<kI8, 128, true>(a, stream);
  }
  if (a.head_dim == 64) return pf::launch<kFP8, 64, true>(a, stream);
  return pf::launch<kFP8, 128, true>(a, stream);
}

}  // namespace pkv
