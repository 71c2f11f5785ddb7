// Internal interface between the C ABI layer (pkv_api.cpp) and the kernel
// launchers (*.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct WriteArgs {
  const uint8_t* k;
  const uint8_t* v;
  int64_t k_stride_bytes;
  int64_t v_stride_bytes;
  uint8_t* k_cache;
  uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* slot_map;
  int64_t num_slots;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int src_dtype;
  int cache_dtype;
};

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream);

// Split-K plan of the decode: keys [s * split_keys, (s+1) * split_keys) of a
// sequence form work unit s.
struct DecodePlan {
  bool stream;          // stream-K kernel (automatic plan) instead of fixed splits
  bool mfma;            // stream-K on the matrix cores (bf16 cache): one unit per KV head
  int32_t split_keys;   // fixed splits: multiple of kDecodeKeysPerWg
  int32_t num_splits;   // fixed splits: units per sequence at the longest possible length
  int32_t head_groups;  // q-head groups of at most 8 per KV head
  int64_t stream_slots; // stream-K: partial slots (waves + units) of one launch
  int32_t slice;         // stream-K: sequences per launch (the batch, or equal slices of it)
  size_t workspace_bytes;
};

constexpr int kDecodeWaves = 4;
constexpr int kDecodeChunk = 32;                              // keys per wave iteration
constexpr int kDecodeKeysPerWg = kDecodeWaves * kDecodeChunk;  // 128
constexpr int kDecodeMaxSplitKeys = 8192;                     // bounds the LDS block table
constexpr int kStreamThreads = 256;                           // stream-K decode workgroup
constexpr int kStreamMaxBatch = 2048;                         // LDS chunk-count table of one launch
constexpr int kStreamMaxWaves = 4096;                         // bounds the stream-K workspace

// Fills `plan`; returns false (with a message in *why) for arguments the
// planner cannot serve.  Pure host arithmetic, no HIP calls.
// mfma: the cache is bf16, so the automatic plan may use the matrix-core
// kernel (whole KV heads as units).
bool plan_decode(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, int32_t max_blocks_per_seq, int32_t split_keys, bool mfma,
                 DecodePlan* plan, const char** why);

struct DecodeArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* cache_seqlens;
  float* workspace;
  int64_t stream_slots;  // stream-K: partial slots in the workspace
  int32_t max_blocks_per_seq;
  int32_t batch;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  float softmax_scale;
  int q_dtype;
  int cache_dtype;
  // Append call (k_new != NULL): the step's new K/V rows, [batch, Hkv, D] of
  // q_dtype, sequences k_new_stride / v_new_stride bytes apart.  The call
  // stores them at position cache_seqlens[b] and attends cache_seqlens[b] + 1
  // keys (len_bias = 1); otherwise len_bias = 0 and nothing is written.
  const uint8_t* k_new;
  const uint8_t* v_new;
  int64_t k_new_stride;
  int64_t v_new_stride;
  int32_t len_bias;
};

hipError_t launch_paged_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

// Bytes of the static decode scratch array (one per GPU) behind
// pkv_paged_decode_noalloc; equal to PKV_NOALLOC_SCRATCH_BYTES.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;

// Device address of that array on the current device (looked up once per
// device, on the first call with that device current).
hipError_t noalloc_scratch(void** ptr);

struct PrefillArgs {
  void* out;
  const void* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* block_table;
  int32_t batch;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  float softmax_scale;
  int32_t causal;
  int32_t max_blocks_per_seq;
  int32_t block_size;
  int32_t num_blocks;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t total_q;
  int32_t total_k;
  int q_dtype;
  int kv_dtype;
};

hipError_t launch_varlen_prefill(const PrefillArgs& a, hipStream_t stream);

// Prefill work items and the stream-K decode in one launch (one-byte caches,
// head_dim 128, decode on the matrix-core plan), then the decode's merge.
hipError_t launch_mixed(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream);

struct CopyBlocksArgs {
  uint8_t* k_cache;
  uint8_t* v_cache;
  const int32_t* pairs;  // [num_pairs, 2] (src, dst) block ids, device
  int64_t block_bytes;   // bytes of one block of one cache (a multiple of 16, < 2^31)
  int32_t num_pairs;
  int32_t num_blocks;
};

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

}  // namespace pkv
