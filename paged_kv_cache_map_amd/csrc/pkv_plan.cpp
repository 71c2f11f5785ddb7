// Host-only planning for the decode split-K; no HIP runtime calls, so it can
// be exercised without a GPU through pkv_paged_decode_workspace_size().
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

namespace {
constexpr int64_t kTargetWorkgroups = 2048;  // ~8 per CU on 256 CUs, counted at the longest length
constexpr int32_t kMinAutoSplit = 256;
constexpr int32_t kMaxAutoSplit = 4096;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
}  // namespace

bool plan_decode(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, int32_t max_blocks_per_seq, int32_t split_keys, bool mfma,
                 DecodePlan* plan, const char** why) {
  if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0) {
    *why = "batch, head counts, block_size and max_blocks_per_seq must be positive";
    return false;
  }
  if (num_heads % num_kv_heads != 0) {
    *why = "num_heads must be a multiple of num_kv_heads";
    return false;
  }
  const int32_t group = num_heads / num_kv_heads;
  // The matrix-core stream kernel serves all q heads of a KV head in one
  // unit.  The vector kernels serve them in groups of at most 4: a wave's
  // live state for 4 heads fits two waves per SIMD; larger groups read their
  // KV head once per group (the repeats hit the caches).
  const bool use_mfma = mfma && split_keys == 0;
  const int32_t valu_groups = group > 4 ? group / 4 : 1;
  int32_t head_groups = use_mfma ? 1 : valu_groups;
  const int64_t max_keys = (int64_t)max_blocks_per_seq * block_size;
  plan->head_groups = head_groups;
  // Automatic plan: stream-K, when the chunk count of a launch fits in 31
  // bits.  A launch's chunk-count table lives in LDS and holds at most
  // kStreamMaxBatch sequences: a larger batch runs as equal slices, launched
  // one after another on the stream, that share one workspace.
  const int64_t slices = ((int64_t)batch + kStreamMaxBatch - 1) / kStreamMaxBatch;
  const int32_t slice = (int32_t)((batch + slices - 1) / slices);
  const int64_t units = (int64_t)slice * num_kv_heads * head_groups;
  const int64_t max_chunks = units * ((max_keys + kDecodeChunk - 1) / kDecodeChunk);
  if (split_keys == 0 && max_chunks < (int64_t)1 << 31) {
    const int64_t per_unit_heads = group / head_groups;
    plan->stream = true;
    plan->mfma = use_mfma;
    plan->split_keys = 0;
    plan->num_splits = 0;
    plan->slice = slice;
    plan->stream_slots = kStreamMaxWaves + units;
    // partial triples of every slot, then the chunk prefix of the slice
    plan->workspace_bytes =
        (size_t)plan->stream_slots * per_unit_heads * (size_t)(head_dim + 2) * sizeof(float) +
        (size_t)(slice + 1) * sizeof(int32_t);
    return true;
  }
  plan->stream = false;
  plan->mfma = false;
  plan->stream_slots = 0;
  plan->slice = batch;
  head_groups = valu_groups;  // the fixed-split kernel runs on the vector ALUs
  int64_t sk;
  if (split_keys == 0) {
    const int64_t units = (int64_t)batch * num_kv_heads * head_groups;
    sk = round_up((max_keys * units + kTargetWorkgroups - 1) / kTargetWorkgroups, kDecodeKeysPerWg);
    if (sk < kMinAutoSplit) sk = kMinAutoSplit;
    if (sk > kMaxAutoSplit) sk = kMaxAutoSplit;
    if (max_keys <= sk) sk = round_up(max_keys, kDecodeKeysPerWg);
  } else {
    if (split_keys < 0 || split_keys % kDecodeKeysPerWg != 0 || split_keys > kDecodeMaxSplitKeys) {
      *why = "split_keys must be 0 or a positive multiple of 128 no larger than 8192";
      return false;
    }
    sk = split_keys;
  }
  const int64_t splits = (max_keys + sk - 1) / sk;
  if (splits > 0x7fffffff) {
    *why = "too many splits";
    return false;
  }
  plan->split_keys = (int32_t)sk;
  plan->num_splits = (int32_t)(splits < 1 ? 1 : splits);
  plan->head_groups = head_groups;
  plan->workspace_bytes =
      plan->num_splits > 1
          ? (size_t)batch * num_heads * plan->num_splits * (size_t)(head_dim + 2) * sizeof(float)
          : 0;
  return true;
}

}  // namespace pkv
