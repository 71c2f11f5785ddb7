// extern "C" entry points of libpkv.so: argument checks, the optional
// metadata validation (PKV_VALIDATE=1) and dispatch to the kernel launchers.
#include <hip/hip_runtime_api.h>
#include <limits.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return PKV_OK;
}

bool validate_mode() {
  const char* v = getenv("PKV_VALIDATE");
  return v && v[0] == '1';
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elt_bytes(int dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    case PKV_INT8: return 1;
    default: return 0;
  }
}

bool pow2_in(int32_t x, int32_t lo, int32_t hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

bool group_ok(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// One-byte caches decoded as code x per-head scale.
bool scaled_cache(int dtype) { return dtype == PKV_FP8_E4M3 || dtype == PKV_INT8; }

// Synchronous copy of n int32 from the device (validation mode only).
bool fetch(std::vector<int32_t>& dst, const int32_t* src, int64_t n, hipStream_t stream) {
  dst.resize((size_t)n);
  if (n == 0) return true;
  if (hipStreamSynchronize(stream) != hipSuccess) return false;
  return hipMemcpy(dst.data(), src, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost) == hipSuccess;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Every block a sequence of `len` keys touches must name a block in [0, num_blocks).
int check_table_rows(const std::vector<int32_t>& table, const std::vector<int32_t>& lens,
                     int32_t max_blocks, int32_t block_size, int32_t num_blocks, const char* what) {
  for (size_t b = 0; b < lens.size(); ++b) {
    const int64_t len = lens[b];
    if (len < 0) return fail(PKV_ERR_INVALID, "%s: sequence %zu has negative length", what, b);
    const int64_t need = (len + block_size - 1) / block_size;
    if (need > max_blocks)
      return fail(PKV_ERR_INVALID, "%s: sequence %zu needs %lld blocks > max_blocks_per_seq %d", what,
                  b, (long long)need, max_blocks);
    for (int64_t j = 0; j < need; ++j) {
      const int32_t id = table[b * (size_t)max_blocks + j];
      if (id < 0 || id >= num_blocks)
        return fail(PKV_ERR_INVALID, "%s: sequence %zu logical block %lld maps to %d (pool %d)", what,
                    b, (long long)j, id, num_blocks);
    }
  }
  return PKV_OK;
}

}  // namespace

namespace {

struct NewRows {  // the append call's new K/V rows (all NULL/0 for the plain decode)
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t k_stride = 0;  // elements between sequences' rows
  int64_t v_stride = 0;
};

int decode_common(const char* name, const NewRows& nr, void* out, const void* q, int q_dtype,
                  const void* k_cache, const void* v_cache, int cache_dtype, const float* k_scale,
                  const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* cache_seqlens, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks, float softmax_scale,
                  int32_t split_keys, void* workspace, size_t workspace_bytes, void* stream,
                  pkv::DecodeArgs* prepared = nullptr, pkv::DecodePlan* prepared_plan = nullptr,
                  bool library_scratch = false) {
  const bool append = nr.k != nullptr || nr.v != nullptr;
  if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID, "%s: sizes must be positive", name);
  if (batch > 65535) return fail(PKV_ERR_INVALID, "%s: batch above 65535", name);
  if (num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "%s: num_heads %% num_kv_heads != 0", name);
  if (!out || !q || !k_cache || !v_cache || !block_table || !cache_seqlens)
    return fail(PKV_ERR_INVALID, "%s: NULL pointer", name);
  if (append && (!nr.k || !nr.v)) return fail(PKV_ERR_INVALID, "%s: NULL k_new or v_new", name);
  const bool pair_ok = (q_dtype == PKV_F32 && cache_dtype == PKV_F32) ||
                       (q_dtype == PKV_BF16 && cache_dtype == PKV_BF16) ||
                       (q_dtype == PKV_BF16 && scaled_cache(cache_dtype));
  if (!pair_ok)
    return fail(PKV_ERR_UNSUPPORTED, "%s: unsupported q/cache dtypes %d/%d", name, q_dtype, cache_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", name, head_dim);
  if (!pow2_in(block_size, 8, 256))
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d not a power of two in [8, 256]", name, block_size);
  if (!group_ok(num_heads / num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "%s: group size %d not in {1,2,4,8,16}", name,
                num_heads / num_kv_heads);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)  // key positions are 32-bit in the kernels
    return fail(PKV_ERR_INVALID, "%s: max_blocks_per_seq * block_size above 2^31 - 1", name);
  if (scaled_cache(cache_dtype) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID, "%s: fp8 and int8 caches need k_scale and v_scale", name);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "%s: q, out and caches must be 16-byte aligned", name);
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  const int qb = elt_bytes(q_dtype);
  if (append) {
    if (nr.k_stride < row || nr.v_stride < row)
      return fail(PKV_ERR_INVALID, "%s: new-row stride below the row width %lld", name, (long long)row);
    if (!aligned16(nr.k) || !aligned16(nr.v) || (nr.k_stride * qb) % 16 != 0 || (nr.v_stride * qb) % 16 != 0)
      return fail(PKV_ERR_INVALID, "%s: k_new, v_new and their strides must be 16-byte aligned", name);
  }
  pkv::DecodePlan plan;
  const char* why = nullptr;
  if (!pkv::plan_decode(batch, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        split_keys, cache_dtype != PKV_F32, &plan, &why))
    return fail(PKV_ERR_INVALID, "%s: %s", name, why);
  if (library_scratch && plan.workspace_bytes > 0) {  // the static array instead of a workspace
    if (plan.workspace_bytes > pkv::kNoAllocScratchBytes)
      return fail(PKV_ERR_INVALID,
                  "%s: these sizes need %zu bytes of decode scratch, above the %zu of the static array "
                  "(call pkv_paged_decode with a workspace instead)",
                  name, plan.workspace_bytes, pkv::kNoAllocScratchBytes);
    const hipError_t e = pkv::noalloc_scratch(&workspace);
    if (e != hipSuccess)
      return fail(PKV_ERR_LAUNCH, "%s: no device address for the scratch array: %s", name, hipGetErrorString(e));
    workspace_bytes = pkv::kNoAllocScratchBytes;
  }
  if (workspace_bytes < plan.workspace_bytes || (plan.workspace_bytes > 0 && !workspace))
    return fail(PKV_ERR_INVALID, "%s: workspace of %zu bytes needed, %zu given", name,
                plan.workspace_bytes, workspace_bytes);
  if (plan.workspace_bytes > 0 && !aligned16(workspace))
    return fail(PKV_ERR_INVALID, "%s: workspace must be 16-byte aligned", name);
  hipStream_t s = (hipStream_t)stream;
  if (!library_scratch && validate_mode()) {  // (its checks copy metadata to host memory)
    std::vector<int32_t> lens, table;
    if (!fetch(lens, cache_seqlens, batch, s) ||
        !fetch(table, block_table, (int64_t)batch * max_blocks_per_seq, s))
      return fail(PKV_ERR_LAUNCH, "%s: could not read metadata", name);
    if (append) {  // keys attended: the cached ones and the new one; new rows in distinct slots
      std::unordered_set<int64_t> seen;
      for (int32_t b = 0; b < batch; ++b) {
        if (lens[b] < 0) return fail(PKV_ERR_INVALID, "%s: sequence %d has negative length", name, b);
        if ((int64_t)lens[b] + 1 > (int64_t)max_blocks_per_seq * block_size)
          return fail(PKV_ERR_INVALID, "%s: sequence %d has no room for its new token", name, b);
        lens[b] += 1;
      }
      const int rc = check_table_rows(table, lens, max_blocks_per_seq, block_size, num_blocks, name);
      if (rc != PKV_OK) return rc;
      for (int32_t b = 0; b < batch; ++b) {
        const int64_t pos = lens[b] - 1;
        const int64_t slot = (int64_t)table[b * (size_t)max_blocks_per_seq + pos / block_size] * block_size +
                             pos % block_size;
        if (!seen.insert(slot).second)
          return fail(PKV_ERR_INVALID, "%s: sequence %d appends to slot %lld twice", name, b, (long long)slot);
      }
    } else {
      const int rc = check_table_rows(table, lens, max_blocks_per_seq, block_size, num_blocks, name);
      if (rc != PKV_OK) return rc;
    }
  }
  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = (const uint8_t*)k_cache;
  a.v_cache = (const uint8_t*)v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.cache_seqlens = cache_seqlens;
  a.workspace = (float*)workspace;
  a.stream_slots = plan.stream_slots;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.batch = batch;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.softmax_scale = softmax_scale;
  a.q_dtype = q_dtype;
  a.cache_dtype = cache_dtype;
  a.k_new = (const uint8_t*)nr.k;
  a.v_new = (const uint8_t*)nr.v;
  a.k_new_stride = nr.k_stride * qb;
  a.v_new_stride = nr.v_stride * qb;
  a.len_bias = append ? 1 : 0;
  if (prepared) {  // checked and planned; the caller launches
    *prepared = a;
    *prepared_plan = plan;
    return ok();
  }
  return launch_status(pkv::launch_paged_decode(a, plan, s), name);
}

// Checks and, unless `prepared` is given, launches a varlen prefill.  With
// `prepared`, *empty is set when there is nothing to compute.
int prefill_common(void* out, const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                       const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                       const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                       int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                       const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t num_blocks, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t total_q, int32_t total_k, void* stream, pkv::PrefillArgs* prepared = nullptr,
                       bool* empty = nullptr) {
  if (empty) *empty = false;
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return fail(PKV_ERR_INVALID, "varlen_prefill: negative size");
  if (batch > 65535) return fail(PKV_ERR_INVALID, "varlen_prefill: batch above 65535");
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "varlen_prefill: num_heads must be a positive multiple of num_kv_heads");
  if (causal != 0 && causal != 1) return fail(PKV_ERR_INVALID, "varlen_prefill: causal must be 0 or 1");
  const bool paged = block_table != nullptr;
  const bool pair_ok = (q_dtype == PKV_BF16 && kv_dtype == PKV_BF16) ||
                       (q_dtype == PKV_BF16 && scaled_cache(kv_dtype) && paged) ||
                       (q_dtype == PKV_F32 && kv_dtype == PKV_F32);
  if (!pair_ok)
    return fail(PKV_ERR_UNSUPPORTED, "varlen_prefill: unsupported q/kv dtypes %d/%d%s", q_dtype, kv_dtype,
                paged ? "" : " (fp8 and int8 need the paged cache)");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "varlen_prefill: head_dim %d not in {64, 128}", head_dim);
  if (!group_ok(num_heads / num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "varlen_prefill: group size %d not in {1,2,4,8,16}",
                num_heads / num_kv_heads);
  if (paged) {
    if (!pow2_in(block_size, 8, 256))
      return fail(PKV_ERR_UNSUPPORTED, "varlen_prefill: block_size %d not a power of two in [8, 256]",
                  block_size);
    if (max_blocks_per_seq <= 0 || num_blocks <= 0)
      return fail(PKV_ERR_INVALID, "varlen_prefill: max_blocks_per_seq and num_blocks must be positive");
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)  // key positions are 32-bit in the kernels
      return fail(PKV_ERR_INVALID, "varlen_prefill: max_blocks_per_seq * block_size above 2^31 - 1");
  }
  if (scaled_cache(kv_dtype) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID, "varlen_prefill: fp8 and int8 caches need k_scale and v_scale");
  if (batch == 0 || max_seqlen_q == 0 || total_q == 0) {
    if (empty) *empty = true;
    return ok();
  }
  if (!out || !q || !k || !v || !cu_seqlens_q || !cu_seqlens_k)
    return fail(PKV_ERR_INVALID, "varlen_prefill: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "varlen_prefill: q, k, v and out must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (validate_mode()) {
    std::vector<int32_t> cq, ck, table;
    if (!fetch(cq, cu_seqlens_q, batch + 1, s) || !fetch(ck, cu_seqlens_k, batch + 1, s))
      return fail(PKV_ERR_LAUNCH, "varlen_prefill: could not read cu_seqlens");
    if (cq[0] != 0 || ck[0] != 0) return fail(PKV_ERR_INVALID, "varlen_prefill: cu_seqlens must start at 0");
    std::vector<int32_t> klens((size_t)batch);
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t lq = cq[b + 1] - cq[b], lk = ck[b + 1] - ck[b];
      if (lq < 0 || lk < 0) return fail(PKV_ERR_INVALID, "varlen_prefill: cu_seqlens not monotone at %d", b);
      if (lq > max_seqlen_q || lk > max_seqlen_k)
        return fail(PKV_ERR_INVALID, "varlen_prefill: request %d exceeds the max_seqlen hints", b);
      klens[b] = lk;
    }
    if (cq[batch] > total_q) return fail(PKV_ERR_INVALID, "varlen_prefill: cu_seqlens_q exceeds total_q");
    if (paged) {
      if (!fetch(table, block_table, (int64_t)batch * max_blocks_per_seq, s))
        return fail(PKV_ERR_LAUNCH, "varlen_prefill: could not read block_table");
      const int rc = check_table_rows(table, klens, max_blocks_per_seq, block_size, num_blocks,
                                      "varlen_prefill");
      if (rc != PKV_OK) return rc;
    } else if (ck[batch] > total_k) {
      return fail(PKV_ERR_INVALID, "varlen_prefill: cu_seqlens_k exceeds total_k");
    }
  }
  pkv::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k = (const uint8_t*)k;
  a.v = (const uint8_t*)v;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.block_table = block_table;
  a.batch = batch;
  a.max_seqlen_q = max_seqlen_q;
  a.max_seqlen_k = max_seqlen_k;
  a.softmax_scale = softmax_scale;
  a.causal = causal;
  a.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  a.block_size = paged ? block_size : 0;
  a.num_blocks = paged ? num_blocks : 0;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.total_q = total_q;
  a.total_k = total_k;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  if (prepared) {
    *prepared = a;
    return ok();
  }
  return launch_status(pkv::launch_varlen_prefill(a, s), "varlen_prefill");
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

int pkv_kv_cache_write(const void* k, int64_t k_token_stride, const void* v, int64_t v_token_stride,
                       int src_dtype, void* k_cache, void* v_cache, int cache_dtype, int64_t num_slots,
                       const float* k_scale, const float* v_scale, const int32_t* slot_map,
                       int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "kv_cache_write: num_tokens < 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || num_slots <= 0)
    return fail(PKV_ERR_INVALID, "kv_cache_write: num_kv_heads, head_dim and num_slots must be positive");
  const bool pair_ok = (src_dtype == PKV_F32 && cache_dtype == PKV_F32) ||
                       (src_dtype == PKV_BF16 && cache_dtype == PKV_BF16) ||
                       ((src_dtype == PKV_BF16 || src_dtype == PKV_F32) && scaled_cache(cache_dtype));
  if (!pair_ok)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write: unsupported dtype pair %d -> %d", src_dtype,
                cache_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write: head_dim %d not in {64, 128}", head_dim);
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row)
    return fail(PKV_ERR_INVALID, "kv_cache_write: token stride below the row width %lld", (long long)row);
  if (!k || !v || !k_cache || !v_cache || (!slot_map && num_tokens > 0))
    return fail(PKV_ERR_INVALID, "kv_cache_write: NULL pointer");
  if (scaled_cache(cache_dtype) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID, "kv_cache_write: fp8 and int8 caches need k_scale and v_scale");
  const int sb = elt_bytes(src_dtype);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (k_token_stride * sb) % 16 != 0 || (v_token_stride * sb) % 16 != 0)
    return fail(PKV_ERR_INVALID, "kv_cache_write: pointers and token strides must be 16-byte aligned");
  if (num_tokens == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  if (validate_mode()) {
    std::vector<int32_t> slots;
    if (!fetch(slots, slot_map, num_tokens, s))
      return fail(PKV_ERR_LAUNCH, "kv_cache_write: could not read slot_map");
    std::unordered_set<int32_t> seen;
    for (int32_t t = 0; t < num_tokens; ++t) {
      const int32_t x = slots[t];
      if (x == -1) continue;
      if (x < 0 || x >= num_slots)
        return fail(PKV_ERR_INVALID, "kv_cache_write: slot_map[%d] = %d outside [0, %lld)", t, x,
                    (long long)num_slots);
      if (!seen.insert(x).second)
        return fail(PKV_ERR_INVALID, "kv_cache_write: slot %d written twice", x);
    }
  }
  pkv::WriteArgs a;
  a.k = (const uint8_t*)k;
  a.v = (const uint8_t*)v;
  a.k_stride_bytes = k_token_stride * sb;
  a.v_stride_bytes = v_token_stride * sb;
  a.k_cache = (uint8_t*)k_cache;
  a.v_cache = (uint8_t*)v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.slot_map = slot_map;
  a.num_slots = num_slots;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.src_dtype = src_dtype;
  a.cache_dtype = cache_dtype;
  return launch_status(pkv::launch_kv_write(a, s), "kv_cache_write");
}

size_t pkv_paged_decode_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t split_keys) {
  // the size does not depend on the dtypes: the larger of the two plans
  size_t bytes = 0;
  for (int mfma = 0; mfma < 2; ++mfma) {
    pkv::DecodePlan p;
    const char* why = nullptr;
    if (!pkv::plan_decode(batch, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                          split_keys, mfma != 0, &p, &why))
      return 0;
    if (p.workspace_bytes > bytes) bytes = p.workspace_bytes;
  }
  return bytes;
}

int pkv_paged_decode(void* out, const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                     int cache_dtype, const float* k_scale, const float* v_scale,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* cache_seqlens, int32_t batch, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     float softmax_scale, int32_t split_keys, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return decode_common("paged_decode", NewRows{}, out, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale,
                       v_scale, block_table, max_blocks_per_seq, cache_seqlens, batch, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, split_keys, workspace,
                       workspace_bytes, stream);
}

static_assert(pkv::kNoAllocScratchBytes == PKV_NOALLOC_SCRATCH_BYTES, "one size for the scratch array");

int pkv_paged_decode_noalloc(void* out, const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                             int cache_dtype, const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* cache_seqlens, int32_t batch, int32_t num_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             float softmax_scale, int32_t split_keys, void* stream) {
  return decode_common("paged_decode_noalloc", NewRows{}, out, q, q_dtype, k_cache, v_cache, cache_dtype,
                       k_scale, v_scale, block_table, max_blocks_per_seq, cache_seqlens, batch, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, split_keys, nullptr, 0,
                       stream, nullptr, nullptr, true);
}

int pkv_paged_decode_append(void* out, const void* q, int q_dtype, const void* k_new, int64_t k_new_stride,
                            const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                            int cache_dtype, const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* cache_seqlens, int32_t batch, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            float softmax_scale, int32_t split_keys, void* workspace, size_t workspace_bytes,
                            void* stream) {
  NewRows nr;
  nr.k = k_new;
  nr.v = v_new;
  nr.k_stride = k_new_stride;
  nr.v_stride = v_new_stride;
  if (!k_new || !v_new) return fail(PKV_ERR_INVALID, "paged_decode_append: NULL k_new or v_new");
  return decode_common("paged_decode_append", nr, out, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale,
                       v_scale, block_table, max_blocks_per_seq, cache_seqlens, batch, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, split_keys, workspace,
                       workspace_bytes, stream);
}


int pkv_varlen_prefill(void* out, const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                       const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                       const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                       int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                       const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t num_blocks, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t total_q, int32_t total_k, void* stream) {
  return prefill_common(out, q, q_dtype, k, v, kv_dtype, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, batch,
                        max_seqlen_q, max_seqlen_k, softmax_scale, causal, block_table, max_blocks_per_seq,
                        block_size, num_blocks, num_heads, num_kv_heads, head_dim, total_q, total_k, stream);
}

int pkv_mixed_attention(const void* k_cache, const void* v_cache, int cache_dtype, const float* k_scale,
                        const float* v_scale, int32_t num_blocks, int32_t block_size, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int q_dtype,
                        void* prefill_out, const void* prefill_q, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t prefill_batch, int32_t max_seqlen_q,
                        int32_t max_seqlen_k, const int32_t* prefill_block_table, int32_t prefill_max_blocks,
                        int32_t total_q, void* decode_out, const void* decode_q,
                        const int32_t* decode_block_table, int32_t decode_max_blocks,
                        const int32_t* cache_seqlens, int32_t decode_batch, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (prefill_batch < 0 || decode_batch < 0)
    return fail(PKV_ERR_INVALID, "mixed_attention: negative batch");
  pkv::PrefillArgs pa;
  bool p_empty = true;
  if (prefill_batch > 0) {
    if (!prefill_block_table) return fail(PKV_ERR_INVALID, "mixed_attention: the prefill reads the paged cache");
    const int rc = prefill_common(prefill_out, prefill_q, q_dtype, k_cache, v_cache, cache_dtype, k_scale, v_scale,
                                  cu_seqlens_q, cu_seqlens_k, prefill_batch, max_seqlen_q, max_seqlen_k,
                                  softmax_scale, 1, prefill_block_table, prefill_max_blocks, block_size,
                                  num_blocks, num_heads, num_kv_heads, head_dim, total_q, 0, stream, &pa, &p_empty);
    if (rc != PKV_OK) return rc;
  }
  pkv::DecodeArgs da;
  pkv::DecodePlan plan;
  const bool has_decode = decode_batch > 0;
  if (has_decode) {
    const int rc = decode_common("mixed_attention", NewRows{}, decode_out, decode_q, q_dtype, k_cache, v_cache,
                                 cache_dtype, k_scale, v_scale, decode_block_table, decode_max_blocks,
                                 cache_seqlens, decode_batch, num_heads, num_kv_heads, head_dim, block_size,
                                 num_blocks, softmax_scale, 0, workspace, workspace_bytes, stream, &da, &plan);
    if (rc != PKV_OK) return rc;
  }
  hipStream_t s = (hipStream_t)stream;
  // one launch for both kinds of work where the shared kernel is built: one-byte
  // caches at head_dim 128 on the matrix-core decode plan, the decode batch in
  // one slice
  const bool fused = has_decode && !p_empty && scaled_cache(cache_dtype) && head_dim == 128 && plan.stream &&
                     plan.mfma && plan.slice >= decode_batch;
  if (fused) return launch_status(pkv::launch_mixed(da, pa, s), "mixed_attention");
  if (!p_empty) {
    const int rc = launch_status(pkv::launch_varlen_prefill(pa, s), "mixed_attention");
    if (rc != PKV_OK) return rc;
  }
  if (has_decode) return launch_status(pkv::launch_paged_decode(da, plan, s), "mixed_attention");
  return ok();
}

int pkv_copy_blocks(void* k_cache, void* v_cache, int cache_dtype, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, const int32_t* block_pairs, int32_t num_pairs,
                    void* stream) {
  if (num_pairs < 0) return fail(PKV_ERR_INVALID, "copy_blocks: num_pairs < 0");
  if (num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID, "copy_blocks: sizes must be positive");
  const int eb = elt_bytes(cache_dtype);
  if (eb == 0) return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: unknown cache dtype %d", cache_dtype);
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * eb;
  if (block_bytes % 16 != 0 || block_bytes >= ((int64_t)1 << 31))
    return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: block of %lld bytes (must be a multiple of 16 below 2 GiB)",
                (long long)block_bytes);
  if (!k_cache || !v_cache || (!block_pairs && num_pairs > 0))
    return fail(PKV_ERR_INVALID, "copy_blocks: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID, "copy_blocks: caches must be 16-byte aligned");
  if (num_pairs == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  if (validate_mode()) {
    std::vector<int32_t> pairs;
    if (!fetch(pairs, block_pairs, 2 * (int64_t)num_pairs, s))
      return fail(PKV_ERR_LAUNCH, "copy_blocks: could not read the pairs");
    std::unordered_set<int32_t> dsts, srcs;
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int32_t a = pairs[2 * i], b = pairs[2 * i + 1];
      if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks)
        return fail(PKV_ERR_INVALID, "copy_blocks: pair %d (%d, %d) outside the pool of %d", i, a, b, num_blocks);
      if (!dsts.insert(b).second) return fail(PKV_ERR_INVALID, "copy_blocks: block %d written twice", b);
      srcs.insert(a);
    }
    for (int32_t b : dsts)
      if (srcs.count(b)) return fail(PKV_ERR_INVALID, "copy_blocks: block %d is both a source and a target", b);
  }
  pkv::CopyBlocksArgs a;
  a.k_cache = (uint8_t*)k_cache;
  a.v_cache = (uint8_t*)v_cache;
  a.pairs = block_pairs;
  a.block_bytes = block_bytes;
  a.num_pairs = num_pairs;
  a.num_blocks = num_blocks;
  return launch_status(pkv::launch_copy_blocks(a, s), "copy_blocks");
}

}  // extern "C"
