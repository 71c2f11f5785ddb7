// Host-side block manager of the paged cache, and the C entry point of the
// copy-on-write block copy.
//
// [ch15] "KV cache / batching / paged attention", section "PagedAttention：メモ
// リを「ページ」で貸し出す": the cache is split into blocks of a fixed number of
// tokens, a block is handed out only when a sequence needs it, blocks need not
// be contiguous (the attention reads them through the block table), and
// answers generated from one prompt share the prompt's blocks, a shared block
// being copied only when one of them must write into it (copy-on-write).
// Section "プレフィックスキャッシュとchunked prefill": requests whose prompts
// begin alike reuse the cache of that prefix, found by a hash of the block's
// tokens.
//
// The manager is plain host code: reference counts per block, a free list, a
// table from prefix hash to block, and a least-recently-released list of
// blocks that nobody holds but that still carry a registered prefix (they are
// handed out again only when the free list is empty, and a lookup of their
// hash revives them).  It never touches device memory; the caller applies the
// copy pairs it returns with pkv_copy_blocks before writing the new tokens.
// Not thread-safe: one manager per scheduler thread.

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <list>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

struct pkv_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;         // holders of each block
  std::vector<uint64_t> hash;       // registered prefix hash (valid where hashed[b])
  std::vector<char> hashed;
  std::vector<int32_t> free_list;   // ref 0, no hash (a stack: the last released first)
  std::list<int32_t> cached;        // ref 0 with a hash, oldest release first
  std::vector<std::list<int32_t>::iterator> cached_at;
  std::vector<char> in_cached;
  std::unordered_map<uint64_t, int32_t> by_hash;
};

namespace {

bool valid_block(const pkv_block_manager* m, int32_t b) { return m && b >= 0 && b < m->num_blocks; }

void drop_hash(pkv_block_manager* m, int32_t b) {
  if (!m->hashed[b]) return;
  auto it = m->by_hash.find(m->hash[b]);
  if (it != m->by_hash.end() && it->second == b) m->by_hash.erase(it);
  m->hashed[b] = 0;
}

// A block nobody holds: a fresh one from the free list, else the cached block
// released longest ago (its prefix is forgotten).  -1 if there is none.
int32_t take_block(pkv_block_manager* m) {
  int32_t b = -1;
  if (!m->free_list.empty()) {
    b = m->free_list.back();
    m->free_list.pop_back();
  } else if (!m->cached.empty()) {
    b = m->cached.front();
    m->cached.pop_front();
    m->in_cached[b] = 0;
    drop_hash(m, b);
  }
  if (b >= 0) m->ref[b] = 1;
  return b;
}

void release_one(pkv_block_manager* m, int32_t b) {
  if (--m->ref[b] > 0) return;
  if (m->hashed[b]) {
    m->cached_at[b] = m->cached.insert(m->cached.end(), b);
    m->in_cached[b] = 1;
  } else {
    m->free_list.push_back(b);
  }
}

int32_t available(const pkv_block_manager* m) {
  return (int32_t)(m->free_list.size() + m->cached.size());
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_block_manager_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  auto* m = new pkv_block_manager;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->ref.assign((size_t)num_blocks, 0);
  m->hash.assign((size_t)num_blocks, 0);
  m->hashed.assign((size_t)num_blocks, 0);
  m->cached_at.resize((size_t)num_blocks);
  m->in_cached.assign((size_t)num_blocks, 0);
  m->free_list.reserve((size_t)num_blocks);
  for (int32_t b = num_blocks - 1; b >= 0; --b) m->free_list.push_back(b);  // block 0 first
  return m;
}

void pkv_block_manager_destroy(pkv_block_manager* m) { delete m; }

int32_t pkv_block_manager_num_free(const pkv_block_manager* m) { return m ? available(m) : -1; }

int32_t pkv_block_manager_refcount(const pkv_block_manager* m, int32_t block) {
  return valid_block(m, block) ? m->ref[block] : -1;
}

int pkv_block_manager_allocate(pkv_block_manager* m, int32_t n, int32_t* out_blocks) {
  if (!m || n < 0 || (n > 0 && !out_blocks)) return PKV_ERR_INVALID;
  if (n > available(m)) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) out_blocks[i] = take_block(m);
  return PKV_OK;
}

int pkv_block_manager_share(pkv_block_manager* m, const int32_t* blocks, int32_t n) {
  if (!m || n < 0 || (n > 0 && !blocks)) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i)
    if (!valid_block(m, blocks[i]) || m->ref[blocks[i]] <= 0) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) ++m->ref[blocks[i]];
  return PKV_OK;
}

int pkv_block_manager_release(pkv_block_manager* m, const int32_t* blocks, int32_t n) {
  if (!m || n < 0 || (n > 0 && !blocks)) return PKV_ERR_INVALID;
  std::unordered_map<int32_t, int32_t> count;  // a block may appear several times
  for (int32_t i = 0; i < n; ++i) {
    if (!valid_block(m, blocks[i])) return PKV_ERR_INVALID;
    if (++count[blocks[i]] > m->ref[blocks[i]]) return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) release_one(m, blocks[i]);
  return PKV_OK;
}

int pkv_block_manager_fork(pkv_block_manager* m, const int32_t* parent_row, int32_t num_tokens,
                           int32_t* child_row, int32_t max_blocks_per_seq) {
  if (!m || !parent_row || !child_row || num_tokens < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID;
  const int64_t used = ((int64_t)num_tokens + m->block_size - 1) / m->block_size;
  if (used > max_blocks_per_seq) return PKV_ERR_INVALID;
  const int rc = pkv_block_manager_share(m, parent_row, (int32_t)used);
  if (rc != PKV_OK) return rc;
  for (int32_t j = 0; j < max_blocks_per_seq; ++j) child_row[j] = j < used ? parent_row[j] : -1;
  return PKV_OK;
}

int pkv_block_manager_append_slot(pkv_block_manager* m, int32_t* table_row, int32_t max_blocks_per_seq,
                                  int32_t num_tokens, int32_t* out_slot, int32_t* out_copy) {
  if (!m || !table_row || !out_slot || !out_copy || num_tokens < 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID;
  out_copy[0] = out_copy[1] = -1;
  const int64_t lb = num_tokens / m->block_size;
  if (lb >= max_blocks_per_seq) return PKV_ERR_INVALID;
  int32_t blk = table_row[lb];
  if (num_tokens % m->block_size == 0 || blk < 0) {
    // the position opens a logical block: a fresh physical one
    if (blk >= 0 && !valid_block(m, blk)) return PKV_ERR_INVALID;
    const bool held = blk >= 0 && m->ref[blk] > 0;
    // a table that already names a block for an empty position: keep it if
    // it is this sequence's alone, else give the sequence its own
    if (held && m->ref[blk] == 1 && !m->hashed[blk]) {
      *out_slot = blk * m->block_size + num_tokens % m->block_size;
      return PKV_OK;
    }
    if (available(m) == 0) return PKV_ERR_INVALID;  // nothing changed
    const int32_t nb = take_block(m);
    if (held) release_one(m, blk);
    table_row[lb] = nb;
    *out_slot = nb * m->block_size + num_tokens % m->block_size;
    return PKV_OK;
  }
  if (!valid_block(m, blk) || m->ref[blk] <= 0) return PKV_ERR_INVALID;
  if (m->ref[blk] > 1 || m->hashed[blk]) {
    // shared (or a registered prefix, which stays as it is): copy on write
    if (available(m) == 0) return PKV_ERR_INVALID;
    const int32_t nb = take_block(m);
    out_copy[0] = blk;
    out_copy[1] = nb;
    release_one(m, blk);
    table_row[lb] = nb;
    blk = nb;
  }
  *out_slot = blk * m->block_size + num_tokens % m->block_size;
  return PKV_OK;
}

uint64_t pkv_block_hash(uint64_t parent_hash, const int32_t* tokens, int32_t num_tokens) {
  // FNV-1a (64-bit: offset basis 14695981039346656037, prime 2^40 + 2^8 +
  // 0xb3) over the parent's hash and the token ids, little-endian
  uint64_t h = 14695981039346656037ull;
  auto mix = [&h](uint64_t x, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (x >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix(parent_hash, 8);
  for (int32_t i = 0; i < num_tokens; ++i) mix((uint32_t)tokens[i], 4);
  return h;
}

int32_t pkv_block_manager_lookup(pkv_block_manager* m, uint64_t hash) {
  if (!m) return -1;
  auto it = m->by_hash.find(hash);
  if (it == m->by_hash.end()) return -1;
  const int32_t b = it->second;
  if (m->in_cached[b]) {  // revive a released prefix block
    m->cached.erase(m->cached_at[b]);
    m->in_cached[b] = 0;
  }
  ++m->ref[b];
  return b;
}

int pkv_block_manager_register(pkv_block_manager* m, int32_t block, uint64_t hash) {
  if (!valid_block(m, block) || m->ref[block] <= 0) return PKV_ERR_INVALID;
  auto it = m->by_hash.find(hash);
  if (it != m->by_hash.end()) return it->second == block ? PKV_OK : 1;  // another block holds it
  drop_hash(m, block);
  m->hash[block] = hash;
  m->hashed[block] = 1;
  m->by_hash[hash] = block;
  return PKV_OK;
}

}  // extern "C"
