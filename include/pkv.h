/*
 * pkv.h -- C ABI of libpkv.so: attention over a paged KV cache on AMD MI355X
 * (gfx950).  Hand-written HIP kernels behind seven calls:
 *
 *   pkv_kv_cache_write   scatter the step's new K/V rows into cache slots
 *   pkv_paged_decode     one query per sequence over its cached keys
 *   pkv_paged_decode_append  the same decode storing the step's new K/V rows
 *                        itself (one launch for write + decode)
 *   pkv_paged_decode_noalloc the decode with library-held scratch, for
 *                        callers that cannot allocate
 *   pkv_varlen_prefill   causal attention for a packed batch of query chunks
 *   pkv_mixed_attention  a chunked-prefill step's prefill and decode in one launch
 *   pkv_copy_blocks      copy-on-write of whole cache blocks
 * and a host-side block manager (pkv_block_manager_*: allocation, sharing,
 * copy-on-write decisions, prefix hashes).
 *
 * Page citations (titles as the pages give them):
 *   [KV-mgmt]   itan.pw, "効率的な KV キャッシュ管理と Attention 計算"
 *   [paged-doc] transformers documentation, "ページド・アテンション"
 *   [ch15]      1s.xyz, "KV cache / batching / paged attention"
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer, except where a comment says
 *   otherwise.  Scalars are passed by value.  Index arrays are int32.
 * - The caller allocates and owns every buffer, including the decode
 *   workspace.  The library's only device memory of its own is one static
 *   array per GPU (64 KiB): the work-queue counters of pkv_varlen_prefill,
 *   one set per stream for the first 64 streams that call it (later streams
 *   run the prefill without queues, at one workgroup per work item).  Each
 *   launch clears its stream's set with a small kernel first, so calls on
 *   one stream never see each other's counts.  A graph captured with a
 *   prefill call keeps the capturing stream's set: two replays of it that
 *   overlap in time (on different streams) race on the counters.
 * - Every call validates its scalar arguments on the host, enqueues its
 *   kernels on `stream` (a hipStream_t; NULL = the null stream) and returns
 *   without synchronising.  It reads no device memory on the host, so
 *   metadata that lives on the device (slot maps, block tables, lengths) is
 *   trusted: see "device-side data" below.
 * - Return value: PKV_OK (0) or a negative PKV_ERR_* code; the message of the
 *   last failure on the calling thread is returned by pkv_last_error().  On an
 *   error no kernel has been launched (except PKV_ERR_LAUNCH).
 *
 * Cache layout ([KV-mgmt] section "Triton カーネルによる KV キャッシュ書き込み"
 * stores a token at slot * (heads * head_dim); section "Python 層からのカーネル
 * 呼び出し" requires that token stride of the cache; [paged-doc] section
 * デコードパス: a block table row lists, per logical block of a sequence, the
 * physical block holding it, -1 meaning unallocated):
 *   k_cache, v_cache: separate tensors [num_blocks, block_size, num_kv_heads,
 *   head_dim], contiguous.  Slot s = block * block_size + offset holds one
 *   token; key j of a sequence lives at slot
 *   block_table[b][j / block_size] * block_size + j % block_size.
 *
 * Element types: PKV_F32 (IEEE fp32), PKV_BF16 (bfloat16) and, for caches
 * only, two one-byte types with one fp32 scale per KV head for K and one for
 * V ([ch15] "KVキャッシュはどれくらいメモリを食う？": an FP8 or INT8 cache takes
 * exactly half the memory of a 16-bit one):
 *   PKV_FP8_E4M3 (OCP E4M3 "FN": bias 7, max 448, S.1111.111 = NaN): stored
 *     code = e4m3(x / scale), round to nearest even, saturating to +-448,
 *     NaN -> 0x7F; value = code * scale.  (The format is the gfx950-native one.)
 *   PKV_INT8 (two's complement): stored code = round-to-nearest-even of
 *     x / scale saturated to [-127, 127] (symmetric; -128 is never stored),
 *     NaN -> 0; value = code * scale.
 * In both, x / scale is an IEEE fp32 division of the fp32 value of x by the
 * head's fp32 scale.  FP8 and INT8 caches are read with BF16 queries.
 *
 * Supported shapes: head_dim in {64, 128}; block_size a power of two in
 * [8, 256]; num_heads a multiple of num_kv_heads with group size
 * G = num_heads / num_kv_heads in {1, 2, 4, 8, 16}.
 *
 * Device-side data (slot_map, block_table, cache_seqlens, cu_seqlens) is not
 * read on the host.  The kernels stay inside the buffers whatever it holds:
 * a slot outside [0, num_slots) is not written, a block id outside
 * [0, num_blocks) is read as an empty block (its keys are skipped), a length
 * beyond max_blocks_per_seq * block_size is cut there, and query rows beyond
 * the max_seqlen_q hint are not computed.  Results for such inputs are
 * unspecified but memory-safe.  With the environment variable PKV_VALIDATE=1
 * each call first synchronises, copies the metadata to the host and rejects
 * such inputs (and duplicate slots) with PKV_ERR_INVALID.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PKV_OK 0
#define PKV_ERR_INVALID (-1)     /* bad argument or, under PKV_VALIDATE=1, bad metadata */
#define PKV_ERR_UNSUPPORTED (-2) /* valid but not built: dtype pair, head_dim, block_size, G */
#define PKV_ERR_LAUNCH (-3)      /* a HIP runtime call failed */

/* element types */
#define PKV_F32 0
#define PKV_BF16 1
#define PKV_FP8_E4M3 2
#define PKV_INT8 3

/* Message of the last failing call on this thread ("" if none).  The string
 * is owned by the library and valid until the next call on this thread. */
const char* pkv_last_error(void);

/* Library version string (static storage). */
const char* pkv_version(void);

/*
 * pkv_kv_cache_write -- the slot-map scatter.
 * [KV-mgmt] section "Triton カーネルによる KV キャッシュ書き込み": each new token
 * stores its whole K row and V row ([num_kv_heads, head_dim]) at the cache
 * slot slot_map[t]; section "Python 層からのカーネル呼び出し": the launcher
 * checks the strides and that there is one slot per token.
 *
 *   k, v            [num_tokens, num_kv_heads, head_dim] of src_dtype (F32 or
 *                   BF16); heads and dims contiguous; consecutive tokens
 *                   k_token_stride / v_token_stride ELEMENTS apart (>= the
 *                   row width num_kv_heads * head_dim).
 *   k_cache,v_cache caches of cache_dtype, layout above, num_slots =
 *                   num_blocks * block_size rows; modified in place.
 *   k_scale,v_scale [num_kv_heads] fp32, required iff cache_dtype is FP8 or
 *                   INT8, else ignored (may be NULL).
 *   slot_map        [num_tokens]; -1 = skip the token.  Slots must be
 *                   distinct (two tokens writing one slot race).
 * Supported pairs: F32->F32, BF16->BF16 (bit copies), F32 or BF16 -> FP8 or
 * INT8 (the encodings above).
 * Pointers and byte strides must be 16-byte aligned.
 * Errors: PKV_ERR_INVALID for NULL pointers, num_tokens < 0, stride below the
 * row width, misalignment, non-positive sizes; PKV_ERR_UNSUPPORTED for other
 * dtype pairs or head_dim.  num_tokens == 0 is a no-op.
 */
int pkv_kv_cache_write(const void* k, int64_t k_token_stride,
                       const void* v, int64_t v_token_stride, int src_dtype,
                       void* k_cache, void* v_cache, int cache_dtype, int64_t num_slots,
                       const float* k_scale, const float* v_scale,
                       const int32_t* slot_map, int32_t num_tokens,
                       int32_t num_kv_heads, int32_t head_dim, void* stream);

/*
 * pkv_paged_decode_workspace_size -- bytes of fp32 scratch pkv_paged_decode
 * needs for the same geometry and split_keys (0 when no merge pass is needed).
 * Returns 0 as well for unsupported arguments (the decode call reports them).
 */
size_t pkv_paged_decode_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t split_keys);

/*
 * pkv_paged_decode -- one query token per sequence attending to its cache.
 * [paged-doc] section デコードパス: every sequence brings one query; the kernel
 * finds its keys through block_table ([batch, max_blocks_per_seq]) and
 * cache_seqlens; [KV-mgmt] section "Attention モジュールの実装" writes the step's
 * K/V before this call, so cache_seqlens[b] counts the new token as well.
 *
 *   out   [batch, num_heads, head_dim] of q_dtype, written.
 *   q     [batch, num_heads, head_dim] of q_dtype (F32 or BF16), contiguous.
 *   k_cache, v_cache of cache_dtype (F32 with F32 q; BF16, FP8 or INT8 with
 *               BF16 q).
 *   k_scale, v_scale [num_kv_heads] fp32, required iff FP8 or INT8.
 *   block_table [batch, max_blocks_per_seq], row-major; entries past the
 *               sequence's last block are never read (may be -1).  An entry
 *               inside the sequence that is negative or >= num_blocks is read
 *               as an empty block: its keys are left out of the softmax.
 *   cache_seqlens [batch] keys per sequence (0 -> output row of zeros;
 *               values above max_blocks_per_seq * block_size are clamped).
 * out[b, h] = sum_j softmax_j(scale * q[b,h] . k_j) v_j over the sequence's
 * keys j < cache_seqlens[b], with k_j, v_j read from KV head h / G (q heads
 * are grouped contiguously).
 *   split_keys  keys per work unit of the split-K plan: 0 = automatic, else a
 *               multiple of 128.  Long contexts are cut into units processed
 *               in parallel; a second kernel merges their partial results.
 *               The automatic plan deals equal shares of 32-key chunks to a
 *               persistent grid; a batch over 2048 runs as equal slices of
 *               at most 2048 sequences, launched in order on `stream`.
 *   workspace   device scratch of at least pkv_paged_decode_workspace_size()
 *               bytes for the same arguments (NULL allowed when that is 0).
 *               Its contents on entry do not matter.
 * Errors: PKV_ERR_INVALID (NULL pointers, sizes <= 0, Hq % Hkv != 0, bad
 * split_keys, workspace too small); PKV_ERR_UNSUPPORTED (dtype pair,
 * head_dim, block_size, G).
 */
int pkv_paged_decode(void* out, const void* q, int q_dtype,
                     const void* k_cache, const void* v_cache, int cache_dtype,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* cache_seqlens, int32_t batch,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, float softmax_scale,
                     int32_t split_keys, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * pkv_paged_decode_noalloc -- pkv_paged_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and the same results.  The kernels' partial
 * results go to a static device array of PKV_NOALLOC_SCRATCH_BYTES (32 MiB)
 * that each GPU holds from this call's first use on it until the process
 * ends; the call itself allocates nothing (no hipMalloc, no hipFree).
 *   Limit: sizes whose pkv_paged_decode_workspace_size exceeds
 *   PKV_NOALLOC_SCRATCH_BYTES are rejected with PKV_ERR_INVALID (the
 *   automatic plan at batch 256, 8 KV heads, G = 4, head_dim 128 needs about
 *   12 MiB).  PKV_VALIDATE is ignored: its checks copy metadata to the host.
 *   Sharing: every call on one GPU uses that GPU's one array, and nothing in
 *   it needs to start at any value.  Calls whose kernels overlap in time on
 *   one GPU (on different streams, or replays of captured graphs) race on it
 *   and give wrong results; serialise them.
 * Errors: those of pkv_paged_decode, and PKV_ERR_LAUNCH when the array's
 * device address cannot be obtained.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pkv_paged_decode_noalloc(void* out, const void* q, int q_dtype,
                             const void* k_cache, const void* v_cache, int cache_dtype,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* cache_seqlens, int32_t batch,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, float softmax_scale,
                             int32_t split_keys, void* stream);

/*
 * pkv_paged_decode_append -- the decode step with its own cache write.
 * [paged-doc] section デコードパス ("キャッシュの動作"): the decode kernel reads
 * the paged cache through the block table and updates it in place; in the
 * section's worked example cache_seqlens lists the keys cached BEFORE the
 * step ([30, 32, 70]) and each new token goes to the next position of its
 * sequence (so sequence 1's token opens its second block).
 *
 * For every sequence b with 0 <= cache_seqlens[b] < max_blocks_per_seq *
 * block_size, the new rows k_new[b], v_new[b] are stored at position
 * p = cache_seqlens[b], i.e. at slot block_table[b][p / block_size] *
 * block_size + p % block_size (exactly the bytes pkv_kv_cache_write would
 * store there, fp8 encoding included), and out[b] is the decode of q[b] over
 * the p + 1 keys that include the new one.  The result equals
 * pkv_kv_cache_write followed by pkv_paged_decode with cache_seqlens + 1, in
 * one launch on the matrix-core plan (bf16 and fp8 caches, automatic split);
 * other plans launch a small append kernel before the decode kernels.
 *
 *   k_new, v_new  [batch, num_kv_heads, head_dim] of q_dtype (the cache's
 *                 element type for F32/BF16 caches; BF16 for FP8 and INT8
 *                 caches),
 *                 heads and dims contiguous, sequences k_new_stride /
 *                 v_new_stride ELEMENTS apart (>= num_kv_heads * head_dim),
 *                 16-byte aligned.
 *   k_cache, v_cache  modified in place (one row per sequence and head).
 *   cache_seqlens [batch] keys cached before this call.  The block holding
 *                 p should be allocated in block_table, and no two sequences
 *                 may append to the same slot.  Metadata that leaves the new
 *                 token no slot is handled as in pkv_paged_decode: a
 *                 position past the block table stores nothing and the
 *                 sequence attends its max_blocks_per_seq * block_size
 *                 cached keys (lengths are clamped); a block entry that is
 *                 negative or >= num_blocks stores nothing and reads as an
 *                 empty block (its keys, the new one included, are left out
 *                 of the softmax; a sequence left with no key returns
 *                 zeros).  A negative cache_seqlens[b] stores nothing; its
 *                 result is unspecified (memory-safe).
 *   Every other argument, the workspace size
 *   (pkv_paged_decode_workspace_size with the same geometry) and the errors
 *   are those of pkv_paged_decode; also PKV_ERR_INVALID for NULL k_new/v_new
 *   or a bad stride.  Under PKV_VALIDATE=1 the call also rejects sequences
 *   without room for the new token and two appends to one slot.
 */
int pkv_paged_decode_append(void* out, const void* q, int q_dtype,
                            const void* k_new, int64_t k_new_stride,
                            const void* v_new, int64_t v_new_stride,
                            void* k_cache, void* v_cache, int cache_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* cache_seqlens, int32_t batch,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, float softmax_scale,
                            int32_t split_keys, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * pkv_varlen_prefill -- causal attention for a packed batch of query chunks.
 * [paged-doc] section "Varlen パス": request b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b],
 * cu_seqlens_k[b+1]); max_seqlen_q / max_seqlen_k bound the lengths.
 * [KV-mgmt] section "Attention モジュールの実装": with a block table the paged
 * caches take the place of k and v (prefix sharing).
 *
 *   out   [total_q, num_heads, head_dim] of q_dtype, written (every row of
 *         every request; rows that see no key are zero).
 *   q     [total_q, num_heads, head_dim] of q_dtype (BF16, or F32), contiguous.
 *   k, v  block_table == NULL: packed [total_k, num_kv_heads, head_dim] of
 *         kv_dtype, contiguous, request b's keys at rows cu_seqlens_k[b]...
 *         block_table != NULL: the paged caches (layout above, num_blocks
 *         blocks of block_size); request b has Lk = cu_seqlens_k[b+1] -
 *         cu_seqlens_k[b] keys read through block_table row b
 *         ([batch, max_blocks_per_seq]).
 *   kv_dtype  BF16 with BF16 q (contiguous or paged), FP8 or INT8 with BF16
 *             q (paged only, k_scale/v_scale required), F32 with F32 q.
 *   causal  1: query row i of a request with Lq queries and Lk keys sees keys
 *           j <= i + Lk - Lq (aligned to the end, so a chunk after a cached
 *           prefix sees the whole prefix); 0: sees all Lk keys.
 *   total_q, total_k  rows held by q/out and, without a block table, by k/v
 *           (host values; rows beyond them are never touched).
 * Errors: as for pkv_paged_decode; also max_seqlen_q < 0 or causal not 0/1.
 */
int pkv_varlen_prefill(void* out, const void* q, int q_dtype,
                       const void* k, const void* v, int kv_dtype,
                       const float* k_scale, const float* v_scale,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                       int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                       int32_t causal, const int32_t* block_table, int32_t max_blocks_per_seq,
                       int32_t block_size, int32_t num_blocks,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t total_q, int32_t total_k, void* stream);

/*
 * pkv_mixed_attention -- the attention of a mixed chunked-prefill step: the
 * prefill chunks (causal, over the paged cache) and the decode sequences in
 * one call.  [ch15] section "プレフィックスキャッシュとchunked prefill": long
 * prefills are cut into chunks that join other requests' decodes in one
 * batch, so that the compute-heavy prefill and the memory-heavy decode
 * complement each other; [paged-doc] sections "Varlen パス" and デコードパス:
 * the varlen kernel takes mixed batches, the decode kernel does not.
 *
 * The results are those of pkv_varlen_prefill(causal = 1, paged) on the
 * prefill arguments and of pkv_paged_decode (split_keys = 0) on the decode
 * arguments (the decode's split points may differ, so its bits may differ
 * within rounding).  Shared arguments: the caches, their dtype and scales,
 * num_blocks, block_size, the head counts, head_dim, softmax_scale and
 * q_dtype.  For one-byte caches (FP8, INT8) at head_dim 128, with a decode
 * batch that the automatic plan serves with its matrix-core stream-K kernel
 * in one slice (batch <= 2048), both kinds of work run in ONE kernel launch (each CU runs
 * a decode worker and prefill tiles side by side; then the decode's merge
 * kernel); otherwise the prefill kernel and the decode kernels are launched
 * one after the other.  prefill_batch or decode_batch may be 0 (that part is
 * skipped).
 *   prefill_*    as pkv_varlen_prefill's out, q, cu_seqlens_q, cu_seqlens_k,
 *                batch, max_seqlen_q, max_seqlen_k, block_table,
 *                max_blocks_per_seq, total_q (the block table is required).
 *   decode_*, cache_seqlens, workspace  as pkv_paged_decode's out, q,
 *                block_table, max_blocks_per_seq, cache_seqlens, batch and
 *                workspace (pkv_paged_decode_workspace_size with split 0).
 * Errors: those of the two calls (the message names the failing part).
 */
int pkv_mixed_attention(const void* k_cache, const void* v_cache, int cache_dtype,
                        const float* k_scale, const float* v_scale, int32_t num_blocks,
                        int32_t block_size, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, float softmax_scale, int q_dtype,
                        void* prefill_out, const void* prefill_q, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t prefill_batch, int32_t max_seqlen_q,
                        int32_t max_seqlen_k, const int32_t* prefill_block_table,
                        int32_t prefill_max_blocks, int32_t total_q, void* decode_out,
                        const void* decode_q, const int32_t* decode_block_table,
                        int32_t decode_max_blocks, const int32_t* cache_seqlens,
                        int32_t decode_batch, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * ---------------------------------------------------------------------------
 * Block management.  [ch15] section "PagedAttention：メモリを「ページ」で貸し出
 * す": the cache is handed out block by block as sequences grow, blocks need
 * not be contiguous, and answers generated from one prompt share the prompt's
 * blocks, a shared block being copied only when one of them must write into
 * it (copy-on-write).  Section "プレフィックスキャッシュとchunked prefill":
 * requests whose prompts begin alike reuse the cache of that prefix, found by
 * a hash of each block's tokens.
 * ---------------------------------------------------------------------------
 */

/*
 * pkv_copy_blocks -- the copy-on-write data move: for each pair i, block
 * block_pairs[2 i] of k_cache and of v_cache is copied to block
 * block_pairs[2 i + 1] (the caches as above, num_blocks blocks of
 * block_size * num_kv_heads * head_dim elements of cache_dtype).
 *   block_pairs  [num_pairs, 2] int32 (src, dst), device.  Targets must be
 *                distinct and no target may be a source of another pair
 *                (the pairs run concurrently); a pair naming a block outside
 *                [0, num_blocks) moves nothing.  Under PKV_VALIDATE=1 such
 *                pairs are rejected.
 * Errors: PKV_ERR_INVALID (NULL pointers, non-positive sizes, misaligned
 * caches); PKV_ERR_UNSUPPORTED (unknown dtype, a block size in bytes that is
 * not a multiple of 16 or not below 2 GiB).  num_pairs == 0 is a no-op.
 */
int pkv_copy_blocks(void* k_cache, void* v_cache, int cache_dtype, int32_t num_blocks,
                    int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                    const int32_t* block_pairs, int32_t num_pairs, void* stream);

/*
 * pkv_block_manager -- host-side allocator of the physical blocks of one
 * cache pool (plain host memory and host calls; no device access; not
 * thread-safe).  Every block has a count of holders (sequences whose block
 * table names it).  A block nobody holds is free; if it carries a registered
 * prefix hash it stays findable by pkv_block_manager_lookup until it is
 * handed out again (free blocks without a hash go first; among hashed ones
 * the one released longest ago).  Calls return PKV_OK, or PKV_ERR_INVALID
 * with nothing changed (NULL arguments, blocks outside the pool, releasing a
 * block more often than it is held, no free block left); they do not set
 * pkv_last_error.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks blocks of block_size tokens, all free; NULL on bad sizes. */
pkv_block_manager* pkv_block_manager_create(int32_t num_blocks, int32_t block_size);
void pkv_block_manager_destroy(pkv_block_manager* m);
/* Blocks that pkv_block_manager_allocate can hand out now (-1 for NULL). */
int32_t pkv_block_manager_num_free(const pkv_block_manager* m);
/* Holders of a block (-1 outside the pool). */
int32_t pkv_block_manager_refcount(const pkv_block_manager* m, int32_t block);
/* n free blocks into out_blocks (host array), each now held once. */
int pkv_block_manager_allocate(pkv_block_manager* m, int32_t n, int32_t* out_blocks);
/* One more holder for each listed block (all must be held already). */
int pkv_block_manager_share(pkv_block_manager* m, const int32_t* blocks, int32_t n);
/* One holder less for each listed block; a block no longer held becomes free. */
int pkv_block_manager_release(pkv_block_manager* m, const int32_t* blocks, int32_t n);
/* A child sequence sharing the parent's blocks: child_row (host, max_blocks_per_seq
 * entries) = the parent's first ceil(num_tokens / block_size) entries, the
 * rest -1; each shared block gains a holder. */
int pkv_block_manager_fork(pkv_block_manager* m, const int32_t* parent_row, int32_t num_tokens,
                           int32_t* child_row, int32_t max_blocks_per_seq);
/* Room for a sequence's next token at position num_tokens (its block-table
 * row, host, is updated in place): a fresh block when the position opens a
 * logical block; when the block holding it is shared or carries a registered
 * prefix, a fresh block replaces it in this row and out_copy = {old, new}
 * names the copy to make with pkv_copy_blocks before the token is written
 * (else out_copy = {-1, -1}).  *out_slot = the token's cache slot, the
 * slot_map entry of pkv_kv_cache_write. */
int pkv_block_manager_append_slot(pkv_block_manager* m, int32_t* table_row, int32_t max_blocks_per_seq,
                                  int32_t num_tokens, int32_t* out_slot, int32_t* out_copy);
/* Hash of a full block of token ids chained to the hash of the blocks before
 * it (0 for the first block): 64-bit FNV-1a over the parent hash and the
 * ids, little-endian. */
uint64_t pkv_block_hash(uint64_t parent_hash, const int32_t* tokens, int32_t num_tokens);
/* The block registered for a prefix hash, now held once more (a free one is
 * taken back from the free blocks), or -1. */
int32_t pkv_block_manager_lookup(pkv_block_manager* m, uint64_t hash);
/* Register a held, full block under a prefix hash.  Returns PKV_OK, 1 when
 * another block already carries that hash (nothing changed), or
 * PKV_ERR_INVALID. */
int pkv_block_manager_register(pkv_block_manager* m, int32_t block, uint64_t hash);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
