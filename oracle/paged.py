"""Paged KV cache: slot-map write, block-table gather and softmax attention, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Storage conventions (host numpy arrays, the same bits the GPU receives):

* ``"f32"``  -> ``np.float32`` values;
* ``"bf16"`` -> ``np.uint16`` bit patterns (the upper half of an IEEE fp32);
* ``"fp8"``  -> ``np.uint8`` OCP E4M3 codes, one fp32 scale per KV head;
* ``"int8"`` -> ``np.int8`` codes, one fp32 scale per KV head.

Cache layout: one K and one V tensor per layer, each ``[num_blocks,
block_size, num_kv_heads, head_dim]`` and contiguous, so that cache slot
``s = block * block_size + offset`` starts at element ``s * kv_heads * head_dim``
([KV-mgmt] "効率的な KV キャッシュ管理と Attention 計算", section "Triton カーネル
による KV キャッシュ書き込み": the store offset is the slot times the per-token
width, and section "Python 層からのカーネル呼び出し" requires the cache's token
stride to equal that width; [paged-doc] "ページド・アテンション", section
デコードパス: the block table names the physical block of each logical block).
"""

import numpy as np

from . import e4m3, int8

# ---------------------------------------------------------------------------
# storage <-> float64
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """A bf16 value is the fp32 whose upper 16 bits are these and lower 16 are 0."""
    wide = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return wide.view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str, scale=None) -> np.ndarray:
    """Exact float64 value of stored elements ``[..., heads, head_dim]``.

    For fp8 the stored code is multiplied by its head's fp32 scale; the product
    of a 4-bit-mantissa value and an fp32 is exact in float64.
    """
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype in ("fp8", "int8"):
        if scale is None:
            raise ValueError(f"{dtype} storage needs a per-head scale")
        per_head = np.asarray(scale, dtype=np.float32).astype(np.float64)
        codes = e4m3.decode(arr) if dtype == "fp8" else int8.decode(arr)
        return codes * per_head[:, None]
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _to_f32_values(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Source K/V (f32 values or bf16 bits) as exact float32 values."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32)
    if dtype == "bf16":
        wide = np.ascontiguousarray(arr, dtype=np.uint16).astype(np.uint32) << 16
        return wide.view(np.float32)
    raise ValueError(f"unsupported source dtype {dtype!r}")


# ---------------------------------------------------------------------------
# index bookkeeping ([paged-doc] worked examples)
# ---------------------------------------------------------------------------


def cu_seqlens(lengths) -> np.ndarray:
    """Exclusive prefix sums with a leading 0: request b owns [cu[b], cu[b+1]).

    [paged-doc] section "Varlen パス", インデックス機構 and 例.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def request_index(cu: np.ndarray) -> np.ndarray:
    """Request that owns each packed token: the b with cu[b] <= t < cu[b+1].

    A request with an empty range owns no token ([paged-doc] "Varlen パス", 例).
    """
    cu = np.asarray(cu, dtype=np.int64)
    owner = np.empty(int(cu[-1]), dtype=np.int64)
    for b in range(len(cu) - 1):
        owner[cu[b]:cu[b + 1]] = b
    return owner


def slot_of(block_table_row, pos: int, block_size: int) -> int:
    """Physical slot of logical position ``pos``: its block's physical id times
    the block size plus the offset inside the block ([paged-doc] "デコードパス")."""
    block = int(block_table_row[pos // block_size])
    if block < 0:
        raise ValueError(f"position {pos} falls in an unallocated block")
    return block * block_size + pos % block_size


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` tokens occupies: ceil(n / bs)."""
    return -(-int(num_tokens) // int(block_size))


# ---------------------------------------------------------------------------
# write: the slot-map scatter ([KV-mgmt] "Triton カーネルによる KV キャッシュ書き込み")
# ---------------------------------------------------------------------------


def kv_cache_write(k, v, k_cache, v_cache, slot_map, src_dtype: str, cache_dtype: str,
                   k_scale=None, v_scale=None):
    """Return copies of the caches after storing token t's K and V rows at slot
    ``slot_map[t]``.

    * Each token moves its whole ``[kv_heads, head_dim]`` row for K and for V.
    * A slot of -1 means "no slot": the token is skipped (reading of the pages;
      the printed kernel has no guard, the decode example uses -1 for
      "unallocated").
    * Other slots must lie in [0, num_slots) and be distinct; anything else is
      a caller error (raised here).
    * f32 -> f32 and bf16 -> bf16 store the source bits unchanged.  For an fp8
      cache the stored code is e4m3(fp32(x) / fp32(scale[head])), with an IEEE
      fp32 division.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    slot_map = np.asarray(slot_map, dtype=np.int64)
    nb, bs, hkv, d = k_cache.shape
    num_slots = nb * bs
    if k.shape[0] != slot_map.shape[0] or v.shape[0] != slot_map.shape[0]:
        raise ValueError("one slot per token")
    k_out = k_cache.copy().reshape(num_slots, hkv, d)
    v_out = v_cache.copy().reshape(num_slots, hkv, d)
    seen = set()
    for t in range(slot_map.shape[0]):
        s = int(slot_map[t])
        if s == -1:
            continue
        if not 0 <= s < num_slots:
            raise ValueError(f"slot {s} out of range [0, {num_slots})")
        if s in seen:
            raise ValueError(f"slot {s} written twice")
        seen.add(s)
        k_out[s] = _store_row(k[t], src_dtype, cache_dtype, k_scale)
        v_out[s] = _store_row(v[t], src_dtype, cache_dtype, v_scale)
    return k_out.reshape(k_cache.shape), v_out.reshape(v_cache.shape)


def _store_row(row, src_dtype, cache_dtype, scale):
    if cache_dtype == src_dtype and cache_dtype in ("f32", "bf16"):
        return row
    if cache_dtype in ("fp8", "int8"):
        x = _to_f32_values(row, src_dtype)                       # [hkv, d] float32
        s = np.asarray(scale, dtype=np.float32)[:, None]
        quotient = (x / s).astype(np.float32)                     # IEEE fp32 division
        return e4m3.encode_fast(quotient) if cache_dtype == "fp8" else int8.encode(quotient)
    raise ValueError(f"unsupported write {src_dtype} -> {cache_dtype}")


# ---------------------------------------------------------------------------
# gather and attention
# ---------------------------------------------------------------------------


def gather_slots(block_table_row, num_keys: int, block_size: int) -> np.ndarray:
    """Slots of logical keys 0..num_keys-1 of one sequence.

    Key j lives in logical block j // bs at offset j % bs; the block table maps
    the logical block to a physical one ([paged-doc] "デコードパス"; [ch15]
    "PagedAttention：メモリを「ページ」で貸し出す": blocks need not be
    contiguous).  Every block that holds a key must be allocated (>= 0).
    """
    j = np.arange(int(num_keys), dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[j // block_size]
    if np.any(blocks < 0):
        raise ValueError("a key falls in an unallocated block")
    return blocks * block_size + j % block_size


def gather(cache: np.ndarray, block_table_row, num_keys: int) -> np.ndarray:
    """Stored rows ``[num_keys, kv_heads, head_dim]`` of one sequence, in logical order."""
    nb, bs, hkv, d = cache.shape
    slots = gather_slots(block_table_row, num_keys, bs)
    return cache.reshape(nb * bs, hkv, d)[slots]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
              heads=None, positions=None, num_queries=None) -> np.ndarray:
    """Textbook scaled softmax attention of one sequence, float64.

    q ``[Lq, Hq, D]``, k and v ``[Lk, Hkv, D]`` -> ``[Lq, Hq, D]``.

    * GQA: q head h reads KV head h // (Hq / Hkv) (contiguous groups; the pages
      say several q heads share a KV head but not which: reading).
    * Logits are ``scale * q . k`` ([KV-mgmt] "Attention モジュールの実装" passes
      ``softmax_scale``).
    * Causal masking is aligned bottom-right: query row i (of Lq) sees keys
      j <= i + Lk - Lq, so the last query sees every key and a chunk that
      follows a cached prefix sees the whole prefix ([KV-mgmt] runs the
      causal varlen call on the paged cache for prefix sharing: reading).
    * A row that sees no key outputs zeros (an empty sum; reading for the
      zero-key request of the [paged-doc] varlen example).
    * ``heads``: optional subset of q heads to compute (others stay 0).
    * ``positions`` / ``num_queries``: the given q rows are rows ``positions``
      of a chunk of ``num_queries`` queries (default: all rows, in order).
    """
    lq, hq, _ = q.shape
    lk, hkv, dv = v.shape
    if hq % hkv:
        raise ValueError("q heads must be a multiple of KV heads")
    group = hq // hkv
    out = np.zeros((lq, hq, dv), dtype=np.float64)
    if lq == 0:
        return out
    rows = (np.arange(lq) if positions is None else np.asarray(positions))[:, None]
    chunk = lq if num_queries is None else int(num_queries)
    cols = np.arange(lk)[None, :]
    if causal:
        visible = cols <= rows + (lk - chunk)
    else:
        visible = np.ones((lq, lk), dtype=bool)
    has_key = visible.any(axis=1)
    for h in (range(hq) if heads is None else heads):
        g = h // group
        logits = scale * (q[:, h, :] @ k[:, g, :].T)
        logits = np.where(visible, logits, -np.inf)
        row_max = np.where(has_key, logits.max(axis=1, initial=-np.inf), 0.0)
        weights = np.where(visible, np.exp(logits - row_max[:, None]), 0.0)
        numer = weights @ v[:, g, :]
        denom = weights.sum(axis=1)
        out[:, h, :] = np.where(has_key[:, None], numer / np.where(has_key, denom, 1.0)[:, None], 0.0)
    return out


def paged_decode(q, q_dtype, k_cache, v_cache, cache_dtype, block_table, cache_seqlens,
                 scale, k_scale=None, v_scale=None, pairs=None):
    """One query per sequence over its whole cached history.

    [paged-doc] "デコードパス": each sequence brings exactly one query token and
    its cached length; [KV-mgmt] "Attention モジュールの実装" writes the step's
    K/V first and then attends, so ``cache_seqlens`` counts the new token too.

    q ``[B, Hq, D]`` (storage bits) -> float64 ``[B, Hq, D]``.
    ``pairs``: optional list of (b, h) to compute; the rest stay 0.
    """
    q64 = to_f64(q, q_dtype)
    bsz, hq, d = q64.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    out = np.zeros_like(q64)
    wanted = {}
    if pairs is None:
        for b in range(bsz):
            wanted[b] = None
    else:
        for b, h in pairs:
            wanted.setdefault(int(b), set()).add(int(h))
    for b, heads in wanted.items():
        lk = int(cache_seqlens[b])
        if heads is None:
            kv_heads = list(range(hkv))
        else:
            kv_heads = sorted({h // group for h in heads})
        k_rows = gather(k_cache, block_table[b], lk)
        v_rows = gather(v_cache, block_table[b], lk)
        k64 = np.zeros((lk, hkv, d))
        v64 = np.zeros((lk, hkv, d))
        for g in kv_heads:
            k64[:, g, :] = _rows_to_f64(k_rows[:, g:g + 1, :], cache_dtype, k_scale, g)[:, 0, :]
            v64[:, g, :] = _rows_to_f64(v_rows[:, g:g + 1, :], cache_dtype, v_scale, g)[:, 0, :]
        out[b] = attention(q64[b][None], k64, v64, scale, causal=True,
                           heads=None if heads is None else sorted(heads))[0]
    return out


def paged_decode_append(q, q_dtype, k_new, v_new, k_cache, v_cache, cache_dtype, block_table,
                        cache_seqlens, scale, k_scale=None, v_scale=None, pairs=None):
    """The decode step that stores its own token first.

    [paged-doc] "デコードパス", "キャッシュの動作": the decode kernel updates the
    paged cache in place; in the section's worked example ``cache_seqlens``
    counts the keys cached before the step and each sequence's new token goes
    to the next position (sequence 1, with 32 keys in blocks of 32, opens its
    second block).  So: token b's rows go to slot ``slot_of(row b, L_b)``
    with ``L_b = cache_seqlens[b]``, then the plain decode runs over
    ``L_b + 1`` keys.

    Returns ``(out, k_cache', v_cache')``.
    """
    lens = np.asarray(cache_seqlens, dtype=np.int64)
    bs = k_cache.shape[1]
    slots = np.array([slot_of(block_table[b], int(lens[b]), bs) for b in range(lens.shape[0])],
                     dtype=np.int64)
    kc, vc = kv_cache_write(k_new, v_new, k_cache, v_cache, slots, q_dtype, cache_dtype, k_scale, v_scale)
    out = paged_decode(q, q_dtype, kc, vc, cache_dtype, block_table, lens + 1, scale, k_scale, v_scale,
                       pairs=pairs)
    return out, kc, vc


def varlen_prefill(q, q_dtype, k, v, kv_dtype, cu_seqlens_q, cu_seqlens_k, scale, causal,
                   block_table=None, k_scale=None, v_scale=None, rows=None):
    """Variable-length batch of query chunks, one sequence after another.

    [paged-doc] "Varlen パス": request b owns packed query rows
    [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]).  Without a block table
    k and v are packed ``[sum Lk, Hkv, D]`` tensors; with one they are the paged
    caches and only the per-request key count Lk = cu_k[b+1] - cu_k[b] is used,
    the keys being gathered through row b of the table ([KV-mgmt] "Attention
    モジュールの実装": with block tables the cache tensors replace k and v).

    ``rows``: optional set of packed query rows to compute (others stay 0).
    """
    q64 = to_f64(q, q_dtype)
    out = np.zeros_like(q64)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    wanted = None if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        if wanted is not None:
            mine = wanted[(wanted >= q0) & (wanted < q1)]
            if len(mine) == 0:
                continue
        lk = int(cu_k[b + 1] - cu_k[b])
        if block_table is None:
            k_rows = k[cu_k[b]:cu_k[b + 1]]
            v_rows = v[cu_k[b]:cu_k[b + 1]]
        else:
            k_rows = gather(k, block_table[b], lk)
            v_rows = gather(v, block_table[b], lk)
        k64 = _rows_to_f64(k_rows, kv_dtype, k_scale)
        v64 = _rows_to_f64(v_rows, kv_dtype, v_scale)
        if wanted is None:
            out[q0:q1] = attention(q64[q0:q1], k64, v64, scale, causal)
        else:
            out[mine] = attention(q64[mine], k64, v64, scale, causal, positions=mine - q0,
                                  num_queries=q1 - q0)
    return out


def _rows_to_f64(rows, dtype, scale, head=None):
    if dtype in ("fp8", "int8"):
        s = np.asarray(scale, dtype=np.float32)
        s = s if head is None else s[head:head + 1]
        return to_f64(rows, dtype, s)
    return to_f64(rows, dtype)
