"""Seeded synthetic workloads for the paged-KV write, decode and prefill path.

Every array is host numpy in the storage format the GPU receives:
``np.float32`` values for fp32, ``np.uint16`` bit patterns for bf16 and
``np.uint8`` OCP-E4M3 codes for an fp8 cache.  Index arrays are ``np.int32``.

A *step* is one engine iteration over a set of sequences.  Sequence n has
``prefix[n]`` tokens already cached and ``new[n]`` new tokens this step.  The
step writes the new K/V rows through ``slot_map`` and then attends: prefill
sequences through the varlen call, decode sequences (one new token each)
through the decode call.  New tokens are packed sequence after sequence, in
the order the sequences are listed.

Recipe (all draws from ``numpy.random.Generator(PCG64)``; config k uses seed
1000 + k; bulk values come from per-chunk sub-streams
``SeedSequence([seed, stage, chunk])`` so that big caches can be drawn in
parallel and still be reproducible):

1. lengths (stage 1),  2. block permutation (stage 2),  3. q (stage 3),
4. cached history K then V (stages 4, 5),  5. new K then V (stages 6, 7),
6. fp8 scales (from the new K/V, no draw).

* Values are N(0, 1), drawn as float32 and rounded to nearest-even bf16 where
  the dtype is bf16.
* An fp8 history holds codes drawn uniformly from the 254 finite E4M3 codes.
  The per-head scales are amax(|new K or V of that head|) / 448 in fp32.
* The block pool is sized to fit: ``num_blocks = sum_n ceil((prefix+new)/bs)``;
  physical ids are a random permutation dealt to the sequences in order, and
  unused table cells are -1.
* Every cache slot that holds no history (unallocated blocks, tails past a
  sequence's length and the slots the step is about to write) is poisoned
  with NaN (fp8: code 0x7F), so a kernel that reads past a length or through
  an unused table cell shows up as NaN in its output.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
_CHUNK = 1 << 24  # values per sub-stream chunk


# ---------------------------------------------------------------------------
# random value helpers
# ---------------------------------------------------------------------------


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bf16, ties to even."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _normal(seed: int, stage: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) values of ``shape`` in storage ``dtype`` ("f32" or "bf16")."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    chunks = [(c, min(_CHUNK, n - c * _CHUNK)) for c in range(max(1, math.ceil(n / _CHUNK)))]

    def fill(chunk):
        c, size = chunk
        if size <= 0:
            return
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stage, c])))
        vals = rng.standard_normal(size, dtype=np.float32)
        lo = c * _CHUNK
        out[lo:lo + size] = vals if dtype == "f32" else _f32_to_bf16_bits(vals)

    _run_chunks(fill, chunks)
    return out.reshape(shape)


def _fp8_codes(seed: int, stage: int, shape) -> np.ndarray:
    """Codes drawn uniformly from the 254 finite E4M3 codes (0x7F, 0xFF excluded)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint8)
    chunks = [(c, min(_CHUNK, n - c * _CHUNK)) for c in range(max(1, math.ceil(n / _CHUNK)))]

    def fill(chunk):
        c, size = chunk
        if size <= 0:
            return
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stage, c])))
        r = rng.integers(0, 254, size=size, dtype=np.int32)
        out[c * _CHUNK:c * _CHUNK + size] = np.where(r < 0x7F, r, r + 1).astype(np.uint8)

    _run_chunks(fill, chunks)
    return out.reshape(shape)


def _int8_codes(seed: int, stage: int, shape) -> np.ndarray:
    """Codes drawn uniformly from [-127, 127] (the symmetric int8 range)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.int8)
    chunks = [(c, min(_CHUNK, n - c * _CHUNK)) for c in range(max(1, math.ceil(n / _CHUNK)))]

    def fill(chunk):
        c, size = chunk
        if size <= 0:
            return
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stage, c])))
        out[c * _CHUNK:c * _CHUNK + size] = rng.integers(-127, 128, size=size, dtype=np.int32).astype(np.int8)

    _run_chunks(fill, chunks)
    return out.reshape(shape)


def _run_chunks(fill, chunks):
    workers = min(len(chunks), max(1, min(16, os.cpu_count() or 1)))
    if workers == 1:
        for ch in chunks:
            fill(ch)
    else:
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(fill, chunks))


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------


@dataclass
class Step:
    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str            # "f32" | "bf16"   (also the new K/V dtype)
    cache_dtype: str        # "f32" | "bf16" | "fp8" | "int8"
    kinds: list             # per sequence: "prefill" | "decode"
    prefix: np.ndarray      # int32 [N] tokens cached before the step
    new: np.ndarray         # int32 [N] tokens added this step
    block_table: np.ndarray  # int32 [N, max_blocks]
    k_cache: np.ndarray     # [num_blocks, bs, Hkv, D] history + poison
    v_cache: np.ndarray
    k_new: np.ndarray       # [T, Hkv, D]
    v_new: np.ndarray
    slot_map: np.ndarray    # int32 [T]
    q: np.ndarray           # [T, Hq, D]
    scale: float
    k_scale: np.ndarray = None  # float32 [Hkv] (fp8 caches only)
    v_scale: np.ndarray = None
    seed: int = 0
    meta: dict = field(default_factory=dict)

    # ---- derived views -------------------------------------------------
    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.new.sum())

    @property
    def total(self) -> np.ndarray:
        """Keys each sequence attends after the write."""
        return (self.prefix + self.new).astype(np.int32)

    def ids(self, kind: str) -> np.ndarray:
        return np.array([i for i, k in enumerate(self.kinds) if k == kind], dtype=np.int64)

    def token_ranges(self) -> np.ndarray:
        starts = np.concatenate([[0], np.cumsum(self.new)]).astype(np.int64)
        return starts

    def decode_inputs(self) -> dict:
        """Arguments of the decode call for the decode sequences of the step."""
        ids = self.ids("decode")
        starts = self.token_ranges()
        rows = starts[ids]
        return dict(
            q=self.q[rows],                                      # [B, Hq, D]
            block_table=np.ascontiguousarray(self.block_table[ids]),
            cache_seqlens=self.total[ids].astype(np.int32),
            max_blocks_per_seq=int(self.block_table.shape[1]),
            seq_ids=ids,
        )

    def decode_append_inputs(self) -> dict:
        """Arguments of the appending decode call: the decode sequences' new
        K/V rows and their lengths before the step (the call stores the rows)."""
        d = self.decode_inputs()
        rows = self.token_ranges()[d["seq_ids"]]
        d["k_new"] = np.ascontiguousarray(self.k_new[rows])
        d["v_new"] = np.ascontiguousarray(self.v_new[rows])
        d["cache_seqlens"] = self.prefix[d["seq_ids"]].astype(np.int32)
        return d

    def prefill_slot_map(self) -> np.ndarray:
        """The step's slot map with the decode sequences' tokens skipped (-1),
        for a step whose decode tokens are stored by the appending decode."""
        sm = self.slot_map.copy()
        starts = self.token_ranges()
        for i in self.ids("decode"):
            sm[starts[i]:starts[i + 1]] = -1
        return sm

    def prefill_inputs(self) -> dict:
        """Arguments of the varlen call (paged K/V) for the prefill sequences."""
        ids = self.ids("prefill")
        starts = self.token_ranges()
        qrows = np.concatenate([np.arange(starts[i], starts[i + 1]) for i in ids]) if len(ids) else \
            np.zeros(0, dtype=np.int64)
        lq = self.new[ids].astype(np.int64)
        lk = self.total[ids].astype(np.int64)
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        return dict(
            q=self.q[qrows],                                     # [sum Lq, Hq, D]
            cu_seqlens_q=cu_q,
            cu_seqlens_k=cu_k,
            max_seqlen_q=int(lq.max()) if len(ids) else 0,
            max_seqlen_k=int(lk.max()) if len(ids) else 0,
            block_table=np.ascontiguousarray(self.block_table[ids]),
            max_blocks_per_seq=int(self.block_table.shape[1]),
            seq_ids=ids,
            q_rows=qrows,
        )


def build_step(name: str, seed: int, *, num_heads: int, num_kv_heads: int, head_dim: int,
               block_size: int, q_dtype: str, cache_dtype: str, prefix, new, kinds,
               block_table=None, num_blocks=None, scale=None, poison=True) -> Step:
    """Assemble a step from per-sequence lengths (stage 1 is the caller's draw).

    ``block_table``/``num_blocks`` may be given explicitly (the worked example);
    otherwise the pool is sized to fit and the blocks are a random permutation.
    """
    prefix = np.asarray(prefix, dtype=np.int32)
    new = np.asarray(new, dtype=np.int32)
    n = len(prefix)
    bs = int(block_size)
    total = (prefix + new).astype(np.int64)
    nblk = (total + bs - 1) // bs

    # 2. block allocation
    if block_table is None:
        num_blocks = int(nblk.sum())
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2, 0])))
        perm = rng.permutation(num_blocks).astype(np.int32)
        max_blocks = int(max(1, nblk.max()) if n else 1)
        block_table = np.full((n, max_blocks), -1, dtype=np.int32)
        off = 0
        for i in range(n):
            block_table[i, :nblk[i]] = perm[off:off + nblk[i]]
            off += int(nblk[i])
    else:
        block_table = np.asarray(block_table, dtype=np.int32)
        if num_blocks is None:
            num_blocks = int(block_table.max()) + 1

    # caller-side slot assignment: position p of sequence i lives in logical
    # block p // bs at offset p % bs of the physical block the table names
    tokens = int(new.sum())
    slot_map = np.empty(tokens, dtype=np.int32)
    t = 0
    for i in range(n):
        for p in range(int(prefix[i]), int(total[i])):
            slot_map[t] = block_table[i, p // bs] * bs + p % bs
            t += 1

    hq, hkv, d = num_heads, num_kv_heads, head_dim
    # 3. queries
    q = _normal(seed, 3, (tokens, hq, d), q_dtype)
    # 4. cached history (whole pool drawn, then non-history slots poisoned)
    shape = (num_blocks, bs, hkv, d)
    if cache_dtype == "fp8":
        k_cache = _fp8_codes(seed, 4, shape)
        v_cache = _fp8_codes(seed, 5, shape)
    elif cache_dtype == "int8":
        k_cache = _int8_codes(seed, 4, shape)
        v_cache = _int8_codes(seed, 5, shape)
    else:
        k_cache = _normal(seed, 4, shape, cache_dtype)
        v_cache = _normal(seed, 5, shape, cache_dtype)
    if poison:
        history = np.zeros(num_blocks * bs, dtype=bool)
        for i in range(n):
            p = np.arange(int(prefix[i]))
            history[block_table[i, p // bs].astype(np.int64) * bs + p % bs] = True
        # int8 has no NaN: -128, a code the encoder never stores, marks the slots
        nan = {"f32": np.float32(np.nan), "bf16": BF16_NAN, "fp8": FP8_NAN, "int8": np.int8(-128)}[cache_dtype]
        k_cache.reshape(num_blocks * bs, hkv * d)[~history] = nan
        v_cache.reshape(num_blocks * bs, hkv * d)[~history] = nan
    # 5. new K/V in the query dtype
    k_new = _normal(seed, 6, (tokens, hkv, d), q_dtype)
    v_new = _normal(seed, 7, (tokens, hkv, d), q_dtype)
    # 6. fp8 scales: per-head amax / 448
    k_scale = v_scale = None
    if cache_dtype in ("fp8", "int8"):
        top = 448.0 if cache_dtype == "fp8" else 127.0  # the code range's largest magnitude
        k_scale = _amax_scale(k_new, q_dtype, top)
        v_scale = _amax_scale(v_new, q_dtype, top)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Step(name=name, num_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                q_dtype=q_dtype, cache_dtype=cache_dtype, kinds=list(kinds), prefix=prefix,
                new=new, block_table=block_table, k_cache=k_cache, v_cache=v_cache,
                k_new=k_new, v_new=v_new, slot_map=slot_map, q=q, scale=float(scale),
                k_scale=k_scale, v_scale=v_scale, seed=seed)


def _amax_scale(x: np.ndarray, dtype: str, top: float = 448.0) -> np.ndarray:
    if dtype == "bf16":
        vals = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        vals = x.astype(np.float32)
    amax = np.abs(vals).max(axis=(0, 2)) if vals.shape[0] else np.ones(vals.shape[1], np.float32)
    amax = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    return (amax / np.float32(top)).astype(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1, 0])))


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

# The decode worked example's block table, cached lengths and block size.
PAGE2_DECODE_TABLE = [[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]]
PAGE2_DECODE_LENS = [30, 32, 70]


def config(name: str, **overrides) -> Step:
    """The named synthetic workloads.

    * ``tiny_decode``: the decode worked example (3 sequences with 30/32/70
      cached tokens, block size 32, 8 physical blocks, the printed block
      table); 8 q heads / 2 KV heads, head_dim 64, fp32; scale 1/8.
    * ``llama8b_decode``: batch 64, 32 q / 8 KV heads, head_dim 128, bf16;
      cached lengths U{512..4096}; block size 16.
    * ``varlen_prefill_prefix``: 16 sequences, new lengths U{128..2048},
      cached prefix U{0..1024}; 32/8 heads, head_dim 128, bf16, block size 16.
    * ``llama70b_long_decode``: batch 8, 131072 cached tokens each, 64 q / 8 KV
      heads, head_dim 128, bf16, block size 16.
    * ``mixed_fp8``: 4 prefill chunks of 512 tokens (prefix U{0..8192}) then 256
      decode sequences (cached U{1024..16384}); 32/8 heads, head_dim 128;
      fp8 E4M3 cache with per-head scales, bf16 queries.
    * ``mixed_int8``: the same step (same lengths) with an int8 cache
      (per-head scales amax / 127).

    ``overrides`` can shrink a workload (``batch``, ``len_lo``, ``len_hi`` ...)
    for the oracle-sized parity cases; the seed stays the config's.
    """
    if name == "tiny_decode":
        seed = 1001
        return build_step(name, seed, num_heads=8, num_kv_heads=2, head_dim=64, block_size=32,
                          q_dtype="f32", cache_dtype="f32", prefix=PAGE2_DECODE_LENS, new=[1, 1, 1],
                          kinds=["decode"] * 3, block_table=PAGE2_DECODE_TABLE, num_blocks=8,
                          scale=1.0 / 8.0)
    if name == "llama8b_decode":
        seed = 1002
        b = overrides.get("batch", 64)
        lo, hi = overrides.get("len_lo", 512), overrides.get("len_hi", 4096)
        lens = _rng(seed).integers(lo, hi + 1, size=b).astype(np.int32)
        return build_step(name, seed, num_heads=overrides.get("num_heads", 32),
                          num_kv_heads=overrides.get("num_kv_heads", 8),
                          head_dim=overrides.get("head_dim", 128),
                          block_size=overrides.get("block_size", 16), q_dtype="bf16",
                          cache_dtype=overrides.get("cache_dtype", "bf16"), prefix=lens,
                          new=np.ones(b, np.int32), kinds=["decode"] * b)
    if name == "varlen_prefill_prefix":
        seed = 1003
        b = overrides.get("batch", 16)
        rng = _rng(seed)
        lq = rng.integers(overrides.get("q_lo", 128), overrides.get("q_hi", 2048) + 1, size=b)
        pre = rng.integers(overrides.get("p_lo", 0), overrides.get("p_hi", 1024) + 1, size=b)
        return build_step(name, seed, num_heads=overrides.get("num_heads", 32),
                          num_kv_heads=overrides.get("num_kv_heads", 8),
                          head_dim=overrides.get("head_dim", 128),
                          block_size=overrides.get("block_size", 16), q_dtype="bf16",
                          cache_dtype=overrides.get("cache_dtype", "bf16"), prefix=pre, new=lq,
                          kinds=["prefill"] * b)
    if name == "llama70b_long_decode":
        seed = 1004
        b = overrides.get("batch", 8)
        length = overrides.get("length", 131072)
        return build_step(name, seed, num_heads=overrides.get("num_heads", 64),
                          num_kv_heads=overrides.get("num_kv_heads", 8), head_dim=128, block_size=16,
                          q_dtype="bf16", cache_dtype="bf16", prefix=np.full(b, length, np.int32),
                          new=np.ones(b, np.int32), kinds=["decode"] * b)
    if name in ("mixed_fp8", "mixed_int8"):
        seed = 1005
        n_pre = overrides.get("prefill_chunks", 4)
        chunk = overrides.get("chunk", 512)
        n_dec = overrides.get("decode_batch", 256)
        rng = _rng(seed)
        pre_p = rng.integers(0, overrides.get("p_hi", 8192) + 1, size=n_pre)
        dec_l = rng.integers(overrides.get("len_lo", 1024), overrides.get("len_hi", 16384) + 1,
                             size=n_dec)
        prefix = np.concatenate([pre_p, dec_l]).astype(np.int32)
        new = np.concatenate([np.full(n_pre, chunk), np.ones(n_dec)]).astype(np.int32)
        return build_step(name, seed, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                          q_dtype="bf16", cache_dtype="fp8" if name == "mixed_fp8" else "int8",
                          prefix=prefix, new=new, kinds=["prefill"] * n_pre + ["decode"] * n_dec)
    raise KeyError(name)


def config_names():
    return ["tiny_decode", "llama8b_decode", "varlen_prefill_prefix", "llama70b_long_decode",
            "mixed_fp8"]


# ---------------------------------------------------------------------------
# contiguous varlen inputs (no cache)
# ---------------------------------------------------------------------------


@dataclass
class VarlenContig:
    name: str
    q: np.ndarray            # [sum Lq, Hq, D]
    k: np.ndarray            # [sum Lk, Hkv, D]
    v: np.ndarray
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    max_seqlen_q: int
    max_seqlen_k: int
    dtype: str
    scale: float


def random_varlen_contig(name: str, seed: int, q_lens, k_lens, *, num_heads: int,
                         num_kv_heads: int, head_dim: int, dtype: str) -> VarlenContig:
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    q = _normal(seed, 3, (int(cu_q[-1]), num_heads, head_dim), dtype)
    k = _normal(seed, 4, (int(cu_k[-1]), num_kv_heads, head_dim), dtype)
    v = _normal(seed, 5, (int(cu_k[-1]), num_kv_heads, head_dim), dtype)
    return VarlenContig(name=name, q=q, k=k, v=v, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                        max_seqlen_q=int(q_lens.max()) if len(q_lens) else 0,
                        max_seqlen_k=int(k_lens.max()) if len(k_lens) else 0, dtype=dtype,
                        scale=1.0 / math.sqrt(head_dim))


def page2_varlen_example(dtype: str = "bf16", num_heads: int = 8, num_kv_heads: int = 2,
                         head_dim: int = 128) -> VarlenContig:
    """The varlen worked example's lengths: q [10, 3, 1], k [0, 1, 7]."""
    return random_varlen_contig("page2_varlen", 1100, [10, 3, 1], [0, 1, 7], num_heads=num_heads,
                                num_kv_heads=num_kv_heads, head_dim=head_dim, dtype=dtype)
