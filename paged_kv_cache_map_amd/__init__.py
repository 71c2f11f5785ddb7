"""Attention over a paged KV cache on AMD MI355X (gfx950).

Thin Python binding of ``libpkv.so`` (C ABI in ``include/pkv.h``).  Every
operation runs in the library's HIP kernels; this module only reads shapes,
strides and device pointers from torch tensors, allocates outputs and the
decode workspace with torch, and passes the current HIP stream.  The first
call (or :func:`library`) raises ImportError when the library has not been
built (``python -m paged_kv_cache_map_amd.build``): there is no fallback path.

Calls (same names as the C entry points without the ``pkv_`` prefix):

* :func:`kv_cache_write` -- scatter new K/V rows into cache slots;
* :func:`paged_decode`   -- one query per sequence through the block table;
* :func:`paged_decode_append` -- the same decode storing the step's new K/V
  rows itself (write + decode in one call);
* :func:`varlen_prefill` -- causal attention for a packed batch of chunks;
* :func:`mixed_attention` -- a chunked-prefill step's prefill and decode in one call;
* :func:`copy_blocks`    -- copy-on-write of whole cache blocks;
* :class:`BlockManager`  -- the host-side block allocator (``pkv_block_manager_*``).
"""

import ctypes
import os
import pathlib

# PKV_LIBRARY may name another build of the same library (A/B timing of
# kernel variants); by default the in-tree build next to this file is used.
LIB_PATH = pathlib.Path(os.environ.get("PKV_LIBRARY") or
                        pathlib.Path(__file__).resolve().with_name("libpkv.so"))

F32, BF16, FP8_E4M3, INT8 = 0, 1, 2, 3
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_LAUNCH = 0, -1, -2, -3


class PkvError(RuntimeError):
    """A libpkv call returned a non-zero status."""

    def __init__(self, code, message):
        super().__init__(f"libpkv error {code}: {message}")
        self.code = code


def _load_library():
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m paged_kv_cache_map_amd.build`")
    # torch ships its own HIP runtime under the same soname as the system's.
    # Loaded first, it is the one the library binds to, so the library runs
    # on the runtime that owns the tensors and streams it is handed; loaded
    # the other way round, the process would hold two runtimes, each with its
    # own device state.
    import torch  # noqa: F401
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_version.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_kv_cache_write.restype = ctypes.c_int
    lib.pkv_kv_cache_write.argtypes = [vp, i64, vp, i64, ctypes.c_int, vp, vp, ctypes.c_int, i64,
                                       vp, vp, vp, i32, i32, i32, vp]
    lib.pkv_paged_decode_workspace_size.restype = sz
    lib.pkv_paged_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.pkv_paged_decode.restype = ctypes.c_int
    lib.pkv_paged_decode.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, i32, vp,
                                     i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.pkv_paged_decode_noalloc.restype = ctypes.c_int
    lib.pkv_paged_decode_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, i32, vp,
                                             i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.pkv_paged_decode_append.restype = ctypes.c_int
    lib.pkv_paged_decode_append.argtypes = [vp, vp, ctypes.c_int, vp, i64, vp, i64, vp, vp, ctypes.c_int,
                                            vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                            vp, sz, vp]
    lib.pkv_varlen_prefill.restype = ctypes.c_int
    lib.pkv_varlen_prefill.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                       i32, i32, i32, f32, i32, vp, i32, i32, i32, i32, i32, i32,
                                       i32, i32, vp]
    lib.pkv_mixed_attention.restype = ctypes.c_int
    lib.pkv_mixed_attention.argtypes = [vp, vp, ctypes.c_int, vp, vp, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                                        vp, vp, vp, vp, i32, i32, i32, vp, i32, i32,
                                        vp, vp, vp, i32, vp, i32, vp, sz, vp]
    lib.pkv_copy_blocks.restype = ctypes.c_int
    lib.pkv_copy_blocks.argtypes = [vp, vp, ctypes.c_int, i32, i32, i32, i32, vp, i32, vp]
    u64, ip = ctypes.c_uint64, ctypes.POINTER(ctypes.c_int32)
    lib.pkv_block_manager_create.restype = vp
    lib.pkv_block_manager_create.argtypes = [i32, i32]
    lib.pkv_block_manager_destroy.restype = None
    lib.pkv_block_manager_destroy.argtypes = [vp]
    lib.pkv_block_manager_num_free.restype = i32
    lib.pkv_block_manager_num_free.argtypes = [vp]
    lib.pkv_block_manager_refcount.restype = i32
    lib.pkv_block_manager_refcount.argtypes = [vp, i32]
    lib.pkv_block_manager_allocate.restype = ctypes.c_int
    lib.pkv_block_manager_allocate.argtypes = [vp, i32, ip]
    lib.pkv_block_manager_share.restype = ctypes.c_int
    lib.pkv_block_manager_share.argtypes = [vp, ip, i32]
    lib.pkv_block_manager_release.restype = ctypes.c_int
    lib.pkv_block_manager_release.argtypes = [vp, ip, i32]
    lib.pkv_block_manager_fork.restype = ctypes.c_int
    lib.pkv_block_manager_fork.argtypes = [vp, ip, i32, ip, i32]
    lib.pkv_block_manager_append_slot.restype = ctypes.c_int
    lib.pkv_block_manager_append_slot.argtypes = [vp, ip, i32, i32, ip, ip]
    lib.pkv_block_hash.restype = u64
    lib.pkv_block_hash.argtypes = [u64, ip, i32]
    lib.pkv_block_manager_lookup.restype = i32
    lib.pkv_block_manager_lookup.argtypes = [vp, u64]
    lib.pkv_block_manager_register.restype = ctypes.c_int
    lib.pkv_block_manager_register.argtypes = [vp, i32, u64]
    return lib


_LIB = None


def library():
    """The loaded ``libpkv.so`` (ctypes handle); raises ImportError if it is not built."""
    global _LIB
    if _LIB is None:
        _LIB = _load_library()
    return _LIB


def _check(code):
    if code != OK:
        raise PkvError(code, library().pkv_last_error().decode())


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    if t.dtype == torch.int8:
        return INT8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def kv_cache_write(k, v, k_cache, v_cache, slot_map, k_scale=None, v_scale=None, stream=None):
    """Store ``k[t]`` and ``v[t]`` ([T, Hkv, D]) at cache slot ``slot_map[t]`` (-1 skips).

    Caches are ``[num_blocks, block_size, Hkv, D]`` (fp32, bf16, uint8 /
    float8_e4m3fn E4M3 codes or int8 codes, the one-byte ones with per-head
    fp32 ``k_scale``/``v_scale``).
    """
    _require(k.dim() == 3 and v.shape == k.shape, "k and v must be [T, Hkv, D]")
    _require(k.stride(2) == 1 and k.stride(1) == k.shape[2], "k heads/dims must be contiguous")
    _require(v.stride(2) == 1 and v.stride(1) == v.shape[2], "v heads/dims must be contiguous")
    _require(k_cache.is_contiguous() and v_cache.is_contiguous() and k_cache.dim() == 4,
             "caches must be contiguous [num_blocks, block_size, Hkv, D]")
    _require(slot_map.numel() == k.shape[0], "one slot per token")
    t, hkv, d = k.shape
    _check(library().pkv_kv_cache_write(
        _ptr(k), k.stride(0) if t > 0 else hkv * d, _ptr(v), v.stride(0) if t > 0 else hkv * d,
        _dtype_code(k), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        k_cache.shape[0] * k_cache.shape[1], _ptr(k_scale), _ptr(v_scale), _ptr(slot_map), t, hkv, d,
        _stream(stream)))


def paged_decode_workspace_size(batch, num_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, split_keys=0):
    return int(library().pkv_paged_decode_workspace_size(batch, num_heads, num_kv_heads, head_dim,
                                                   block_size, max_blocks_per_seq, split_keys))


def paged_decode(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale, k_scale=None,
                 v_scale=None, out=None, split_keys=0, workspace=None, stream=None):
    """One query per sequence: q [B, Hq, D] -> out [B, Hq, D] (q's dtype)."""
    import torch
    _require(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B, Hq, D]")
    _require(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    _require(block_table.dim() == 2 and block_table.is_contiguous() and
             block_table.dtype == torch.int32, "block_table must be contiguous int32 [B, max_blocks]")
    _require(cache_seqlens.dtype == torch.int32, "cache_seqlens must be int32")
    b, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    need = paged_decode_workspace_size(b, hq, hkv, d, bs, block_table.shape[1], split_keys)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pkv_paged_decode(
        _ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
        b, hq, hkv, d, bs, nb, float(softmax_scale), int(split_keys), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return out


def paged_decode_noalloc(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale, k_scale=None,
                         v_scale=None, out=None, split_keys=0, stream=None):
    """``paged_decode`` with the library's static scratch array instead of a workspace:
    the C call allocates nothing (``out`` is allocated here only when not given)."""
    import torch
    _require(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B, Hq, D]")
    _require(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    _require(block_table.dim() == 2 and block_table.is_contiguous() and
             block_table.dtype == torch.int32, "block_table must be contiguous int32 [B, max_blocks]")
    _require(cache_seqlens.dtype == torch.int32, "cache_seqlens must be int32")
    b, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    _check(library().pkv_paged_decode_noalloc(
        _ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
        b, hq, hkv, d, bs, nb, float(softmax_scale), int(split_keys), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def paged_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, softmax_scale,
                        k_scale=None, v_scale=None, out=None, split_keys=0, workspace=None, stream=None):
    """Store ``k_new[b]``/``v_new[b]`` ([B, Hkv, D]) at position ``cache_seqlens[b]`` of
    sequence b, then decode q [B, Hq, D] over the ``cache_seqlens[b] + 1`` keys."""
    import torch
    _require(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B, Hq, D]")
    _require(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    _require(block_table.dim() == 2 and block_table.is_contiguous() and
             block_table.dtype == torch.int32, "block_table must be contiguous int32 [B, max_blocks]")
    _require(cache_seqlens.dtype == torch.int32, "cache_seqlens must be int32")
    b, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    _require(k_new.dim() == 3 and tuple(k_new.shape) == (b, hkv, d) and v_new.shape == k_new.shape,
             "k_new and v_new must be [B, Hkv, D]")
    _require(k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new and v_new must have q's dtype")
    _require(k_new.stride(2) == 1 and k_new.stride(1) == d, "k_new heads/dims must be contiguous")
    _require(v_new.stride(2) == 1 and v_new.stride(1) == d, "v_new heads/dims must be contiguous")
    if out is None:
        out = torch.empty_like(q)
    need = paged_decode_workspace_size(b, hq, hkv, d, bs, block_table.shape[1], split_keys)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pkv_paged_decode_append(
        _ptr(out), _ptr(q), _dtype_code(q), _ptr(k_new), k_new.stride(0), _ptr(v_new), v_new.stride(0),
        _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), b, hq, hkv, d, bs, nb,
        float(softmax_scale), int(split_keys), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def varlen_prefill(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale,
                   causal=True, block_table=None, k_scale=None, v_scale=None, out=None, stream=None):
    """Packed varlen attention: q [sum Lq, Hq, D] -> out [sum Lq, Hq, D].

    Without ``block_table`` k/v are packed [sum Lk, Hkv, D]; with it they are
    the paged caches [num_blocks, block_size, Hkv, D].
    """
    import torch
    _require(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [sum Lq, Hq, D]")
    _require(k.is_contiguous() and v.is_contiguous(), "k and v must be contiguous")
    _require(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32,
             "cu_seqlens must be int32")
    total_q, hq, d = q.shape
    batch = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    if block_table is not None:
        _require(block_table.dim() == 2 and block_table.is_contiguous() and
                 block_table.dtype == torch.int32, "block_table must be contiguous int32")
        nb, bs, hkv, _ = k.shape
        maxblk, total_k = block_table.shape[1], 0
    else:
        nb, bs, maxblk = 0, 0, 0
        total_k, hkv = k.shape[0], k.shape[1]
    _check(library().pkv_varlen_prefill(
        _ptr(out), _ptr(q), _dtype_code(q), _ptr(k), _ptr(v), _dtype_code(k), _ptr(k_scale),
        _ptr(v_scale), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, int(max_seqlen_q),
        int(max_seqlen_k), float(softmax_scale), int(bool(causal)), _ptr(block_table), maxblk, bs, nb,
        hq, hkv, d, total_q, total_k, _stream(stream)))
    return out


def mixed_attention(k_cache, v_cache, softmax_scale, prefill=None, decode=None, k_scale=None, v_scale=None,
                    workspace=None, stream=None):
    """A chunked-prefill step's attention in one call.

    ``prefill``: dict(q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
    block_table[, out]) as for :func:`varlen_prefill` (causal, paged);
    ``decode``: dict(q, block_table, cache_seqlens[, out]) as for
    :func:`paged_decode`.  Returns (prefill_out, decode_out) (None for a
    missing part)."""
    import torch
    _require(k_cache.is_contiguous() and v_cache.is_contiguous() and k_cache.dim() == 4,
             "caches must be contiguous [num_blocks, block_size, Hkv, D]")
    nb, bs, hkv, d = k_cache.shape
    p_out = d_out = None
    pq = pcq = pck = pbt = None
    pb = mq = mk = pmax = tq = 0
    hq = None
    q_dtype = None
    if prefill is not None:
        pq = prefill["q"]
        _require(pq.dim() == 3 and pq.is_contiguous(), "prefill q must be contiguous [sum Lq, Hq, D]")
        pbt = prefill["block_table"]
        _require(pbt.dim() == 2 and pbt.is_contiguous() and pbt.dtype == torch.int32,
                 "prefill block_table must be contiguous int32")
        pcq, pck = prefill["cu_seqlens_q"], prefill["cu_seqlens_k"]
        _require(pcq.dtype == torch.int32 and pck.dtype == torch.int32, "cu_seqlens must be int32")
        p_out = prefill.get("out")
        p_out = torch.empty_like(pq) if p_out is None else p_out
        pb, mq, mk, pmax, tq = pcq.numel() - 1, int(prefill["max_seqlen_q"]), int(prefill["max_seqlen_k"]), \
            pbt.shape[1], pq.shape[0]
        hq, q_dtype = pq.shape[1], pq.dtype
    dq = dbt = dlen = None
    db = dmax = 0
    if decode is not None:
        dq = decode["q"]
        _require(dq.dim() == 3 and dq.is_contiguous(), "decode q must be contiguous [B, Hq, D]")
        dbt, dlen = decode["block_table"], decode["cache_seqlens"]
        _require(dbt.dim() == 2 and dbt.is_contiguous() and dbt.dtype == torch.int32,
                 "decode block_table must be contiguous int32")
        _require(dlen.dtype == torch.int32, "cache_seqlens must be int32")
        d_out = decode.get("out")
        d_out = torch.empty_like(dq) if d_out is None else d_out
        db, dmax = dq.shape[0], dbt.shape[1]
        _require(hq is None or hq == dq.shape[1], "prefill and decode q must have the same heads")
        hq, q_dtype = dq.shape[1], dq.dtype
        need = paged_decode_workspace_size(db, hq, hkv, d, bs, dmax, 0)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dq.device)
    if hq is None:
        return None, None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    qcode = F32 if q_dtype == torch.float32 else BF16
    _check(library().pkv_mixed_attention(
        _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale), nb, bs, hq, hkv, d,
        float(softmax_scale), qcode, _ptr(p_out), _ptr(pq), _ptr(pcq), _ptr(pck), pb, mq, mk, _ptr(pbt), pmax, tq,
        _ptr(d_out), _ptr(dq), _ptr(dbt), dmax, _ptr(dlen), db, _ptr(workspace), ws_bytes, _stream(stream)))
    return p_out, d_out


def copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """Copy block ``src`` to block ``dst`` of both caches for every row
    ``(src, dst)`` of ``block_pairs`` ([n, 2] int32, device)."""
    import torch
    _require(k_cache.is_contiguous() and v_cache.is_contiguous() and k_cache.dim() == 4 and
             v_cache.shape == k_cache.shape, "caches must be contiguous [num_blocks, block_size, Hkv, D]")
    _require(block_pairs.dtype == torch.int32 and block_pairs.is_contiguous() and
             (block_pairs.numel() == 0 or (block_pairs.dim() == 2 and block_pairs.shape[1] == 2)),
             "block_pairs must be contiguous int32 [n, 2]")
    nb, bs, hkv, d = k_cache.shape
    n = block_pairs.shape[0] if block_pairs.numel() else 0
    _check(library().pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), nb, bs, hkv, d,
                                     _ptr(block_pairs), n, _stream(stream)))


def _i32_array(values):
    values = list(values)
    return (ctypes.c_int32 * max(1, len(values)))(*values), len(values)


class BlockManager:
    """Host-side allocator of a pool's physical blocks (``pkv_block_manager_*``):
    reference counts, forks that share blocks, copy-on-write decisions and
    prefix hashes.  Block-table rows are plain Python lists of ints here."""

    def __init__(self, num_blocks, block_size):
        self._lib = library()
        self._h = self._lib.pkv_block_manager_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if self._h:
            self._lib.pkv_block_manager_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def _ok(self, code, what):
        if code != OK:
            raise PkvError(code, f"block manager: {what} refused")

    @property
    def num_free(self):
        return int(self._lib.pkv_block_manager_num_free(self._h))

    def refcount(self, block):
        return int(self._lib.pkv_block_manager_refcount(self._h, int(block)))

    def allocate(self, n):
        arr, _ = _i32_array([0] * n)
        self._ok(self._lib.pkv_block_manager_allocate(self._h, int(n), arr), f"allocate({n})")
        return list(arr)[:n]

    def share(self, blocks):
        arr, n = _i32_array(blocks)
        self._ok(self._lib.pkv_block_manager_share(self._h, arr, n), "share")

    def release(self, blocks):
        arr, n = _i32_array(blocks)
        self._ok(self._lib.pkv_block_manager_release(self._h, arr, n), "release")

    def fork(self, parent_row, num_tokens):
        parent, width = _i32_array(parent_row)
        child, _ = _i32_array([-1] * width)
        self._ok(self._lib.pkv_block_manager_fork(self._h, parent, int(num_tokens), child, width), "fork")
        return list(child)[:width]

    def append_slot(self, row, num_tokens):
        """Slot of the token at position ``num_tokens``; ``row`` (a list) is
        updated in place.  Returns (slot, copy) with copy = (src, dst) or None."""
        arr, width = _i32_array(row)
        slot = ctypes.c_int32(0)
        copy = (ctypes.c_int32 * 2)()
        self._ok(self._lib.pkv_block_manager_append_slot(self._h, arr, width, int(num_tokens),
                                                         ctypes.byref(slot), copy), "append_slot")
        row[:] = list(arr)[:width]
        return int(slot.value), (None if copy[0] < 0 else (int(copy[0]), int(copy[1])))

    def lookup(self, block_hash):
        return int(self._lib.pkv_block_manager_lookup(self._h, int(block_hash)))

    def register(self, block, block_hash):
        code = self._lib.pkv_block_manager_register(self._h, int(block), int(block_hash))
        if code not in (OK, 1):
            self._ok(code, "register")
        return code == OK


def block_hash(parent_hash, tokens):
    """Chained hash of one full block of token ids (``pkv_block_hash``)."""
    arr, n = _i32_array(tokens)
    return int(library().pkv_block_hash(int(parent_hash), arr, n))


def version():
    return library().pkv_version().decode()
