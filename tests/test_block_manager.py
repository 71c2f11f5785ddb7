"""The host-side block manager (CPU): hand-made copy-on-write scenarios, then
random operation sequences checked step by step against the plain model in
``oracle/blocks.py``."""

import numpy as np
import pytest

import paged_kv_cache_map_amd as pkv
from oracle import blocks


def test_model_fork_then_write_copies_only_the_shared_partial_block():
    """[ch15] PagedAttention section: two answers of one prompt share its
    blocks; the first write into a shared block copies that block only."""
    m = blocks.BlockModel(8, 4)
    row = [-1, -1, -1]
    for t in range(6):  # a 6-token prompt: blocks for positions 0-3 and 4-5
        chosen = _grow(row, t, m)
        slot = m.append(row, t, chosen, None)
        row[:] = chosen
        assert slot // 4 == row[t // 4] and slot % 4 == t % 4
    full, part = row[0], row[1]
    child = list(row)
    m.share(full)
    m.share(part)
    assert m.ref[full] == 2 and m.ref[part] == 2
    new = min(m.free_blocks())
    chosen = [full, new, -1]
    slot = m.append(child, 6, chosen, (part, new))
    assert slot == new * 4 + 2
    assert m.ref[full] == 2 and m.ref[part] == 1 and m.ref[new] == 1
    with pytest.raises(AssertionError):  # a copy that is not needed is an error
        blocks.BlockModel(8, 4).append([-1], 1, [3], (0, 3))


def _grow(row, t, m):
    """The choice a correct manager makes for an unshared sequence."""
    out = list(row)
    if t % m.block_size == 0:
        out[t // m.block_size] = min(m.free_blocks())
    return out


def test_copy_blocks_reference():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    v = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    k2, v2 = blocks.copy_blocks(k, v, [(1, 4), (1, 5), (0, 3)])
    for s, d in ((1, 4), (1, 5), (0, 3)):
        assert k2[d].tobytes() == k[s].tobytes() and v2[d].tobytes() == v[s].tobytes()
    for b in (0, 1, 2):
        assert k2[b].tobytes() == k[b].tobytes() and v2[b].tobytes() == v[b].tobytes()
    with pytest.raises(AssertionError):
        blocks.copy_blocks(k, v, [(1, 4), (4, 5)])  # a target that is also a source


# ---------------------------------------------------------------------------
# the library
# ---------------------------------------------------------------------------


def test_allocate_share_release_counts():
    bm = pkv.BlockManager(5, 16)
    assert bm.num_free == 5
    got = bm.allocate(3)
    assert len(set(got)) == 3 and bm.num_free == 2
    bm.share(got[:1])
    assert bm.refcount(got[0]) == 2
    bm.release([got[0], got[0]])
    assert bm.refcount(got[0]) == 0 and bm.num_free == 3
    with pytest.raises(pkv.PkvError):
        bm.release([got[0]])  # not held
    with pytest.raises(pkv.PkvError):
        bm.allocate(4)        # only 3 free: nothing is allocated
    assert bm.num_free == 3
    with pytest.raises(pkv.PkvError):
        bm.share([7])         # outside the pool
    assert bm.refcount(9) == -1


def test_fork_and_copy_on_write():
    bm = pkv.BlockManager(6, 4)
    row = [-1] * 4
    for t in range(6):
        slot, copy = bm.append_slot(row, t)
        assert copy is None and slot == row[t // 4] * 4 + t % 4
    child = bm.fork(row, 6)
    assert child == row and bm.refcount(row[0]) == 2 and bm.refcount(row[1]) == 2
    slot, copy = bm.append_slot(child, 6)
    assert copy == (row[1], child[1]) and child[1] != row[1] and child[0] == row[0]
    assert slot == child[1] * 4 + 2
    assert bm.refcount(row[1]) == 1 and bm.refcount(child[1]) == 1 and bm.refcount(row[0]) == 2
    # the parent now owns its partial block alone: no copy
    slot, copy = bm.append_slot(row, 6)
    assert copy is None and slot == row[1] * 4 + 2
    # a new logical block is never a copy
    slot, copy = bm.append_slot(row, 8)
    assert copy is None and row[2] >= 0 and slot == row[2] * 4


def test_append_without_free_block_changes_nothing():
    bm = pkv.BlockManager(2, 4)
    row = [-1, -1]
    bm.append_slot(row, 0)
    child = bm.fork(row, 1)
    bm.append_slot(child, 1)             # copy: the pool is now full
    assert bm.num_free == 0
    before = (list(row), [bm.refcount(b) for b in range(2)])
    with pytest.raises(pkv.PkvError):
        bm.append_slot(row, 4)           # needs a new block
    assert (list(row), [bm.refcount(b) for b in range(2)]) == before


def test_prefix_hash_lookup_register_and_eviction():
    bs = 4
    bm = pkv.BlockManager(3, bs)
    prompt = [11, 12, 13, 14, 15, 16, 17, 18]
    h0 = pkv.block_hash(0, prompt[:4])
    h1 = pkv.block_hash(h0, prompt[4:])
    assert h0 != h1 and pkv.block_hash(0, prompt[:4]) == h0
    assert pkv.block_hash(0, [11, 12, 13, 15]) != h0
    assert pkv.block_hash(1, prompt[:4]) != h0        # chained: the parent matters
    assert bm.lookup(h0) == -1
    a, b = bm.allocate(2)
    assert bm.register(a, h0) and bm.register(b, h1)
    assert not bm.register(b, h0)                       # another block holds h0
    assert bm.lookup(h0) == a and bm.refcount(a) == 2   # a second request reuses it
    bm.release([a, a, b])
    assert bm.num_free == 3                             # cached blocks count as free
    assert bm.lookup(h1) == b and bm.refcount(b) == 1   # revived
    bm.release([b])
    # the fresh block goes first, then the one released longest ago (a)
    first, second = bm.allocate(2)
    assert bm.refcount(first) == 1 and first not in (a, b) and second == a
    assert bm.lookup(h0) == -1 and bm.lookup(h1) == b


def test_append_into_registered_block_copies():
    bm = pkv.BlockManager(4, 4)
    row = [-1, -1]
    for t in range(3):
        bm.append_slot(row, t)
    assert bm.register(row[0], 1234)
    old = row[0]
    slot, copy = bm.append_slot(row, 3)
    assert copy == (old, row[0]) and row[0] != old and slot == row[0] * 4 + 3
    assert bm.lookup(1234) == old


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_the_model(seed):
    """Random allocate / fork / append / release / prefix operations: after
    every step the library's counts equal the model's, every copy it asks for
    is one the model requires, and every block's holders are exactly the
    sequences whose rows name it."""
    rng = np.random.default_rng(seed)
    nb, bs, width = 24, 4, 8
    bm = pkv.BlockManager(nb, bs)
    model = blocks.BlockModel(nb, bs)
    seqs = {}  # id -> (row, tokens)
    extra = []  # blocks held by lookups (a request that reuses a prefix)
    next_id = 0
    for _ in range(500):
        op = rng.choice(["new", "append", "append", "append", "fork", "free", "register", "lookup",
                         "drop"])
        if op == "new" or not seqs:
            seqs[next_id] = ([-1] * width, 0)
            next_id += 1
            continue
        sid = list(seqs)[int(rng.integers(len(seqs)))]
        row, n = seqs[sid]
        used = -(-n // bs)
        if op == "append":
            if n >= width * bs:
                continue
            lib_row = list(row)
            try:
                slot, copy = bm.append_slot(lib_row, n)
            except pkv.PkvError:
                assert lib_row == row and bm.num_free == 0
                continue
            assert slot == model.append(row, n, lib_row, copy)
            seqs[sid] = (lib_row, n + 1)
        elif op == "fork":
            child = bm.fork(row, n)
            for b in row[:used]:
                model.share(b)
            assert child[:used] == row[:used] and all(x == -1 for x in child[used:])
            seqs[next_id] = (child, n)
            next_id += 1
        elif op == "free":
            bm.release(row[:used])
            for b in row[:used]:
                model.release(b)
            del seqs[sid]
        elif op == "register":
            if n // bs == 0:
                continue
            b = row[int(rng.integers(n // bs))]
            h = int(rng.integers(1, 1 << 62))
            assert bm.register(b, h)
            model.hash[b] = h
        elif op == "lookup":
            if not model.hash or rng.random() < 0.2:
                assert bm.lookup(int(rng.integers(1 << 62, 1 << 63))) == -1
                continue
            b, h = list(model.hash.items())[int(rng.integers(len(model.hash)))]
            assert bm.lookup(h) == b
            model.ref[b] += 1
            extra.append(b)
        elif op == "drop" and extra:
            b = extra.pop(int(rng.integers(len(extra))))
            bm.release([b])
            model.release(b)
        assert [bm.refcount(b) for b in range(nb)] == model.ref
        assert bm.num_free == model.num_free()
        held = [b for r, n2 in seqs.values() for b in r[:-(-n2 // bs)]] + extra
        for b in range(nb):
            assert model.ref[b] == held.count(b), b


def _fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit: offset basis 14695981039346656037, prime 1099511628211
    (the published parameters of the Fowler/Noll/Vo hash)."""
    h = 14695981039346656037
    for byte in data:
        h = ((h ^ byte) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def test_fnv1a64_reference_matches_published_vectors():
    # test vectors published with the FNV hash: the empty string hashes to the
    # offset basis itself
    assert _fnv1a64(b"") == 0xCBF29CE484222325
    assert _fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert _fnv1a64(b"foobar") == 0x85944171F73967E8


@pytest.mark.parametrize("parent,tokens", [
    (0, []),
    (0, [11, 12, 13, 14]),
    (0xCBF29CE484222325, [0, 1, 2, 3, 4, 5, 6, 7]),
    (0xFFFFFFFFFFFFFFFF, [2 ** 31 - 1, 0, 65535, 7]),
])
def test_block_hash_is_fnv1a64_of_parent_and_tokens(parent, tokens):
    """pkv_block_hash = FNV-1a-64 over the parent hash (8 bytes) and the token
    ids (4 bytes each), little-endian."""
    data = parent.to_bytes(8, "little") + b"".join(t.to_bytes(4, "little", signed=True) for t in tokens)
    assert pkv.block_hash(parent, tokens) == _fnv1a64(data)
