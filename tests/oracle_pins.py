"""Checks that pin the oracle to things other than itself.

Each ``check_*`` takes the oracle module under test (``oracle.paged`` or a
deliberately broken copy of it) and raises ``AssertionError`` when the module
disagrees with:

* the worked examples the pages print (``tests/golden/``),
* a library routine the method reduces to in a special case
  (``torch.nn.functional.scaled_dot_product_attention`` in float64), or
* an exact special case / invariant of softmax attention over a paged cache.

``test_oracle.py`` runs them on the real oracle; ``test_oracle_mutations.py``
runs them on planted mistakes to show that each plausible mistake is caught.
"""

import json
import math
import pathlib

import numpy as np
import torch

GOLDEN = pathlib.Path(__file__).parent / "golden"


def load_golden(name):
    return json.loads((GOLDEN / name).read_text())


def _sdpa(q, k, v, scale, causal):
    """Library attention, float64 CPU: q [Lq,Hq,D], k/v [Lk,Hkv,D] (GQA by
    repeating each KV head over its contiguous group of q heads)."""
    hq, hkv = q.shape[1], k.shape[1]
    kk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1)
    vv = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1)
    qq = torch.from_numpy(q)
    out = torch.nn.functional.scaled_dot_product_attention(
        qq.transpose(0, 1)[None], kk.transpose(0, 1)[None], vv.transpose(0, 1)[None],
        is_causal=causal, scale=scale)
    return out[0].transpose(0, 1).numpy()


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _paged_from_contig(rng, k, v, block_size, extra_blocks=2, poison=True):
    """Scatter contiguous per-sequence K/V into a randomly permuted block pool.

    Written here, independently of the oracle's write, so that the gather is
    checked against data placed by other code.  Returns (k_cache, v_cache, table).
    """
    seqs = len(k)
    nblk = [max(1, -(-len(kk) // block_size)) for kk in k]
    num_blocks = sum(nblk) + extra_blocks
    perm = rng.permutation(num_blocks)
    hkv, d = k[0].shape[1], k[0].shape[2]
    fill = np.nan if poison else 0.0
    kc = np.full((num_blocks, block_size, hkv, d), fill)
    vc = np.full((num_blocks, block_size, hkv, d), fill)
    table = np.full((seqs, max(nblk) + 1), -1, dtype=np.int32)
    off = 0
    for s in range(seqs):
        ids = perm[off:off + nblk[s]]
        off += nblk[s]
        table[s, :nblk[s]] = ids
        for j in range(len(k[s])):
            kc[ids[j // block_size], j % block_size] = k[s][j]
            vc[ids[j // block_size], j % block_size] = v[s][j]
    return kc, vc, table


# ---------------------------------------------------------------------------
# worked examples
# ---------------------------------------------------------------------------


def check_varlen_example(paged):
    g = load_golden("page2_varlen_example.json")
    cu_q = paged.cu_seqlens(g["q_lens"])
    cu_k = paged.cu_seqlens(g["k_lens"])
    assert list(cu_q) == g["cu_seqlens_q"]
    assert list(cu_k) == g["cu_seqlens_k"]
    assert int(np.max(np.diff(cu_q))) == g["max_seqlen_q"]
    assert int(np.max(np.diff(cu_k))) == g["max_seqlen_k"]
    assert int(cu_q[-1]) == g["q_tokens"] and int(cu_k[-1]) == g["k_tokens"]
    assert list(paged.request_index(cu_q)) == g["q_request_index"]
    assert list(paged.request_index(cu_k)) == g["k_request_index"]


def check_decode_example(paged):
    g = load_golden("page2_decode_example.json")
    p, dv = g["printed"], g["derived"]
    bs = p["block_size"]
    table = np.array(p["block_table"], dtype=np.int32)
    slots = [paged.slot_of(table[b], p["cache_seqlens"][b], bs) for b in range(3)]
    assert slots == dv["new_token_slots"]
    after = [paged.blocks_needed(n + 1, bs) for n in p["cache_seqlens"]]
    assert after == dv["blocks_after_append"]
    # the allocated entries of each row are exactly the blocks needed after the append
    assert after == [int((row >= 0).sum()) for row in table]
    # sequence 0's new token stays in its first block; sequence 1 moves to its second
    assert [n // bs for n in p["cache_seqlens"]] == dv["new_token_logical_block"]


# ---------------------------------------------------------------------------
# dense attention special cases (library routine)
# ---------------------------------------------------------------------------


def check_dense_causal_square(paged, seed=0):
    """Lq == Lk: bottom-right and top-left causal coincide; compare with SDPA."""
    rng = np.random.default_rng(seed)
    for hq, hkv, lq, d in [(8, 2, 13, 16), (4, 4, 7, 8), (6, 1, 5, 32)]:
        q, k, v = _rand(rng, lq, hq, d), _rand(rng, lq, hkv, d), _rand(rng, lq, hkv, d)
        scale = 0.37
        got = paged.attention(q, k, v, scale, causal=True)
        want = _sdpa(q, k, v, scale, causal=True)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def check_dense_noncausal(paged, seed=1):
    rng = np.random.default_rng(seed)
    for hq, hkv, lq, lk, d in [(8, 2, 5, 19, 16), (4, 2, 11, 3, 8), (3, 3, 1, 40, 64)]:
        q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
        scale = 1.0 / math.sqrt(d)
        got = paged.attention(q, k, v, scale, causal=False)
        want = _sdpa(q, k, v, scale, causal=False)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def check_prefix_alignment(paged, seed=2):
    """A chunk of Lq queries after a prefix P (Lk = P + Lq): causal row i equals
    plain attention of that one query over the first P + i + 1 keys."""
    rng = np.random.default_rng(seed)
    hq, hkv, d, p, lq = 4, 2, 16, 9, 6
    lk = p + lq
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    got = paged.attention(q, k, v, 0.5, causal=True)
    for i in range(lq):
        want = _sdpa(q[i:i + 1], k[:p + i + 1], v[:p + i + 1], 0.5, causal=False)
        np.testing.assert_allclose(got[i:i + 1], want, rtol=1e-12, atol=1e-12)


def check_varlen_example_outputs(paged, seed=3):
    """The varlen example under the zero-output reading: r0 (no keys) -> 0;
    r1 causal rows 0-1 see nothing -> 0, row 2 sees its one key -> that V row
    exactly; non-causal every r1 row -> that V row exactly; r2 -> SDPA."""
    g = load_golden("page2_varlen_example.json")
    rng = np.random.default_rng(seed)
    hq, hkv, d = 4, 2, 8
    cu_q = np.array(g["cu_seqlens_q"])
    cu_k = np.array(g["cu_seqlens_k"])
    q = _rand(rng, int(cu_q[-1]), hq, d)
    k = _rand(rng, int(cu_k[-1]), hkv, d)
    v = _rand(rng, int(cu_k[-1]), hkv, d)
    qb, kb, vb = q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)
    out = paged.varlen_prefill(qb, "f32", kb, vb, "f32", cu_q, cu_k, 0.3, True)
    assert np.all(out[0:10] == 0.0)
    assert np.all(out[10:12] == 0.0)
    group = hq // hkv
    for h in range(hq):
        assert np.array_equal(out[12, h], vb[0, h // group].astype(np.float64))
    out_nc = paged.varlen_prefill(qb, "f32", kb, vb, "f32", cu_q, cu_k, 0.3, False)
    for r in (10, 11, 12):
        for h in range(hq):
            assert np.array_equal(out_nc[r, h], vb[0, h // group].astype(np.float64))
    want = _sdpa(qb[13:14].astype(np.float64), kb[1:8].astype(np.float64),
                 vb[1:8].astype(np.float64), 0.3, causal=False)
    np.testing.assert_allclose(out[13:14], want, rtol=1e-12, atol=1e-12)


def check_equal_keys_mean(paged, seed=4):
    """All keys equal -> uniform weights -> the mean of the visible V rows."""
    rng = np.random.default_rng(seed)
    lq, lk, d = 3, 10, 8
    q = _rand(rng, lq, 2, d)
    k = np.repeat(_rand(rng, 1, 1, d), lk, axis=0)
    v = _rand(rng, lk, 1, d)
    out = paged.attention(q, k, v, 1.0, causal=True)
    for i in range(lq):
        vis = lk - lq + i + 1
        np.testing.assert_allclose(out[i, 0], v[:vis, 0].mean(axis=0), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(out[i, 1], v[:vis, 0].mean(axis=0), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# paging: gather through the block table
# ---------------------------------------------------------------------------


def check_paged_decode_matches_dense(paged, seed=5):
    """Decode over a randomly permuted, NaN-poisoned pool equals SDPA of the
    single query over the contiguous keys, for two different permutations."""
    rng = np.random.default_rng(seed)
    hq, hkv, d, bs = 8, 2, 16, 4
    lens = [1, 4, 5, 13, 16]
    ks = [_rand(rng, n, hkv, d) for n in lens]
    vs = [_rand(rng, n, hkv, d) for n in lens]
    q = _rand(rng, len(lens), hq, d)
    outs = []
    for perm_seed in (11, 12):
        kc, vc, table = _paged_from_contig(np.random.default_rng(perm_seed), ks, vs, bs)
        out = paged.paged_decode(q.astype(np.float32), "f32", kc.astype(np.float32), vc.astype(np.float32),
                                 "f32", table, np.array(lens, np.int32), 0.25)
        assert np.all(np.isfinite(out))
        outs.append(out)
        for b, n in enumerate(lens):
            want = _sdpa(q[b:b + 1].astype(np.float32).astype(np.float64),
                         ks[b].astype(np.float32).astype(np.float64),
                         vs[b].astype(np.float32).astype(np.float64), 0.25, causal=False)
            np.testing.assert_allclose(out[b:b + 1], want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(outs[0], outs[1])


def check_paged_prefill_matches_contig(paged, seed=6):
    """Varlen through a block table equals varlen on the packed contiguous K/V."""
    rng = np.random.default_rng(seed)
    hq, hkv, d, bs = 4, 2, 8, 8
    q_lens, k_lens = [3, 1, 7], [3, 9, 20]
    ks = [_rand(rng, n, hkv, d) for n in k_lens]
    vs = [_rand(rng, n, hkv, d) for n in k_lens]
    q = _rand(rng, sum(q_lens), hq, d).astype(np.float32)
    kc, vc, table = _paged_from_contig(np.random.default_rng(7), ks, vs, bs)
    cu_q = paged.cu_seqlens(q_lens)
    cu_k = paged.cu_seqlens(k_lens)
    a = paged.varlen_prefill(q, "f32", kc.astype(np.float32), vc.astype(np.float32), "f32",
                             cu_q, cu_k, 0.3, True, block_table=table)
    b = paged.varlen_prefill(q, "f32", np.concatenate(ks).astype(np.float32),
                             np.concatenate(vs).astype(np.float32), "f32", cu_q, cu_k, 0.3, True)
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(a, b)


def check_decode_is_varlen_with_one_query(paged, seed=8):
    rng = np.random.default_rng(seed)
    hq, hkv, d, bs = 6, 3, 8, 4
    lens = [2, 9, 12]
    ks = [_rand(rng, n, hkv, d) for n in lens]
    vs = [_rand(rng, n, hkv, d) for n in lens]
    q = _rand(rng, 3, hq, d).astype(np.float32)
    kc, vc, table = _paged_from_contig(np.random.default_rng(9), ks, vs, bs)
    kc, vc = kc.astype(np.float32), vc.astype(np.float32)
    dec = paged.paged_decode(q, "f32", kc, vc, "f32", table, np.array(lens, np.int32), 0.7)
    var = paged.varlen_prefill(q, "f32", kc, vc, "f32", paged.cu_seqlens([1, 1, 1]),
                               paged.cu_seqlens(lens), 0.7, True, block_table=table)
    np.testing.assert_array_equal(dec, var)


# ---------------------------------------------------------------------------
# the write
# ---------------------------------------------------------------------------


def check_write_example(paged, seed=10):
    """The decode example's step: three new tokens land at slots 94, 32, 198 of
    an 8-block pool; every other byte of both caches is unchanged."""
    g = load_golden("page2_decode_example.json")
    p = g["printed"]
    bs = p["block_size"]
    table = np.array(p["block_table"], dtype=np.int32)
    rng = np.random.default_rng(seed)
    hkv, d = 2, 64
    kc = rng.standard_normal((8, bs, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((8, bs, hkv, d)).astype(np.float32)
    kn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([paged.slot_of(table[b], p["cache_seqlens"][b], bs) for b in range(3)], np.int32)
    k2, v2 = paged.kv_cache_write(kn, vn, kc, vc, slots, "f32", "f32")
    flat_k_old, flat_k = kc.reshape(-1, hkv, d), k2.reshape(-1, hkv, d)
    flat_v_old, flat_v = vc.reshape(-1, hkv, d), v2.reshape(-1, hkv, d)
    changed = [s for s in range(8 * bs) if not np.array_equal(flat_k[s], flat_k_old[s])]
    assert sorted(changed) == sorted(g["derived"]["new_token_slots"])
    for t, s in enumerate(g["derived"]["new_token_slots"]):
        assert flat_k[s].tobytes() == kn[t].tobytes()
        assert flat_v[s].tobytes() == vn[t].tobytes()
    untouched = np.ones(8 * bs, bool)
    untouched[g["derived"]["new_token_slots"]] = False
    assert flat_k[untouched].tobytes() == flat_k_old[untouched].tobytes()
    assert flat_v[untouched].tobytes() == flat_v_old[untouched].tobytes()


# ---------------------------------------------------------------------------
# the decode that stores its own token ([paged-doc] "デコードパス", キャッシュの動作)
# ---------------------------------------------------------------------------


def check_append_example(paged, seed=12):
    """The decode example as one appending step: lengths [30, 32, 70] before
    the step; the three new rows land at slots 94, 32, 198 (nothing else in
    the pool changes) and each output is SDPA over the sequence's keys in
    order, the new one last, walked here through the printed table."""
    g = load_golden("page2_decode_example.json")
    p = g["printed"]
    bs = p["block_size"]
    table = np.array(p["block_table"], dtype=np.int32)
    lens = p["cache_seqlens"]
    rng = np.random.default_rng(seed)
    hq, hkv, d = 8, 2, 64
    kc = rng.standard_normal((8, bs, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((8, bs, hkv, d)).astype(np.float32)
    kn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    q = rng.standard_normal((3, hq, d)).astype(np.float32)
    out, k2, v2 = paged.paged_decode_append(q, "f32", kn, vn, kc, vc, "f32", table,
                                            np.array(lens, np.int32), 0.125)
    slots = g["derived"]["new_token_slots"]
    fk_old, fk = kc.reshape(-1, hkv, d), k2.reshape(-1, hkv, d)
    fv_old, fv = vc.reshape(-1, hkv, d), v2.reshape(-1, hkv, d)
    changed = [s for s in range(8 * bs) if not np.array_equal(fk[s], fk_old[s])]
    assert sorted(changed) == sorted(slots)
    for b, s in enumerate(slots):
        assert fk[s].tobytes() == kn[b].tobytes() and fv[s].tobytes() == vn[b].tobytes()
    keep = np.ones(8 * bs, bool)
    keep[slots] = False
    assert fv[keep].tobytes() == fv_old[keep].tobytes()
    for b, n in enumerate(lens):
        walk = [table[b][j // bs] * bs + j % bs for j in range(n)]
        kk = np.concatenate([fk_old[walk], kn[b][None]]).astype(np.float64)
        vv = np.concatenate([fv_old[walk], vn[b][None]]).astype(np.float64)
        want = _sdpa(q[b:b + 1].astype(np.float64), kk, vv, 0.125, causal=False)
        np.testing.assert_allclose(out[b:b + 1], want, rtol=1e-12, atol=1e-12)


def check_append_to_empty_sequence(paged, seed=13):
    """A sequence with no cached key attends to its new token alone: every q
    head returns the new V row of its KV head exactly (softmax of one logit)."""
    rng = np.random.default_rng(seed)
    hq, hkv, d, bs = 6, 2, 8, 4
    kc = np.full((3, bs, hkv, d), np.nan, np.float32)
    vc = np.full((3, bs, hkv, d), np.nan, np.float32)
    table = np.array([[2, -1], [0, 1]], np.int32)
    kc[0], vc[0] = rng.standard_normal((2, bs, hkv, d)).astype(np.float32)
    kc[1, :1], vc[1, :1] = rng.standard_normal((2, 1, hkv, d)).astype(np.float32)
    kn = rng.standard_normal((2, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((2, hkv, d)).astype(np.float32)
    q = rng.standard_normal((2, hq, d)).astype(np.float32)
    out, _, _ = paged.paged_decode_append(q, "f32", kn, vn, kc, vc, "f32", table,
                                          np.array([0, 5], np.int32), 0.9)
    for h in range(hq):
        assert np.array_equal(out[0, h], vn[0, h // (hq // hkv)].astype(np.float64))
    assert np.all(np.isfinite(out[1]))


# ---------------------------------------------------------------------------
# the int8 codec (a reading: symmetric, round half to even, saturate at 127)
# ---------------------------------------------------------------------------


def int8_checks(mod):
    """Pins of ``oracle.int8`` (or a planted copy): the definition's spot
    values, then torch's round-half-to-even and clamp on the same quotients."""
    import torch

    def spot():
        x = np.array([0.0, -0.0, 0.5, 1.5, 2.5, -2.5, -0.5, 0.49999997, 126.5, 127.4, 127.6, 200.0, -127.5,
                      -200.0, np.inf, -np.inf, np.nan], np.float32)
        want = [0, 0, 0, 2, 2, -2, 0, 0, 126, 127, 127, 127, -127, -127, 127, -127, 0]
        assert mod.encode(x).tolist() == want
        assert mod.encode(x).dtype == np.int8
        codes = np.arange(-127, 128).astype(np.int8)
        assert np.array_equal(mod.decode(codes), np.arange(-127, 128, dtype=np.float64))
        assert np.array_equal(mod.encode(mod.decode(codes).astype(np.float32)), codes)

    def library():
        rng = np.random.default_rng(3)
        x = np.concatenate([rng.standard_normal(4000) * s for s in (0.7, 30.0, 400.0)]).astype(np.float32)
        x = np.concatenate([x, np.arange(-130, 131, dtype=np.float32) + np.float32(0.5)])
        ref = torch.clamp(torch.round(torch.from_numpy(x)), -127, 127).to(torch.int8).numpy()
        assert np.array_equal(mod.encode(x), ref)

    return [lambda _m: spot(), lambda _m: library()]
