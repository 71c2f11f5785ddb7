"""GPU parity of the appending decode (pkv_paged_decode_append) against the
fp64 oracle: the call stores each decode sequence's new K/V rows at position
cache_seqlens[b] and attends cache_seqlens[b] + 1 keys.

Bars as for the other calls: both caches bit-exact over the whole pool, fp32
attention <= 1e-5, bf16 and fp8-cache attention <= 2e-2.  On the matrix-core
plan the appending call must also return exactly the bits of the write
followed by the plain decode (same kernels, same schedule).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_map_amd as pkv
import workloads
from oracle import paged
from workloads import configs
from gpu_helpers import (TOL, GpuStep, assert_cache_equal, max_err, oracle_append_decode, oracle_prefill,
                         oracle_write, out_f64, sample_pairs, say, to_dev)

pytestmark = pytest.mark.gpu


def check_append(step, *, split_keys=0, pairs=None, same_as_separate=True):
    say(step.name, "append", "seqs", len(step.ids("decode")), "blocks", step.num_blocks, "split", split_keys)
    g = GpuStep(step)
    if len(step.ids("prefill")):
        g.write_prefill_only()
    got = out_f64(g.append_decode(split_keys))
    torch.cuda.synchronize()
    want, kc, vc = oracle_append_decode(step, pairs=pairs)
    assert_cache_equal(g.k_cache, kc, step.cache_dtype, "k_cache")
    assert_cache_equal(g.v_cache, vc, step.cache_dtype, "v_cache")
    # the oracle's two paths agree: its write of the whole slot map gives the same caches
    kc_all, vc_all = oracle_write(step)
    assert np.array_equal(kc_all.view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(vc_all.view(np.uint8), vc.view(np.uint8))
    if pairs is not None:
        idx = tuple(np.array(pairs).T)
        got_s, want_s = got[idx], want[idx]
    else:
        got_s, want_s = got, want
    err = max_err(got_s, want_s)
    print(step.name, "append max|err|", err, flush=True)
    assert err <= TOL[step.cache_dtype], (step.name, err)
    if same_as_separate:
        say(step.name, "write + decode for comparison")
        g2 = GpuStep(step)
        g2.write()
        sep = out_f64(g2.decode(split_keys))
        assert np.array_equal(sep, got), "append call differs from write + decode"
    return g, kc, vc, got


def test_append_page_example_f32():
    """The decode worked example (lengths 30, 32, 70 before the step; new rows
    at slots 94, 32, 198), fp32 cache: append kernel + vector stream plan."""
    step = workloads.config("tiny_decode")
    assert list(step.decode_append_inputs()["cache_seqlens"]) == [30, 32, 70]
    check_append(step)


def test_append_llama8b_full():
    check_append(workloads.config("llama8b_decode"))


def test_append_llama70b_long_sampled():
    step = workloads.config("llama70b_long_decode")
    pairs = sample_pairs(np.random.default_rng(21), 8, 64, 12)
    check_append(step, pairs=pairs, same_as_separate=False)


def test_append_mixed_fp8_reduced():
    """Mixed step: prefill tokens by the slot-map write, decode tokens by the
    appending decode; then the prefill over the same caches."""
    step = workloads.config("mixed_fp8", prefill_chunks=3, chunk=200, decode_batch=12, p_hi=700,
                            len_lo=0, len_hi=900)
    g, kc, vc, _ = check_append(step)
    say(step.name, "prefill after append")
    out = out_f64(g.prefill())
    want = oracle_prefill(step, kc, vc)
    assert max_err(out, want) <= TOL["fp8"]


def test_append_mixed_fp8_full_sampled():
    step = workloads.config("mixed_fp8")
    pairs = sample_pairs(np.random.default_rng(22), 256, 32, 40)
    check_append(step, pairs=pairs, same_as_separate=False)


# (head_dim, q heads, KV heads, cache dtype, block size, split_keys)
SHAPES = [
    (64, 8, 2, "fp8", 16, 0),      # 64-byte fp8 head rows: two heads share a 128-byte line
    (64, 4, 2, "bf16", 8, 0),
    (128, 4, 4, "bf16", 32, 0),    # G = 1
    (128, 16, 2, "bf16", 16, 0),   # G = 8
    (128, 32, 2, "fp8", 16, 0),    # G = 16
    (128, 16, 4, "bf16", 256, 0),
    (128, 16, 4, "bf16", 16, 256),  # fixed splits: append kernel, then the split kernels
    (128, 16, 4, "fp8", 16, 128),
    (128, 8, 2, "f32", 16, 0),     # fp32 cache: append kernel + vector stream plan
    (64, 8, 8, "f32", 8, 128),
]


@pytest.mark.parametrize("d,hq,hkv,cdt,bs,split", SHAPES,
                         ids=[f"d{s[0]}_g{s[1] // s[2]}_{s[3]}_bs{s[4]}_split{s[5]}" for s in SHAPES])
def test_append_shapes_and_plans(d, hq, hkv, cdt, bs, split):
    """Lengths before the step at and around block boundaries, including 0
    (the new token is then the only key: out = its V row)."""
    prefix = [0, 1, bs - 1, bs, bs + 1, 2 * bs - 1, 3 * bs, 97, 0, 515, 1000, 31, 32, 33, 63, 64]
    qdt = "f32" if cdt == "f32" else "bf16"
    step = workloads.build_step(f"append_d{d}_{cdt}_bs{bs}", 40 + d + hq + bs, num_heads=hq,
                                num_kv_heads=hkv, head_dim=d, block_size=bs, q_dtype=qdt, cache_dtype=cdt,
                                prefix=prefix, new=[1] * len(prefix), kinds=["decode"] * len(prefix))
    _, _, _, got = check_append(step, split_keys=split)
    if cdt != "fp8":
        # empty history: every q head returns the new V row of its KV head (a
        # softmax weight of one; bf16 outputs round back to the row exactly)
        vn = step.decode_append_inputs()["v_new"]
        vn64 = (vn.astype(np.float64) if qdt == "f32" else
                (vn.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        for b in (0, 8):
            for h in range(hq):
                want = vn64[b, h // (hq // hkv)]
                if qdt == "bf16":
                    assert np.array_equal(got[b, h], want), (b, h)
                else:
                    np.testing.assert_allclose(got[b, h], want, rtol=1e-6, atol=1e-30)


def test_append_repeated_steps_grow_the_cache():
    """Three appending steps in a row on one pool (lengths +1 each step): the
    caches and every step's output match the oracle run step by step."""
    step = workloads.config("llama8b_decode", batch=5, len_lo=0, len_hi=60)
    d = step.decode_append_inputs()
    # room for three more tokens per sequence: extend each row with fresh blocks
    bs = step.block_size
    lens = d["cache_seqlens"].astype(np.int64)
    need = (lens + 3 + bs - 1) // bs
    extra = int(np.maximum(need - (lens + 1 + bs - 1) // bs, 0).sum())
    nb = step.num_blocks + extra
    table = np.full((len(lens), int(need.max())), -1, np.int32)
    table[:, :d["block_table"].shape[1]] = d["block_table"]
    nxt = step.num_blocks
    for b in range(len(lens)):
        for j in range(int(need[b])):
            if table[b, j] < 0:
                table[b, j] = nxt
                nxt += 1
    assert nxt == nb
    pad = np.zeros((extra,) + step.k_cache.shape[1:], step.k_cache.dtype)
    kc = np.concatenate([step.k_cache, pad])
    vc = np.concatenate([step.v_cache, pad])
    gk, gv = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    gt = to_dev(table, "i32")
    for it in range(3):
        say("repeated append step", it)
        q = workloads.configs._normal(900 + it, 3, d["q"].shape, "bf16")
        kn = workloads.configs._normal(900 + it, 6, d["k_new"].shape, "bf16")
        vn = workloads.configs._normal(900 + it, 7, d["v_new"].shape, "bf16")
        cur = (lens + it).astype(np.int32)
        got = out_f64(pkv.paged_decode_append(to_dev(q, "bf16"), to_dev(kn, "bf16"), to_dev(vn, "bf16"),
                                              gk, gv, gt, to_dev(cur, "i32"), step.scale))
        want, kc, vc = paged.paged_decode_append(q, "bf16", kn, vn, kc, vc, "bf16", table, cur, step.scale)
        assert_cache_equal(gk, kc, "bf16", f"k_cache step {it}")
        assert_cache_equal(gv, vc, "bf16", f"v_cache step {it}")
        assert max_err(got, want) <= TOL["bf16"], it


def test_append_batch_past_the_stream_table():
    """2100 sequences (more than one stream launch's chunk table holds): the
    appending matrix-core stream kernel over two slices of 1050 sequences."""
    rng = np.random.default_rng(23)
    prefix = rng.integers(0, 40, size=2100)
    step = workloads.build_step("append_big_batch", 2100, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                                q_dtype="bf16", cache_dtype="bf16", prefix=prefix, new=[1] * 2100,
                                kinds=["decode"] * 2100)
    pairs = sample_pairs(np.random.default_rng(24), 2100, 8, 64)
    check_append(step, pairs=pairs)


@pytest.mark.parametrize("cdt", ["f32", "bf16", "fp8", "int8"])
@pytest.mark.parametrize("split", [0, 128])
def test_append_bad_metadata_stores_nothing(cdt, split):
    """The appending call's handling of metadata that leaves a new token no
    slot (include/pkv.h: an entry that is negative or >= num_blocks is an
    empty block; lengths are clamped to the table): the row is not stored and
    the key is left out of the softmax, so the output is the plain decode
    over the keys that remain.  Sequence 0's new token opens a block whose
    entry is -1; sequence 1 (empty) has an out-of-range entry and returns
    zeros; sequence 2 appends normally; sequence 3's table is full."""
    rng = np.random.default_rng(21 + split)
    hq, hkv, d, bs, width, nb = 8, 2, 64, 16, 3, 24
    qdt = "f32" if cdt == "f32" else "bf16"
    lens = np.array([16, 0, 31, 48], np.int32)
    table = rng.permutation(nb)[: 4 * width].reshape(4, width).astype(np.int32)
    table[0, 1] = -1
    table[1, 0] = nb + 5
    seed = 400 + split
    if cdt in ("fp8", "int8"):  # codes of the one-byte cache, per-head scales
        codes = configs._fp8_codes if cdt == "fp8" else configs._int8_codes
        kc, vc = codes(seed, 1, (nb, bs, hkv, d)), codes(seed, 2, (nb, bs, hkv, d))
        top = 448.0 if cdt == "fp8" else 127.0
        scales = (np.full(hkv, 3.0 / top, np.float32), np.full(hkv, 5.0 / top, np.float32))
    else:
        kc = configs._normal(seed, 1, (nb, bs, hkv, d), cdt)
        vc = configs._normal(seed, 2, (nb, bs, hkv, d), cdt)
        scales = (None, None)
    ks, vs = [None if x is None else to_dev(x, "f32") for x in scales]
    q = configs._normal(seed, 3, (4, hq, d), qdt)
    kn = configs._normal(seed, 4, (4, hkv, d), qdt)
    vn = configs._normal(seed, 5, (4, hkv, d), qdt)
    scale = 0.125
    say("append bad metadata", cdt, "split", split)
    gk, gv = to_dev(kc, cdt), to_dev(vc, cdt)
    got = out_f64(pkv.paged_decode_append(to_dev(q, qdt), to_dev(kn, qdt), to_dev(vn, qdt), gk, gv,
                                          to_dev(table, "i32"), to_dev(lens, "i32"), scale, ks, vs, split_keys=split))
    torch.cuda.synchronize()
    # only sequence 2's rows are stored
    want2, wk, wv = paged.paged_decode_append(q[2:3], qdt, kn[2:3], vn[2:3], kc, vc, cdt, table[2:3], lens[2:3],
                                              scale, *scales)
    assert_cache_equal(gk, wk, cdt, "k_cache")
    assert_cache_equal(gv, wv, cdt, "v_cache")
    want = np.zeros((4, hq, d))
    want[0] = paged.paged_decode(q[0:1], qdt, kc, vc, cdt, table[0:1], np.array([16]), scale, *scales)[0]
    want[2] = want2[0]
    want[3] = paged.paged_decode(q[3:4], qdt, kc, vc, cdt, table[3:4], np.array([48]), scale, *scales)[0]
    assert np.array_equal(got[1], np.zeros((hq, d)))
    err = max_err(got, want)
    print("append bad metadata", cdt, split, "max|err|", err, flush=True)
    assert err <= TOL[cdt]

