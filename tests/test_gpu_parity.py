"""GPU parity: libpkv through its C ABI against the fp64 oracle on the same bits.

Bars: cache writes bit-exact over the whole cache; fp32 attention max abs
error <= 1e-5; bf16 and fp8-cache attention <= 2e-2.  Full-size workloads are
checked on sampled outputs (sampled (sequence, head) pairs or query rows that
the oracle computes one by one), reduced copies of the same workloads in full.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import (TOL, GpuStep, assert_cache_equal, max_err, oracle_decode, oracle_prefill,
                         oracle_write, out_f64, sample_pairs, sample_rows, say, sequence_pairs, to_dev,
                         unit_pairs)
import paged_kv_cache_map_amd as pkv
from oracle import paged

pytestmark = pytest.mark.gpu


def run_step_and_check(step, *, full=True, pairs=None, rows=None, split_keys=0):
    say(step.name, "tokens", step.num_tokens, "blocks", step.num_blocks, "split", split_keys)
    g = GpuStep(step)
    g.write()
    torch.cuda.synchronize()
    kc, vc = oracle_write(step)
    assert_cache_equal(g.k_cache, kc, step.cache_dtype, "k_cache")
    assert_cache_equal(g.v_cache, vc, step.cache_dtype, "v_cache")
    tol = TOL[step.cache_dtype]
    errs = {}
    if len(step.ids("prefill")):
        say(step.name, "prefill")
        out = out_f64(g.prefill())
        cu = step.prefill_inputs()["cu_seqlens_q"]
        use_rows = None if full else rows
        want = oracle_prefill(step, kc, vc, rows=use_rows)
        if use_rows is not None:
            out, want = out[use_rows], want[use_rows]
        errs["prefill"] = max_err(out, want)
        assert errs["prefill"] <= tol, (step.name, errs)
        assert int(cu[-1]) == out.shape[0] or use_rows is not None
    if len(step.ids("decode")):
        say(step.name, "decode")
        out = out_f64(g.decode(split_keys))
        use_pairs = None if full else pairs
        want = oracle_decode(step, kc, vc, pairs=use_pairs)
        if use_pairs is not None:
            idx = tuple(np.array(use_pairs).T)
            out, want = out[idx], want[idx]
        errs["decode"] = max_err(out, want)
        assert errs["decode"] <= tol, (step.name, errs)
    print(step.name, errs, flush=True)
    return g


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------


def test_tiny_decode_page_example():
    step = workloads.config("tiny_decode")
    assert list(step.slot_map) == [94, 32, 198]
    run_step_and_check(step)


def test_llama8b_decode_full():
    run_step_and_check(workloads.config("llama8b_decode"))


def test_varlen_prefill_prefix_reduced():
    run_step_and_check(workloads.config("varlen_prefill_prefix", batch=5, q_hi=300, q_lo=1, p_hi=200))


def test_varlen_prefill_prefix_full_sampled():
    step = workloads.config("varlen_prefill_prefix")
    rng = np.random.default_rng(0)
    rows = sample_rows(rng, step.prefill_inputs()["cu_seqlens_q"], 96)
    run_step_and_check(step, full=False, rows=rows)


def test_llama70b_long_decode_sampled():
    """Every (sequence, KV head) unit of the 8 x 131k-key decode, one q head each."""
    step = workloads.config("llama70b_long_decode")
    pairs = unit_pairs(np.random.default_rng(1), 8, step.num_heads, step.num_kv_heads)
    assert len(pairs) == 64
    run_step_and_check(step, full=False, pairs=pairs)


def test_mixed_fp8_reduced():
    step = workloads.config("mixed_fp8", prefill_chunks=3, chunk=200, decode_batch=12, p_hi=700,
                            len_lo=1, len_hi=900)
    run_step_and_check(step)


def test_mixed_fp8_full_sampled():
    """Every decode sequence once; the first and last row of every prefill
    chunk and 256 more drawn at random."""
    step = workloads.config("mixed_fp8")
    rng = np.random.default_rng(2)
    rows = sample_rows(rng, step.prefill_inputs()["cu_seqlens_q"], 256)
    pairs = sequence_pairs(rng, 256, 32)
    assert len(rows) >= 256 + 4 and {b for b, _ in pairs} == set(range(256))
    run_step_and_check(step, full=False, rows=rows, pairs=pairs)


# ---------------------------------------------------------------------------
# decode: split plan, determinism, shapes, edge cases
# ---------------------------------------------------------------------------


def test_decode_split_invariance_and_determinism():
    step = workloads.config("llama8b_decode", batch=6, len_lo=1, len_hi=1500)
    g = GpuStep(step)
    g.write()
    kc, vc = oracle_write(step)
    want = oracle_decode(step, kc, vc)
    outs = {}
    for sk in (0, 128, 256, 640, 4096):
        say("split", sk)
        outs[sk] = out_f64(g.decode(sk))
        assert max_err(outs[sk], want) <= TOL["bf16"], sk
    again = out_f64(g.decode(128))
    assert np.array_equal(again, outs[128]), "run-to-run results differ"


def test_decode_workspace_reuse():
    """One workspace, never cleared, serves calls of different shapes and plans
    in a row (stale partials of earlier calls must not leak into results)."""
    ws = torch.full((64 << 20,), 0xff, dtype=torch.uint8, device="cuda")   # every float NaN
    cases = [
        workloads.config("llama8b_decode", batch=7, len_lo=1, len_hi=2000),
        workloads.config("llama8b_decode", batch=3, len_lo=500, len_hi=3000, num_heads=16,
                         num_kv_heads=2),
        workloads.config("llama8b_decode", batch=9, len_lo=0, len_hi=300, num_heads=8,
                         num_kv_heads=8, head_dim=64, block_size=32),
    ]
    for rep in range(2):
        for i, step in enumerate(cases):
            say("workspace reuse", rep, i)
            g = GpuStep(step)
            g.write()
            kc, vc = oracle_write(step)
            want = oracle_decode(step, kc, vc)
            for sk in (0, 256, 0):
                out = out_f64(g.decode(sk, workspace=ws))
                assert max_err(out, want) <= TOL["bf16"], (rep, i, sk)


def test_stream_decode_is_deterministic():
    step = workloads.config("llama8b_decode", batch=16, len_lo=1, len_hi=3000, num_heads=64,
                            num_kv_heads=8)
    g = GpuStep(step)
    g.write()
    a = g.decode().cpu()
    b = g.decode().cpu()
    assert torch.equal(a, b)


@pytest.mark.parametrize("hq,hkv,d,bs,dtype", [
    (8, 8, 128, 16, "bf16"),     # MHA, G = 1
    (8, 1, 128, 16, "bf16"),     # MQA, G = 8
    (16, 1, 128, 32, "bf16"),    # G = 16 (two head groups)
    (4, 2, 64, 8, "bf16"),       # G = 2, D = 64, bs = 8
    (16, 4, 64, 64, "bf16"),
    (8, 2, 128, 256, "bf16"),
    (8, 2, 64, 16, "f32"),
    (4, 1, 128, 16, "f32"),
    (32, 8, 128, 16, "fp8"),
    (8, 8, 64, 32, "fp8"),
])
def test_decode_shapes(hq, hkv, d, bs, dtype):
    step = workloads.config("llama8b_decode", batch=5, len_lo=1, len_hi=700, num_heads=hq,
                            num_kv_heads=hkv, head_dim=d, block_size=bs,
                            cache_dtype=dtype) if dtype != "f32" else \
        workloads.build_step("f32_decode", 77, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                             block_size=bs, q_dtype="f32", cache_dtype="f32",
                             prefix=[0, 5, 130, 333, 700], new=[1] * 5, kinds=["decode"] * 5)
    run_step_and_check(step, split_keys=128)
    run_step_and_check(step)


@pytest.mark.parametrize("prefix,hq,hkv,cache", [
    ([40000], 4, 1, "bf16"),           # one unit shared by every wave of the grid
    ([3000, 4, 4, 4], 32, 8, "bf16"),  # fewer chunks than waves: one-chunk parts, waves without chunks
    ([3000, 0, 17, 0], 32, 8, "fp8"),  # the same with one-key sequences (then empty ones) between
])
def test_decode_units_split_over_many_waves(prefix, hq, hkv, cache):
    """Units whose partial results come from many waves of the persistent
    grid (up to every wave), and waves that own no chunk at all."""
    step = workloads.build_step("split_extremes", 91, num_heads=hq, num_kv_heads=hkv, head_dim=128,
                                block_size=16, q_dtype="bf16", cache_dtype=cache, prefix=prefix,
                                new=[1] * len(prefix), kinds=["decode"] * len(prefix))
    g = run_step_and_check(step)
    a = g.decode().cpu()
    b = g.decode().cpu()
    assert torch.equal(a, b), "run-to-run results differ"
    if min(prefix) == 0:
        # the one-key sequences become empty: their rows are zeros, the rest unchanged
        d = step.decode_inputs()
        lens = d["cache_seqlens"].copy()
        lens[np.array(prefix) == 0] = 0
        say("split extremes, empty sequences")
        g.dec_len = to_dev(lens, "i32")
        out = out_f64(g.decode())
        kc, vc = oracle_write(step)
        want = paged.paged_decode(d["q"], step.q_dtype, kc, vc, step.cache_dtype, d["block_table"], lens,
                                  step.scale, step.k_scale, step.v_scale)
        assert np.all(out[lens == 0] == 0)
        assert max_err(out, want) <= TOL[cache]


def test_decode_few_units_many_parts():
    """The per-GPU share of the 70B decode at eight-way tensor parallelism
    (one KV head, G = 8), shortened: 8 units over the whole grid, about 128
    parts each, merged by a workgroup per row (four waves, a quarter of the
    parts each); every row checked, twice for run-to-run bits."""
    step = workloads.build_step("tp8_share", 92, num_heads=8, num_kv_heads=1, head_dim=128, block_size=16,
                                q_dtype="bf16", cache_dtype="bf16", prefix=[20000, 19999, 20001, 4096, 12345, 1, 30000,
                                                                            20000],
                                new=[1] * 8, kinds=["decode"] * 8)
    g = run_step_and_check(step)
    assert torch.equal(g.decode().cpu(), g.decode().cpu()), "run-to-run results differ"


def test_decode_zero_length_sequence_gives_zeros():
    step = workloads.config("tiny_decode")
    g = GpuStep(step)
    g.write()
    g.dec_len = to_dev(np.array([0, 33, 0], np.int32), "i32")
    out = out_f64(g.decode())
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    kc, vc = oracle_write(step)
    d = step.decode_inputs()
    want = paged.paged_decode(d["q"], "f32", kc, vc, "f32", d["block_table"],
                              np.array([0, 33, 0], np.int32), step.scale)
    assert max_err(out, want) <= TOL["f32"]


def test_block_permutation_gives_identical_bits():
    """Same logical data in two different physical block arrangements."""
    step = workloads.config("llama8b_decode", batch=4, len_lo=30, len_hi=400)
    g1 = GpuStep(step)
    g1.write()
    a = g1.decode().cpu()
    # relabel every physical block b -> perm[b]
    perm = np.random.default_rng(9).permutation(step.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    step2 = workloads.config("llama8b_decode", batch=4, len_lo=30, len_hi=400)
    step2.k_cache = step.k_cache[inv]
    step2.v_cache = step.v_cache[inv]
    step2.block_table = np.where(step.block_table >= 0, perm[np.maximum(step.block_table, 0)], -1)
    step2.block_table = step2.block_table.astype(np.int32)
    bs = step.block_size
    step2.slot_map = (perm[step.slot_map // bs] * bs + step.slot_map % bs).astype(np.int32)
    g2 = GpuStep(step2)
    g2.write()
    b = g2.decode().cpu()
    assert torch.equal(a, b)


@pytest.mark.parametrize("cache_dtype,split", [("bf16", 0), ("bf16", 128), ("fp8", 0)])
def test_decode_bad_block_ids_read_as_empty_blocks(cache_dtype, split):
    """A block id past the pool or negative inside a sequence's range: the
    kernels stay in their buffers and leave that block's keys out (the method
    defines no result for it; the library documents this behaviour).  Expected
    values: the oracle's attention over the remaining keys."""
    step = workloads.config("llama8b_decode", batch=3, len_lo=100, len_hi=300, cache_dtype=cache_dtype)
    say("bad block ids", cache_dtype, split)
    g = GpuStep(step)
    g.write()
    kc, vc = oracle_write(step)
    d = step.decode_inputs()
    bt = d["block_table"].copy()
    bs, hkv, hd = step.block_size, step.num_kv_heads, step.head_dim
    bt[1, 1] = step.num_blocks + 7
    bt[2, 0] = -1
    g.dec_bt = to_dev(bt, "i32")
    out = out_f64(g.decode(split))
    q64 = paged.to_f64(d["q"], step.q_dtype)
    want = np.zeros_like(out)
    for b in range(3):
        lk = int(d["cache_seqlens"][b])
        keys = [j for j in range(lk) if 0 <= bt[b, j // bs] < step.num_blocks]
        slots = np.array([bt[b, j // bs] * bs + j % bs for j in keys], dtype=np.int64)
        k_rows = kc.reshape(-1, hkv, hd)[slots]
        v_rows = vc.reshape(-1, hkv, hd)[slots]
        k64 = np.stack([paged._rows_to_f64(k_rows[:, gi:gi + 1], cache_dtype, step.k_scale, gi)[:, 0]
                        for gi in range(hkv)], axis=1)
        v64 = np.stack([paged._rows_to_f64(v_rows[:, gi:gi + 1], cache_dtype, step.v_scale, gi)[:, 0]
                        for gi in range(hkv)], axis=1)
        want[b] = paged.attention(q64[b][None], k64, v64, step.scale, True)[0]
    assert max_err(out, want) <= TOL[cache_dtype]


def test_decode_batch_past_the_stream_table():
    """More sequences than one stream launch's LDS chunk table holds (2048):
    the automatic plan runs the matrix-core stream kernels over two slices of
    1050 sequences, one after the other."""
    step = workloads.config("llama8b_decode", batch=2100, len_lo=1, len_hi=40)
    rng = np.random.default_rng(31)
    run_step_and_check(step, full=False, pairs=sample_pairs(rng, 2100, step.num_heads, 300))


@pytest.mark.parametrize("cdt", ["f32", "fp8", "int8"])
def test_decode_batch_in_uneven_slices(cdt):
    """4100 sequences: three stream slices of 1367, 1367 and 1366 (the vector
    stream kernel for fp32, the matrix-core one for the one-byte caches);
    sampled rows from every slice, the slice edges among them."""
    rng = np.random.default_rng(37)
    n = 4100
    prefix = rng.integers(0, 70, size=n)
    step = workloads.build_step(f"decode_slices_{cdt}", 4100, num_heads=8, num_kv_heads=2, head_dim=128,
                                block_size=16, q_dtype="f32" if cdt == "f32" else "bf16", cache_dtype=cdt,
                                prefix=prefix, new=[1] * n, kinds=["decode"] * n)
    pairs = sample_pairs(rng, n, 8, 200) + [(b, h) for b in (0, 1366, 1367, 2733, 2734, 4099) for h in (0, 7)]
    run_step_and_check(step, full=False, pairs=pairs)


def test_decode_batch_past_the_stream_table_fixed_splits():
    """The same batch of 2100 on an explicit fixed-split plan (vector
    kernels, one grid over the whole batch)."""
    step = workloads.config("llama8b_decode", batch=2100, len_lo=1, len_hi=300)
    rng = np.random.default_rng(33)
    run_step_and_check(step, full=False, pairs=sample_pairs(rng, 2100, step.num_heads, 300), split_keys=128)


# ---------------------------------------------------------------------------
# prefill: the page-2 example, shapes, non-causal
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_page2_varlen_example_contiguous(dtype, causal):
    c = workloads.page2_varlen_example(dtype=dtype)
    say("page2 varlen", dtype, causal)
    out = pkv.varlen_prefill(to_dev(c.q, dtype), to_dev(c.k, dtype), to_dev(c.v, dtype),
                             to_dev(c.cu_seqlens_q, "i32"), to_dev(c.cu_seqlens_k, "i32"),
                             c.max_seqlen_q, c.max_seqlen_k, c.scale, causal)
    got = out_f64(out)
    want = paged.varlen_prefill(c.q, dtype, c.k, c.v, dtype, c.cu_seqlens_q, c.cu_seqlens_k, c.scale,
                                causal)
    assert max_err(got, want) <= TOL[dtype]
    # request 0 has no key: its ten rows are exactly zero
    assert np.all(got[0:10] == 0)
    if causal:
        assert np.all(got[10:12] == 0)


@pytest.mark.parametrize("hq,hkv,d,bs,dtype", [
    (8, 8, 128, 16, "bf16"),
    (16, 1, 128, 32, "bf16"),
    (4, 2, 64, 8, "bf16"),
    # bf16 at head_dim 64: two 32-column blocks a wave (64 columns: 64 / G rows)
    (8, 8, 64, 16, "bf16"),      # G = 1: the second block holds rows 32-63
    (32, 8, 64, 32, "bf16"),     # G = 4
    (16, 1, 64, 16, "bf16"),     # G = 16: 4 rows a wave, the second block rows 2-3
    (8, 2, 64, 64, "fp8"),
    (32, 8, 128, 16, "fp8"),
    (8, 8, 128, 8, "fp8"),       # fp8 P.V at G = 1, block size 8
    (64, 8, 128, 256, "fp8"),    # G = 8, block size 256
    (16, 1, 128, 32, "fp8"),     # G = 16
    (4, 2, 64, 16, "f32"),
])
def test_prefill_shapes(hq, hkv, d, bs, dtype):
    rng = np.random.default_rng(hq * 1000 + d + bs)
    lq = rng.integers(1, 300, size=4)
    pre = rng.integers(0, 260, size=4)
    step = workloads.build_step("prefill_shape", 5000 + hq + d + bs, num_heads=hq, num_kv_heads=hkv,
                                head_dim=d, block_size=bs,
                                q_dtype="f32" if dtype == "f32" else "bf16", cache_dtype=dtype,
                                prefix=pre, new=lq, kinds=["prefill"] * 4)
    run_step_and_check(step)


def test_prefill_head_dim_64_many_items_per_request():
    """bf16 at head_dim 64 (two column blocks a wave, 64 rows an item at G =
    4): requests of up to 700 rows over up to 1000 cached keys span up to 11
    work items each, with ragged last items and a one-row request."""
    step = workloads.build_step("prefill_d64_items", 6401, num_heads=32, num_kv_heads=8, head_dim=64,
                                block_size=16, q_dtype="bf16", cache_dtype="bf16",
                                prefix=[0, 300, 64, 1000], new=[700, 1, 257, 513],
                                kinds=["prefill"] * 4)
    run_step_and_check(step)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8", "int8"])
def test_prefill_bad_block_ids_read_as_empty_blocks(cache_dtype):
    """Block ids past the pool or negative inside a request's keys: the
    prefill stays in its buffers and leaves those blocks' keys out, as the
    decode does.  Expected values: per row, the oracle's attention over the
    keys it sees that lie in valid blocks."""
    prefix, new = [200, 90, 300], [120, 64, 33]
    step = workloads.build_step(f"prefill_bad_blocks_{cache_dtype}", 4321, num_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=16, q_dtype="bf16", cache_dtype=cache_dtype,
                                prefix=prefix, new=new, kinds=["prefill"] * 3)
    say("prefill bad block ids", cache_dtype)
    g = GpuStep(step)
    g.write()
    kc, vc = oracle_write(step)
    p = step.prefill_inputs()
    bt = p["block_table"].copy()
    bs, hkv, hd, hq = step.block_size, step.num_kv_heads, step.head_dim, step.num_heads
    bt[0, 3] = step.num_blocks + 5     # keys 48..63 of request 0
    bt[1, 0] = -1                      # keys 0..15 of request 1
    bt[2, 18] = step.num_blocks        # keys 288..303 of request 2 (the last cached ones and 4 new ones)
    g.pre_bt = to_dev(bt, "i32")
    out = out_f64(g.prefill())
    cu_q, cu_k = p["cu_seqlens_q"], p["cu_seqlens_k"]
    q64 = paged.to_f64(p["q"], step.q_dtype)
    want = np.zeros_like(out)
    for b in range(3):
        lq, lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        valid = [j for j in range(lk) if 0 <= bt[b, j // bs] < step.num_blocks]
        slots = np.array([bt[b, j // bs] * bs + j % bs for j in valid], dtype=np.int64)
        k64 = np.stack([paged._rows_to_f64(kc.reshape(-1, hkv, hd)[slots][:, gi:gi + 1], cache_dtype,
                                           step.k_scale, gi)[:, 0] for gi in range(hkv)], axis=1)
        v64 = np.stack([paged._rows_to_f64(vc.reshape(-1, hkv, hd)[slots][:, gi:gi + 1], cache_dtype,
                                           step.v_scale, gi)[:, 0] for gi in range(hkv)], axis=1)
        keys = np.array(valid)
        for i in range(lq):
            seen = keys <= i + lk - lq
            r = int(cu_q[b]) + i
            want[r] = paged.attention(q64[r][None], k64[seen], v64[seen], step.scale, False)[0]
    assert max_err(out, want) <= TOL[cache_dtype]


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_noncausal_contiguous_matches_oracle(d):
    c = workloads.random_varlen_contig("nc", 321, [70, 1, 200, 0, 33], [5, 260, 1, 9, 120],
                                       num_heads=8, num_kv_heads=2, head_dim=d, dtype="bf16")
    for causal in (False, True):
        out = pkv.varlen_prefill(to_dev(c.q, "bf16"), to_dev(c.k, "bf16"), to_dev(c.v, "bf16"),
                                 to_dev(c.cu_seqlens_q, "i32"), to_dev(c.cu_seqlens_k, "i32"),
                                 c.max_seqlen_q, c.max_seqlen_k, c.scale, causal)
        want = paged.varlen_prefill(c.q, "bf16", c.k, c.v, "bf16", c.cu_seqlens_q, c.cu_seqlens_k,
                                    c.scale, causal)
        assert max_err(out_f64(out), want) <= TOL["bf16"], causal


def test_negative_and_zero_scale():
    """The softmax scale is any real: negative and zero scales match the oracle
    for prefill (packed and paged) and decode."""
    c = workloads.random_varlen_contig("neg", 77, [40, 130, 1], [40, 200, 65], num_heads=8,
                                       num_kv_heads=2, head_dim=128, dtype="bf16")
    for sc in (-0.2, 0.0):
        say("scale", sc)
        out = pkv.varlen_prefill(to_dev(c.q, "bf16"), to_dev(c.k, "bf16"), to_dev(c.v, "bf16"),
                                 to_dev(c.cu_seqlens_q, "i32"), to_dev(c.cu_seqlens_k, "i32"),
                                 c.max_seqlen_q, c.max_seqlen_k, sc, True)
        want = paged.varlen_prefill(c.q, "bf16", c.k, c.v, "bf16", c.cu_seqlens_q, c.cu_seqlens_k,
                                    sc, True)
        assert max_err(out_f64(out), want) <= TOL["bf16"], sc
    step = workloads.build_step("neg_scale", 78, num_heads=8, num_kv_heads=2, head_dim=128,
                                block_size=16, q_dtype="bf16", cache_dtype="bf16",
                                prefix=[100, 0, 300], new=[70, 1, 1],
                                kinds=["prefill", "decode", "decode"])
    step.scale = -0.15
    run_step_and_check(step)


# ---------------------------------------------------------------------------
# fp8 codec through the library
# ---------------------------------------------------------------------------


def test_fp8_write_every_bf16_pattern():
    """All 65536 bf16 bit patterns (NaN and inf included) through the write,
    per-head scales 1 and 1/3: codes equal the oracle's bit for bit."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    hkv, d = 2, 128
    t = 65536 // (hkv * d)
    k = bits.reshape(t, hkv, d)
    v = bits[::-1].copy().reshape(t, hkv, d)
    scale = np.array([1.0, 1.0 / 3.0], np.float32)
    nb, bs = t // 16, 16
    kc = np.zeros((nb, bs, hkv, d), np.uint8)
    slots = np.random.default_rng(4).permutation(t).astype(np.int32)
    want_k, want_v = paged.kv_cache_write(k, v, kc, kc, slots, "bf16", "fp8", scale, scale)
    gk, gv = to_dev(kc, "fp8"), to_dev(kc, "fp8")
    pkv.kv_cache_write(to_dev(k, "bf16"), to_dev(v, "bf16"), gk, gv, to_dev(slots, "i32"),
                       to_dev(scale, "f32"), to_dev(scale, "f32"))
    assert_cache_equal(gk, want_k, "fp8", "k")
    assert_cache_equal(gv, want_v, "fp8", "v")


def test_fp8_decode_every_code():
    """A one-key sequence returns its V row exactly: every finite E4M3 code
    decodes to its value (scale 1; values are exact in bf16)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    hkv, d, bs = 1, 128, 16
    n = len(codes)
    seqs = (n + d - 1) // d
    padded = np.resize(codes, seqs * d)
    v = np.full((seqs, bs, hkv, d), 0x7F, np.uint8)
    k = np.full((seqs, bs, hkv, d), 0x7F, np.uint8)
    v[:, 0, 0, :] = padded.reshape(seqs, d)
    k[:, 0, 0, :] = 0x38
    table = np.arange(seqs, dtype=np.int32)[:, None]
    ones = np.ones(1, np.float32)
    q = np.full((seqs, 4, d), 0x3F80, np.uint16)
    out = pkv.paged_decode(to_dev(q, "bf16"), to_dev(k, "fp8"), to_dev(v, "fp8"), to_dev(table, "i32"),
                           to_dev(np.ones(seqs, np.int32), "i32"), 0.1, to_dev(ones, "f32"),
                           to_dev(ones, "f32"))
    got = out_f64(out)
    from oracle import e4m3
    want = e4m3.decode(padded).reshape(seqs, d)
    for h in range(4):
        assert np.array_equal(got[:, h, :], want)
