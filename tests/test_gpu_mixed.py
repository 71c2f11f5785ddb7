"""GPU parity of the mixed-step call (pkv_mixed_attention): a chunked-prefill
step's prefill chunks and decode sequences in one call, against the fp64
oracle; for one-byte caches at head_dim 128 the two run in one kernel launch.
The prefill rows must also equal the plain prefill call's bits (the same
workgroup code on the same work items)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_map_amd as pkv
import workloads
from gpu_helpers import (TOL, GpuStep, max_err, oracle_decode, oracle_prefill, oracle_write, out_f64, sample_pairs,
                         sample_rows, say, sequence_pairs, to_dev)

pytestmark = pytest.mark.gpu


def run_mixed(step, *, rows=None, pairs=None, parts=("prefill", "decode")):
    say(step.name, "mixed attention", parts)
    g = GpuStep(step)
    g.write()
    p = step.prefill_inputs()
    prefill = decode = None
    if "prefill" in parts and len(p["seq_ids"]):
        prefill = dict(q=g.pre_q, cu_seqlens_q=g.pre_cu_q, cu_seqlens_k=g.pre_cu_k, max_seqlen_q=p["max_seqlen_q"],
                       max_seqlen_k=p["max_seqlen_k"], block_table=g.pre_bt)
    if "decode" in parts and len(step.ids("decode")):
        decode = dict(q=g.dec_q, block_table=g.dec_bt, cache_seqlens=g.dec_len)
    p_out, d_out = pkv.mixed_attention(g.k_cache, g.v_cache, step.scale, prefill, decode, g.k_scale, g.v_scale)
    torch.cuda.synchronize()
    kc, vc = oracle_write(step)
    tol = TOL[step.cache_dtype]
    if prefill is not None:
        got = out_f64(p_out)
        want = oracle_prefill(step, kc, vc, rows=rows)
        if rows is not None:
            got_s, want_s = got[rows], want[rows]
        else:
            got_s, want_s = got, want
        err = max_err(got_s, want_s)
        print(step.name, "mixed prefill max|err|", err, flush=True)
        assert err <= tol
        say(step.name, "plain prefill for comparison")
        assert torch.equal(g.prefill().cpu(), p_out.cpu()), "prefill rows differ from the plain prefill call"
    else:
        assert p_out is None
    if decode is not None:
        got = out_f64(d_out)
        want = oracle_decode(step, kc, vc, pairs=pairs)
        if pairs is not None:
            idx = tuple(np.array(pairs).T)
            got, want = got[idx], want[idx]
        err = max_err(got, want)
        print(step.name, "mixed decode max|err|", err, flush=True)
        assert err <= tol
    else:
        assert d_out is None


@pytest.mark.parametrize("name", ["mixed_fp8", "mixed_int8"])
def test_mixed_step_reduced(name):
    step = workloads.config(name, prefill_chunks=3, chunk=200, decode_batch=12, p_hi=700, len_lo=1, len_hi=900)
    run_mixed(step)


@pytest.mark.parametrize("name", ["mixed_fp8", "mixed_int8"])
def test_mixed_step_full_sampled(name):
    """Every decode sequence once; the first and last row of every prefill
    chunk and 256 more drawn at random."""
    step = workloads.config(name)
    rng = np.random.default_rng(31)
    rows = sample_rows(rng, step.prefill_inputs()["cu_seqlens_q"], 256)
    pairs = sequence_pairs(rng, 256, 32)
    run_mixed(step, rows=rows, pairs=pairs)


@pytest.mark.parametrize("hq,hkv,cdt", [(8, 8, "fp8"), (16, 2, "int8"), (32, 2, "fp8"), (8, 4, "bf16")])
def test_mixed_step_groups_and_fallback(hq, hkv, cdt):
    """G = 1, 8, 16 on the one-launch kernel; a bf16 cache takes the two-launch path."""
    prefix = [300, 0, 77, 5, 1000, 16, 0, 2500]
    new = [150, 260, 1, 1, 1, 1, 1, 1]
    kinds = ["prefill", "prefill"] + ["decode"] * 6
    step = workloads.build_step(f"mixed_{cdt}_g{hq // hkv}", 77 + hq, num_heads=hq, num_kv_heads=hkv, head_dim=128,
                                block_size=16, q_dtype="bf16", cache_dtype=cdt, prefix=prefix, new=new, kinds=kinds)
    run_mixed(step)


@pytest.mark.parametrize("parts", [("prefill",), ("decode",)])
def test_mixed_step_one_part(parts):
    step = workloads.config("mixed_fp8", prefill_chunks=2, chunk=90, decode_batch=5, p_hi=300, len_lo=1, len_hi=400)
    run_mixed(step, parts=parts)


def test_mixed_step_more_decode_waves_than_chunks():
    """A decode part smaller than one 4-wave share per CU: most decode waves own no chunk."""
    step = workloads.build_step("mixed_tiny_decode", 515, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                q_dtype="bf16", cache_dtype="fp8", prefix=[700, 3, 0], new=[400, 1, 1],
                                kinds=["prefill", "decode", "decode"])
    run_mixed(step)


def test_mixed_step_two_launch_paths():
    """head_dim 64 with an fp8 cache, and a decode batch past one stream
    launch's table (the decode runs in two slices): the call launches the
    prefill and the decode one after the other, with the same results."""
    step = workloads.build_step("mixed_fp8_d64", 64, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                                q_dtype="bf16", cache_dtype="fp8", prefix=[40, 0, 300, 7],
                                new=[100, 33, 1, 1], kinds=["prefill", "prefill", "decode", "decode"])
    run_mixed(step)
    rng = np.random.default_rng(65)
    n_dec = 2100
    prefix = np.concatenate([[120], rng.integers(0, 30, size=n_dec)])
    new = np.concatenate([[64], np.ones(n_dec, np.int64)])
    step = workloads.build_step("mixed_fp8_big_batch", 65, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                                q_dtype="bf16", cache_dtype="fp8", prefix=prefix, new=new,
                                kinds=["prefill"] + ["decode"] * n_dec)
    run_mixed(step, pairs=sample_pairs(rng, n_dec, 8, 64))
