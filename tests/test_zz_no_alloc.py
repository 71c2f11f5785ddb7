"""The decode call that allocates nothing (pkv_paged_decode_noalloc): its
kernels use the library's static scratch array instead of a workspace.  Its
results must equal pkv_paged_decode's bit for bit (same kernels, same plan),
on consecutive calls that share the array, the later ones smaller."""

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import TOL, GpuStep, max_err, oracle_decode, oracle_write, out_f64, say
import paged_kv_cache_map_amd as pkv

pytestmark = pytest.mark.gpu


def _both(g, split_keys=0):
    """(pkv_paged_decode with its own workspace, pkv_paged_decode_noalloc)."""
    ref = g.decode(split_keys).clone()
    got = pkv.paged_decode_noalloc(g.dec_q, g.k_cache, g.v_cache, g.dec_bt, g.dec_len, g.s.scale,
                                   g.k_scale, g.v_scale, split_keys=split_keys)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_decode_matches_workspace_decode_on_consecutive_calls():
    big = workloads.config("llama8b_decode")                       # 64 sequences, bf16 cache
    small = workloads.config("llama8b_decode", batch=5, len_lo=1, len_hi=700,
                             cache_dtype="fp8")                     # smaller, other dtype
    for step in (big, small):
        need = pkv.paged_decode_workspace_size(len(step.decode_inputs()["seq_ids"]), step.num_heads,
                                               step.num_kv_heads, step.head_dim, step.block_size,
                                               step.decode_inputs()["block_table"].shape[1])
        assert 0 < need <= pkv.NOALLOC_SCRATCH_BYTES, need
    gb = GpuStep(big)
    gb.write()
    say("noalloc: first call", big.name, "batch", len(big.decode_inputs()["seq_ids"]))
    ref, got = _both(gb)
    assert torch.equal(ref, got)
    gs = GpuStep(small)
    gs.write()
    say("noalloc: second call (smaller)", small.name, small.cache_dtype)
    ref, got = _both(gs)
    assert torch.equal(ref, got)
    kc, vc = oracle_write(small)
    assert max_err(out_f64(got), oracle_decode(small, kc, vc)) <= TOL["fp8"]
    say("noalloc: third call (fixed splits)")
    ref, got = _both(gs, split_keys=256)
    assert torch.equal(ref, got)
    say("noalloc: the large call again, after the small ones")
    ref, got = _both(gb)
    assert torch.equal(ref, got)


def test_noalloc_decode_on_a_side_stream():
    step = workloads.config("llama8b_decode", batch=9, len_lo=1, len_hi=2000, num_heads=64,
                            num_kv_heads=8)
    g = GpuStep(step)
    g.write()
    ref = g.decode().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say("noalloc: side stream")
    with torch.cuda.stream(side):
        got = pkv.paged_decode_noalloc(g.dec_q, g.k_cache, g.v_cache, g.dec_bt, g.dec_len, step.scale,
                                       stream=side)
    side.synchronize()
    assert torch.equal(ref, got)


def test_noalloc_decode_in_slices():
    """2100 sequences: the stream plan runs two slices of 1050 one after the
    other, both through the static array."""
    rng = np.random.default_rng(41)
    n = 2100
    step = workloads.build_step("noalloc_slices", 41, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                                q_dtype="bf16", cache_dtype="bf16", prefix=rng.integers(0, 60, size=n),
                                new=[1] * n, kinds=["decode"] * n)
    need = pkv.paged_decode_workspace_size(n, 8, 2, 128, 16, step.decode_inputs()["block_table"].shape[1])
    assert 0 < need <= pkv.NOALLOC_SCRATCH_BYTES, need
    g = GpuStep(step)
    g.write()
    say("noalloc: two slices")
    ref, got = _both(g)
    assert torch.equal(ref, got)
    pairs = [(b, h) for b in (0, 1049, 1050, 2099) for h in range(8)]
    kc, vc = oracle_write(step)
    idx = tuple(np.array(pairs).T)
    assert max_err(out_f64(got)[idx], oracle_decode(step, kc, vc, pairs=pairs)[idx]) <= TOL["bf16"]
