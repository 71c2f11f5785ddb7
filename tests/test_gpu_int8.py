"""GPU parity of INT8 caches (one fp32 scale per KV head; code = RNE(x /
scale) saturated to [-127, 127]): the write bit-exact against the oracle's
codec, decode (both plans), prefill (head_dim 128 and 64), the appending
decode and the mixed step, attention within 2e-2 of the fp64 oracle over the
stored codes."""

import numpy as np
import pytest

import paged_kv_cache_map_amd as pkv
import workloads
from gpu_helpers import assert_cache_equal, out_f64, sample_pairs, sample_rows, to_dev
from oracle import int8, paged
from test_gpu_append import check_append
from test_gpu_parity import run_step_and_check

pytestmark = pytest.mark.gpu


def test_int8_write_every_bf16_pattern():
    """All 65536 bf16 bit patterns (NaN and inf included) through the write,
    per-head scales 1 and 1/3: codes equal the oracle's bit for bit."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    hkv, d = 2, 128
    t = 65536 // (hkv * d)
    k = bits.reshape(t, hkv, d)
    v = bits[::-1].copy().reshape(t, hkv, d)
    scale = np.array([1.0, 1.0 / 3.0], np.float32)
    nb, bs = t // 16, 16
    kc = np.zeros((nb, bs, hkv, d), np.int8)
    slots = np.random.default_rng(5).permutation(t).astype(np.int32)
    want_k, want_v = paged.kv_cache_write(k, v, kc, kc, slots, "bf16", "int8", scale, scale)
    gk, gv = to_dev(kc, "int8"), to_dev(kc, "int8")
    pkv.kv_cache_write(to_dev(k, "bf16"), to_dev(v, "bf16"), gk, gv, to_dev(slots, "i32"),
                       to_dev(scale, "f32"), to_dev(scale, "f32"))
    assert_cache_equal(gk, want_k, "int8", "k")
    assert_cache_equal(gv, want_v, "int8", "v")


def test_int8_write_f32_source():
    rng = np.random.default_rng(6)
    t, hkv, d = 300, 4, 64
    k = (rng.standard_normal((t, hkv, d)) * 3).astype(np.float32)
    v = (rng.standard_normal((t, hkv, d)) * 3).astype(np.float32)
    k[0, 0, :4] = [np.nan, np.inf, -np.inf, 1e9]
    scale = np.array([0.01, 0.03, 0.05, 0.07], np.float32)
    kc = np.zeros((40, 8, hkv, d), np.int8)
    slots = np.random.default_rng(7).permutation(320)[:t].astype(np.int32)
    want_k, want_v = paged.kv_cache_write(k, v, kc, kc, slots, "f32", "int8", scale, scale)
    gk, gv = to_dev(kc, "int8"), to_dev(kc, "int8")
    pkv.kv_cache_write(to_dev(k, "f32"), to_dev(v, "f32"), gk, gv, to_dev(slots, "i32"),
                       to_dev(scale, "f32"), to_dev(scale, "f32"))
    assert_cache_equal(gk, want_k, "int8", "k")
    assert_cache_equal(gv, want_v, "int8", "v")


def test_int8_decode_every_code():
    """A one-key sequence returns its V row exactly: every int8 code in
    [-127, 127] decodes to its value (scale 1; integers are exact in bf16)."""
    codes = np.arange(-127, 128).astype(np.int8)
    hkv, d, bs = 1, 128, 16
    seqs = (len(codes) + d - 1) // d
    padded = np.resize(codes, seqs * d)
    v = np.full((seqs, bs, hkv, d), -128, np.int8)
    k = np.full((seqs, bs, hkv, d), -128, np.int8)
    v[:, 0, 0, :] = padded.reshape(seqs, d)
    k[:, 0, 0, :] = 1
    table = np.arange(seqs, dtype=np.int32)[:, None]
    ones = np.ones(1, np.float32)
    q = np.full((seqs, 4, d), 0x3F80, np.uint16)
    out = pkv.paged_decode(to_dev(q, "bf16"), to_dev(k, "int8"), to_dev(v, "int8"), to_dev(table, "i32"),
                           to_dev(np.ones(seqs, np.int32), "i32"), 0.1, to_dev(ones, "f32"), to_dev(ones, "f32"))
    got = out_f64(out)
    want = int8.decode(padded).reshape(seqs, d)
    for h in range(4):
        assert np.array_equal(got[:, h, :], want)


@pytest.mark.parametrize("hq,hkv,d,bs", [(32, 8, 128, 16), (8, 8, 64, 32), (16, 1, 128, 8), (8, 2, 64, 16)])
def test_int8_decode_shapes(hq, hkv, d, bs):
    step = workloads.config("llama8b_decode", batch=5, len_lo=1, len_hi=700, num_heads=hq, num_kv_heads=hkv,
                            head_dim=d, block_size=bs, cache_dtype="int8")
    run_step_and_check(step, split_keys=128)   # fixed splits (vector kernels)
    run_step_and_check(step)                   # stream-K on the matrix cores


@pytest.mark.parametrize("hq,hkv,d,bs", [(32, 8, 128, 16), (8, 2, 64, 64), (16, 4, 128, 32)])
def test_int8_prefill_shapes(hq, hkv, d, bs):
    rng = np.random.default_rng(hq * 1000 + d + bs + 1)
    lq = rng.integers(1, 300, size=4)
    pre = rng.integers(0, 260, size=4)
    step = workloads.build_step("prefill_int8", 6000 + hq + d + bs, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                                block_size=bs, q_dtype="bf16", cache_dtype="int8", prefix=pre, new=lq,
                                kinds=["prefill"] * 4)
    run_step_and_check(step)


def test_mixed_int8_reduced():
    step = workloads.config("mixed_int8", prefill_chunks=3, chunk=200, decode_batch=12, p_hi=700, len_lo=1,
                            len_hi=900)
    run_step_and_check(step)


def test_mixed_int8_full_sampled():
    step = workloads.config("mixed_int8")
    rng = np.random.default_rng(12)
    rows = sample_rows(rng, step.prefill_inputs()["cu_seqlens_q"], 48)
    pairs = sample_pairs(rng, 256, 32, 40)
    run_step_and_check(step, full=False, rows=rows, pairs=pairs)


@pytest.mark.parametrize("split", [0, 256])
def test_int8_append(split):
    step = workloads.config("mixed_int8", prefill_chunks=2, chunk=100, decode_batch=20, p_hi=300, len_lo=0,
                            len_hi=600)
    check_append(step, split_keys=split)

