"""What an fp8 P.V product would cost in accuracy (CPU study, no GPU).

The prefill kernel rounds the softmax weights p to bf16 before its P.V
matrix product.  A kernel that fed the E4M3 matrix cores instead would round
p to E4M3 (3 mantissa bits, subnormals below 2^-6).  This module emulates
both on the oracle's own arithmetic: the logits and their exponentials in
float64 exactly as the oracle takes them, then p rounded to the given format
(the oracle's E4M3 codec for fp8), the weighted sum and the sum of weights
over the rounded p.  The maximum absolute error against the oracle output on
sampled prefill rows of the mixed fp8 step (4 chunks of 512 queries over
4.8k-7.8k cached keys, 32 q heads on 8 KV heads) shows what such a kernel
costs against the 2e-2 bar of the fp8 parity tests on long rows.  (Rows
that see fewer keys fare worse: over the 600 rows of a reduced step with
656-826 keys the scaled E4M3 form reaches 1.5e-2, and a kernel built that
way measured 2.3e-2 there, so the prefill keeps bf16 p.)
"""

import numpy as np
import pytest

import workloads
from oracle import e4m3, paged

TOL = 2e-2


def _round_bf16(x):
    """Round-to-nearest-even of the float32 value of x to bf16, as float64."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _round_e4m3(x, prescale=1.0):
    """p * prescale through the oracle's E4M3 encoder (from its float32 value), back / prescale."""
    codes = e4m3.encode_fast(np.asarray(x * prescale, dtype=np.float32))
    return e4m3.decode(codes) / prescale


ROUNDINGS = {
    "exact": lambda p: p,
    "bf16": _round_bf16,
    "e4m3": _round_e4m3,
    "e4m3_x256": lambda p: _round_e4m3(p, 256.0),
}


def emulate_rows(step, kc, vc, rows, rounding):
    """Prefill output rows over the caches kc, vc (after the step's write) with
    p rounded by ``rounding`` before P.V and the sum of weights; the oracle's
    attention steps otherwise (causal, bottom-right aligned, per KV-head
    group)."""
    p_in = step.prefill_inputs()
    cu_q, cu_k = p_in["cu_seqlens_q"], p_in["cu_seqlens_k"]
    q = paged.to_f64(p_in["q"], step.q_dtype)
    group = step.num_heads // step.num_kv_heads
    out = {}
    for r in rows:
        b = int(np.searchsorted(cu_q, r, side="right") - 1)
        lq, lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        i = r - int(cu_q[b])
        seen = min(lk, i + lk - lq + 1)
        k = paged.to_f64(paged.gather(kc, p_in["block_table"][b], lk), "fp8", step.k_scale)[:seen]
        v = paged.to_f64(paged.gather(vc, p_in["block_table"][b], lk), "fp8", step.v_scale)[:seen]
        o = np.zeros((step.num_heads, step.head_dim))
        for h in range(step.num_heads):
            g = h // group
            s = step.scale * (k[:, g, :] @ q[r, h, :])
            p = rounding(np.exp(s - s.max()))
            o[h] = (p @ v[:, g, :]) / p.sum()
        out[r] = o
    return out


@pytest.fixture(scope="module")
def step_and_rows():
    step = workloads.config("mixed_fp8")
    cu = step.prefill_inputs()["cu_seqlens_q"]
    rng = np.random.default_rng(5)
    rows = set()
    for b in range(len(cu) - 1):  # first and last row of every chunk, 6 more at random
        rows.update((int(cu[b]), int(cu[b + 1]) - 1))
        rows.update(int(x) for x in rng.choice(np.arange(cu[b], cu[b + 1]), size=6, replace=False))
    # and the three rows with the largest E4M3 error in a wider sample (168
    # rows: the first and last of every chunk and 160 drawn with seed 11)
    rows.update((317, 1070, 1807))
    # the chunks attend their own new keys: the caches after the step's write
    kc, vc = paged.kv_cache_write(step.k_new, step.v_new, step.k_cache, step.v_cache, step.slot_map,
                                  step.q_dtype, step.cache_dtype, step.k_scale, step.v_scale)
    return step, kc, vc, sorted(rows)


def test_emulation_without_rounding_is_the_oracle(step_and_rows):
    """With p left exact, the emulation reproduces the oracle's rows."""
    step, kc, vc, rows = step_and_rows
    p_in = step.prefill_inputs()
    want = paged.varlen_prefill(p_in["q"], step.q_dtype, kc, vc, "fp8",
                                p_in["cu_seqlens_q"], p_in["cu_seqlens_k"], step.scale, True,
                                block_table=p_in["block_table"], k_scale=step.k_scale,
                                v_scale=step.v_scale, rows=rows[:4])
    got = emulate_rows(step, kc, vc, rows[:4], ROUNDINGS["exact"])
    for r in rows[:4]:
        assert np.all(np.isfinite(want[r]))
        np.testing.assert_allclose(got[r], want[r], rtol=0, atol=1e-12)


def test_roundings_are_the_formats():
    assert _round_bf16(np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]))[0] == 1.0          # tie to even
    assert _round_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    assert _round_e4m3(np.array([1.0 + 2 ** -4]))[0] == 1.0                               # tie to even
    assert _round_e4m3(np.array([2 ** -10]))[0] == 0.0                                    # below half the least subnormal: 0
    assert _round_e4m3(np.array([2 ** -9]))[0] == 2 ** -9                                 # least subnormal
    assert _round_e4m3(np.array([2 ** -10]), 256.0)[0] == 2 ** -10


def test_fp8_pv_error_on_the_mixed_fp8_prefill(step_and_rows):
    """The study's figures: bf16 p (what the kernel does) stays near 3e-4.
    E4M3 p misses the 2e-2 bar on rows whose weight is spread over many keys
    (7.4e-2 at row 317: the weights below 2^-10 round to zero), while E4M3
    of p scaled by 2^8 (small weights then stay out of the subnormals) stays
    near 5e-3, a margin of about 4x.  Over the 168-row sample: 3.3e-4 (bf16),
    7.4e-2 (E4M3), 5.5e-3 (E4M3 after the 2^8 scale)."""
    step, kc, vc, rows = step_and_rows
    exact = emulate_rows(step, kc, vc, rows, ROUNDINGS["exact"])
    err = {}
    for name in ("bf16", "e4m3", "e4m3_x256"):
        got = emulate_rows(step, kc, vc, rows, ROUNDINGS[name])
        err[name] = max(float(np.max(np.abs(got[r] - exact[r]))) for r in rows)
    print("max abs error over", len(rows), "rows x", step.num_heads, "heads:", err)
    assert err["bf16"] < 1e-3
    assert err["e4m3"] > TOL
    assert err["e4m3_x256"] < TOL / 3
