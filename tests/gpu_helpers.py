"""Shared plumbing of the GPU parity tests: move workloads to the device, run
the library through its binding, run the oracle on the same host bits."""

import sys

import numpy as np
import torch

import paged_kv_cache_map_amd as pkv
from oracle import paged
from workloads.device import to_dev, to_host  # noqa: F401

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 2e-2, "int8": 2e-2}   # max abs error vs the fp64 oracle


def say(*parts):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu]", *parts, flush=True)
    sys.stdout.flush()


def out_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_err(got, want):
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - want))) if got.size else 0.0


class GpuStep:
    """A workload step resident on the GPU."""

    def __init__(self, step):
        self.s = step
        self.k_cache = to_dev(step.k_cache, step.cache_dtype)
        self.v_cache = to_dev(step.v_cache, step.cache_dtype)
        self.k_new = to_dev(step.k_new, step.q_dtype)
        self.v_new = to_dev(step.v_new, step.q_dtype)
        self.slot_map = to_dev(step.slot_map, "i32")
        self.k_scale = None if step.k_scale is None else to_dev(step.k_scale, "f32")
        self.v_scale = None if step.v_scale is None else to_dev(step.v_scale, "f32")
        d = step.decode_inputs()
        self.dec = d
        self.dec_q = to_dev(d["q"], step.q_dtype) if len(d["seq_ids"]) else None
        self.dec_bt = to_dev(d["block_table"], "i32") if len(d["seq_ids"]) else None
        self.dec_len = to_dev(d["cache_seqlens"], "i32") if len(d["seq_ids"]) else None
        p = step.prefill_inputs()
        self.pre = p
        if len(p["seq_ids"]):
            self.pre_q = to_dev(p["q"], step.q_dtype)
            self.pre_cu_q = to_dev(p["cu_seqlens_q"], "i32")
            self.pre_cu_k = to_dev(p["cu_seqlens_k"], "i32")
            self.pre_bt = to_dev(p["block_table"], "i32")

    def write(self):
        pkv.kv_cache_write(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slot_map,
                           self.k_scale, self.v_scale)

    def decode(self, split_keys=0, workspace=None):
        return pkv.paged_decode(self.dec_q, self.k_cache, self.v_cache, self.dec_bt, self.dec_len,
                                self.s.scale, self.k_scale, self.v_scale, split_keys=split_keys,
                                workspace=workspace)

    def append_decode(self, split_keys=0, workspace=None):
        """The appending decode: stores the decode sequences' new rows and attends."""
        d = self.s.decode_append_inputs()
        return pkv.paged_decode_append(self.dec_q, to_dev(d["k_new"], self.s.q_dtype),
                                       to_dev(d["v_new"], self.s.q_dtype), self.k_cache, self.v_cache,
                                       self.dec_bt, to_dev(d["cache_seqlens"], "i32"), self.s.scale,
                                       self.k_scale, self.v_scale, split_keys=split_keys,
                                       workspace=workspace)

    def write_prefill_only(self):
        pkv.kv_cache_write(self.k_new, self.v_new, self.k_cache, self.v_cache,
                           to_dev(self.s.prefill_slot_map(), "i32"), self.k_scale, self.v_scale)

    def prefill(self):
        p = self.pre
        return pkv.varlen_prefill(self.pre_q, self.k_cache, self.v_cache, self.pre_cu_q,
                                  self.pre_cu_k, p["max_seqlen_q"], p["max_seqlen_k"], self.s.scale,
                                  True, self.pre_bt, self.k_scale, self.v_scale)


def oracle_write(step):
    return paged.kv_cache_write(step.k_new, step.v_new, step.k_cache, step.v_cache, step.slot_map,
                                step.q_dtype, step.cache_dtype, step.k_scale, step.v_scale)


def oracle_decode(step, kc, vc, pairs=None):
    d = step.decode_inputs()
    return paged.paged_decode(d["q"], step.q_dtype, kc, vc, step.cache_dtype, d["block_table"],
                              d["cache_seqlens"], step.scale, step.k_scale, step.v_scale, pairs=pairs)


def oracle_append_decode(step, pairs=None):
    """The oracle's appending decode on the step's decode sequences, after the
    oracle's write of the prefill sequences' tokens.  Returns (out, kc, vc)."""
    kc, vc = paged.kv_cache_write(step.k_new, step.v_new, step.k_cache, step.v_cache,
                                  step.prefill_slot_map(), step.q_dtype, step.cache_dtype,
                                  step.k_scale, step.v_scale)
    d = step.decode_append_inputs()
    return paged.paged_decode_append(d["q"], step.q_dtype, d["k_new"], d["v_new"], kc, vc,
                                     step.cache_dtype, d["block_table"], d["cache_seqlens"], step.scale,
                                     step.k_scale, step.v_scale, pairs=pairs)


def oracle_prefill(step, kc, vc, rows=None):
    p = step.prefill_inputs()
    return paged.varlen_prefill(p["q"], step.q_dtype, kc, vc, step.cache_dtype, p["cu_seqlens_q"],
                                p["cu_seqlens_k"], step.scale, True, block_table=p["block_table"],
                                k_scale=step.k_scale, v_scale=step.v_scale, rows=rows)


def assert_cache_equal(gpu_cache, want, dtype, what):
    got = to_host(gpu_cache, dtype)
    if not np.array_equal(got.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)):
        bad = np.argwhere(got.reshape(got.shape[0] * got.shape[1], -1) !=
                          want.reshape(want.shape[0] * want.shape[1], -1))
        raise AssertionError(f"{what}: {len(bad)} elements differ, first slots "
                             f"{np.unique(bad[:, 0])[:8].tolist()}")


def sample_pairs(rng, batch, heads, n):
    """n distinct (b, h) pairs, always including the first and last sequence."""
    pairs = {(0, 0), (batch - 1, heads - 1)}
    while len(pairs) < min(n, batch * heads):
        pairs.add((int(rng.integers(batch)), int(rng.integers(heads))))
    return sorted(pairs)


def unit_pairs(rng, batch, hq, hkv):
    """One q head, drawn at random, of every (sequence, KV head) unit."""
    group = hq // hkv
    return [(b, g * group + int(rng.integers(group))) for b in range(batch) for g in range(hkv)]


def sequence_pairs(rng, batch, heads):
    """Every sequence once (a random q head), plus the first and last pair."""
    return sorted({(b, int(rng.integers(heads))) for b in range(batch)} | {(0, 0), (batch - 1, heads - 1)})


def sample_rows(rng, cu, n):
    """Packed query rows: first and last row of every request plus n random ones."""
    rows = set()
    for b in range(len(cu) - 1):
        if cu[b + 1] > cu[b]:
            rows.update((int(cu[b]), int(cu[b + 1]) - 1))
    total = int(cu[-1])
    if total:
        rows.update(int(r) for r in rng.choice(total, size=min(n, total), replace=False))
    return sorted(rows)
