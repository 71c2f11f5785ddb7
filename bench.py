"""Throughput of the paged-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs all|main]

A step is one pass of the hot path over one batch: the KV write of the new
tokens followed by the attention call(s) that read them (decode, prefill, or
both for the mixed step).  The headline line measures the largest decode
workload that fits one GPU, the Llama-3.1-70B-layer-shaped long-context step
(8 sequences x 131 072 cached tokens, 64/8 heads, head_dim 128, bf16, block
size 16, randomly scattered blocks) done by the appending decode, which
stores the 8 new tokens and attends in one call; `value` is that step's
algorithmic HBM bytes (write + decode) per second.  The same step as two
calls (slot-map write, then the plain decode), the Llama-3.1-8B-shaped decode
(batch 64, contexts U{512..4096}), the varlen prefill and the mixed steps are
reported beside it, with the prefill kernel's own roofline.  Inputs are
resident in HBM before timing starts; small KV pools are replicated and
rotated so that consecutive steps never find them in the 256 MB Infinity
Cache.  Kernel durations come from HIP events recorded on the stream the
kernels run on.  One JSON line is printed.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "paged-decode HBM GB/s (% of peak); varlen prefill TFLOPS (% MFMA peak)"
ROTATE_BYTES = 1 << 30         # replicate small pools to at least this many bytes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--configs", default="all", choices=["all", "main"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--split-keys", type=int, default=0,
                    help="decode split size in keys (0: the library's automatic plan)")
    ap.add_argument("--only", default=None,
                    help="diagnostic: time one named workload and print its kernel times only")
    ap.add_argument("--append", action="store_true",
                    help="diagnostic (--only): store the decode tokens with the appending decode")
    ap.add_argument("--mixed", action="store_true",
                    help="diagnostic (--only): prefill and decode through the one mixed-step call")
    ap.add_argument("--set", action="append", default=[], metavar="KEY=VALUE",
                    help="diagnostic (--only): a workload override such as batch=3000 or cache_dtype=fp8")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also time a plain 512 MiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (what the method must move / compute)
# ---------------------------------------------------------------------------

ELT = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}


def write_bytes(step):
    """Read the new K/V rows, write them to the cache, read the slot map."""
    row = step.num_kv_heads * step.head_dim
    return step.num_tokens * (2 * row * (ELT[step.q_dtype] + ELT[step.cache_dtype]) + 4)


def decode_bytes(step):
    d = step.decode_inputs()
    b = len(d["seq_ids"])
    keys = int(d["cache_seqlens"].astype(np.int64).sum())
    kv = keys * 2 * step.num_kv_heads * step.head_dim * ELT[step.cache_dtype]
    qo = 2 * b * step.num_heads * step.head_dim * ELT[step.q_dtype]
    meta = 4 * b + 4 * sum(-(-int(n) // step.block_size) for n in d["cache_seqlens"])
    return kv + qo + meta


def prefill_flops(step):
    """4 * Hq * D per visible (query, key) pair: Q.K and P.V, 2 flops per MAC."""
    p = step.prefill_inputs()
    lq = np.diff(p["cu_seqlens_q"]).astype(np.int64)
    lk = np.diff(p["cu_seqlens_k"]).astype(np.int64)
    pre = lk - lq
    pairs = int(np.sum(lq * pre + lq * (lq + 1) // 2))
    return 4 * step.num_heads * step.head_dim * pairs


# HBM traffic of one call of the dominant kernels, from the hardware counters
# (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, averaged per dispatch), each
# scaled by bytes / counter of a plain 512 MiB device copy measured in the
# same runs: the appending decode call (decode kernel + merge) on the headline
# workload, and the prefill kernel on varlen_prefill_prefix.  The figures
# belong to the kernel sources with the given digest: after any change to
# them the traffic is reported as null until the counters are taken again.
DECODE_TRAFFIC = {"digest": "050d554da647d6d2", "read_bytes": 4317107797, "write_bytes": 4426240}
PREFILL_TRAFFIC = {"digest": "050d554da647d6d2", "read_bytes": 1669342094, "write_bytes": 127675573}
KERNEL_SOURCES = ("paged_kv_cache_map_amd/csrc/paged_decode.hip",
                  "paged_kv_cache_map_amd/csrc/varlen_prefill.hip",
                  "paged_kv_cache_map_amd/csrc/attention.hip",
                  "paged_kv_cache_map_amd/csrc/work_queue.hpp",
                  "paged_kv_cache_map_amd/csrc/pkv_device.hpp",
                  "paged_kv_cache_map_amd/csrc/pkv_plan.cpp",
                  "paged_kv_cache_map_amd/csrc/pkv_internal.h")


def kernel_sources_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic(table):
    if table is None or table["digest"] != kernel_sources_digest():
        return None
    return table["read_bytes"] + table["write_bytes"]


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------


class Runner:
    """A workload step on the GPU with `copies` rotated replicas of its KV pool."""

    def __init__(self, step, copies=1, split_keys=0, append=False, mixed=False):
        import torch
        from workloads.device import to_dev
        self.torch = torch
        self.s = step
        self.split_keys = split_keys
        self.append = append
        self.mixed = mixed  # prefill and decode through the one mixed-step call
        self.copies = []
        for _ in range(copies):
            self.copies.append((to_dev(step.k_cache, step.cache_dtype),
                                to_dev(step.v_cache, step.cache_dtype)))
        self.k_new = to_dev(step.k_new, step.q_dtype)
        self.v_new = to_dev(step.v_new, step.q_dtype)
        self.slot_map = to_dev(step.slot_map, "i32")
        self.k_scale = None if step.k_scale is None else to_dev(step.k_scale, "f32")
        self.v_scale = None if step.v_scale is None else to_dev(step.v_scale, "f32")
        d = step.decode_inputs()
        self.has_decode = len(d["seq_ids"]) > 0
        if self.has_decode:
            import paged_kv_cache_map_amd as pkv
            self.dq = to_dev(d["q"], step.q_dtype)
            self.dbt = to_dev(d["block_table"], "i32")
            self.dlen = to_dev(d["cache_seqlens"], "i32")
            self.dout = torch.empty_like(self.dq)
            nb, bs = step.k_cache.shape[:2]
            need = pkv.paged_decode_workspace_size(self.dq.shape[0], step.num_heads,
                                                   step.num_kv_heads, step.head_dim, bs,
                                                   d["block_table"].shape[1], split_keys)
            self.dws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            if append:  # the decode sequences' rows go through the appending decode
                a = step.decode_append_inputs()
                self.akn = to_dev(a["k_new"], step.q_dtype)
                self.avn = to_dev(a["v_new"], step.q_dtype)
                self.alen = to_dev(a["cache_seqlens"], "i32")
                self.slot_map = to_dev(step.prefill_slot_map(), "i32")
        self.write_tokens = int((step.prefill_slot_map() >= 0).sum()) if append else step.num_tokens
        p = step.prefill_inputs()
        self.has_prefill = len(p["seq_ids"]) > 0
        if self.has_prefill:
            self.p = p
            self.pq = to_dev(p["q"], step.q_dtype)
            self.pcq = to_dev(p["cu_seqlens_q"], "i32")
            self.pck = to_dev(p["cu_seqlens_k"], "i32")
            self.pbt = to_dev(p["block_table"], "i32")
            self.pout = torch.empty_like(self.pq)
        torch.cuda.synchronize()

    def prefill(self, kc, vc):
        import paged_kv_cache_map_amd as pkv
        p = self.p
        pkv.varlen_prefill(self.pq, kc, vc, self.pcq, self.pck, p["max_seqlen_q"], p["max_seqlen_k"],
                           self.s.scale, True, self.pbt, self.k_scale, self.v_scale, out=self.pout)

    def run(self, i, ev=None):
        import paged_kv_cache_map_amd as pkv
        kc, vc = self.copies[i % len(self.copies)]
        s = self.s
        if ev is not None:
            ev[0].record()
        if self.write_tokens:
            pkv.kv_cache_write(self.k_new, self.v_new, kc, vc, self.slot_map, self.k_scale, self.v_scale)
        if ev is not None:
            ev[1].record()
        if self.mixed:
            p = self.p
            pkv.mixed_attention(kc, vc, s.scale,
                                dict(q=self.pq, cu_seqlens_q=self.pcq, cu_seqlens_k=self.pck,
                                     max_seqlen_q=p["max_seqlen_q"], max_seqlen_k=p["max_seqlen_k"],
                                     block_table=self.pbt, out=self.pout),
                                dict(q=self.dq, block_table=self.dbt, cache_seqlens=self.dlen, out=self.dout),
                                self.k_scale, self.v_scale, workspace=self.dws)
            if ev is not None:
                ev[2].record()
                ev[3].record()
            return
        if self.has_prefill:
            self.prefill(kc, vc)
        if ev is not None and self.has_prefill:
            ev[2].record()
        elif ev is not None:
            ev[2] = ev[1]
        if self.has_decode and self.append:
            pkv.paged_decode_append(self.dq, self.akn, self.avn, kc, vc, self.dbt, self.alen, s.scale,
                                    self.k_scale, self.v_scale, out=self.dout, split_keys=self.split_keys,
                                    workspace=self.dws)
        elif self.has_decode:
            pkv.paged_decode(self.dq, kc, vc, self.dbt, self.dlen, s.scale, self.k_scale,
                             self.v_scale, out=self.dout, split_keys=self.split_keys,
                             workspace=self.dws)
        if ev is not None:
            ev[3].record()

    def time(self, steps, warmup):
        """ms_per_step from K back-to-back steps with nothing else enqueued,
        then per-kernel times from a second pass with HIP events around each
        call (recorded on the library's stream)."""
        torch = self.torch
        for i in range(warmup):
            self.run(i)
        torch.cuda.synchronize()
        region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t0 = time.perf_counter()
        region[0].record()
        for i in range(steps):
            self.run(warmup + i)
        region[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            self.run(warmup + steps + i, evs[i])
        torch.cuda.synchronize()
        write = [e[0].elapsed_time(e[1]) for e in evs]
        pre = [e[1].elapsed_time(e[2]) for e in evs] if self.has_prefill else [0.0]
        dec = [e[2].elapsed_time(e[3]) for e in evs] if self.has_decode else [0.0]
        # the write alone, K calls back to back (idempotent: the same rows to
        # the same slots), HIP events around the region
        write_region = 0.0
        if self.write_tokens:
            import paged_kv_cache_map_amd as pkv
            wr = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            wr[0].record()
            for i in range(steps):
                kc, vc = self.copies[i % len(self.copies)]
                pkv.kv_cache_write(self.k_new, self.v_new, kc, vc, self.slot_map, self.k_scale, self.v_scale)
            wr[1].record()
            torch.cuda.synchronize()
            write_region = wr[0].elapsed_time(wr[1]) / steps
        # the prefill alone, K calls back to back (it only reads the caches),
        # HIP events around the region
        prefill_region = 0.0
        if self.has_prefill and not self.mixed:
            pr = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            pr[0].record()
            for i in range(steps):
                kc, vc = self.copies[i % len(self.copies)]
                self.prefill(kc, vc)
            pr[1].record()
            torch.cuda.synchronize()
            prefill_region = pr[0].elapsed_time(pr[1]) / steps
        return dict(ms_per_step=wall * 1e3 / steps,
                    write_region_ms=write_region, prefill_region_ms=prefill_region,
                    region_ms_per_step=region[0].elapsed_time(region[1]) / steps,
                    write_ms=float(np.mean(write)), write_ms_min=float(np.min(write)),
                    prefill_ms=float(np.mean(pre)), prefill_ms_min=float(np.min(pre)),
                    decode_ms=float(np.mean(dec)), decode_ms_min=float(np.min(dec)))


def copy_probe(reps=5, nbytes=512 << 20):
    """A plain device-to-device copy of a known size (torch's copy kernel)."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": float(np.mean(ms)),
            "gbs": 2 * nbytes / (float(np.mean(ms)) * 1e6)}


def measure_copy_blocks(steps, warmup, pairs=4096, num_blocks=12288):
    """The copy-on-write block copy on Llama-3.1-8B-shaped blocks (16 tokens x
    8 KV heads x 128, bf16: 32 KiB per block and cache): ``pairs`` random
    (src, dst) pairs over a pool of ``num_blocks`` blocks (targets distinct,
    never a source).  Algorithmic bytes: every copied byte read once and
    written once."""
    import torch
    import paged_kv_cache_map_amd as pkv
    rng = np.random.default_rng(5)
    shape = (num_blocks, 16, 8, 128)
    k = torch.empty(shape, dtype=torch.bfloat16, device="cuda").normal_()
    v = torch.empty_like(k).normal_()
    perm = rng.permutation(num_blocks)
    pr = np.stack([rng.choice(perm[pairs:], size=pairs), perm[:pairs]], 1).astype(np.int32)
    pt = torch.from_numpy(pr).cuda()
    for _ in range(warmup):
        pkv.copy_blocks(k, v, pt)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        pkv.copy_blocks(k, v, pt)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    nbytes = 2 * 2 * pairs * 16 * 8 * 128 * 2
    del k, v
    torch.cuda.empty_cache()
    return {"pairs": pairs, "block_bytes_per_cache": 32768, "bytes": nbytes, "ms": round(ms, 5),
            "gbs": round(nbytes / (ms * 1e6), 2), "frac_hbm": round(nbytes / (ms * 1e6) / HBM_PEAK_GBS, 4)}


def measure_write_sweep(steps, sizes=(65536, 262144)):
    """The slot-map write alone at large token counts (8 KV heads x 128, bf16
    source and cache, block size 16, slots a random permutation of the pool):
    where launch latency no longer matters.  Algorithmic bytes per token:
    2 x 2 KiB read + 2 x 2 KiB written + 4 (its slot)."""
    import torch
    import paged_kv_cache_map_amd as pkv
    out = {}
    rng = np.random.default_rng(9)
    for t in sizes:
        k = torch.empty((t, 8, 128), dtype=torch.bfloat16, device="cuda").normal_()
        v = torch.empty_like(k).normal_()
        kc = torch.empty((t // 16, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        slots = torch.from_numpy(rng.permutation(t).astype(np.int32)).cuda()
        pkv.kv_cache_write(k, v, kc, vc, slots)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            pkv.kv_cache_write(k, v, kc, vc, slots)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        nbytes = t * (2 * 8 * 128 * (2 + 2) + 4)
        out[str(t)] = {"ms": round(ms, 5), "gbs": round(nbytes / (ms * 1e6), 2),
                       "frac_hbm": round(nbytes / (ms * 1e6) / HBM_PEAK_GBS, 4)}
        del k, v, kc, vc, slots
        torch.cuda.empty_cache()
    return out


def copies_for(step):
    pool = step.k_cache.nbytes + step.v_cache.nbytes
    return max(1, math.ceil(ROTATE_BYTES / pool))


def measure(name, steps, warmup, split_keys=0, append=False, mixed=False, **overrides):
    """Time one workload step.  append=True: the decode sequences' new rows
    are stored by the appending decode call (one launch for their write and
    their attention); the slot-map write then covers the prefill tokens only,
    and the decode figures count the appended rows' write bytes as well."""
    import workloads
    step = workloads.config(name, **overrides)
    r = Runner(step, copies_for(step), split_keys, append, mixed)
    t = r.time(steps, warmup)
    res = dict(t)
    if mixed:  # one call for both parts: its time is the prefill's plus the decode's share
        res["mixed_call_ms"] = t["prefill_ms"] + t["decode_ms"]
    step_write = write_bytes(step)
    res["write_bytes"] = step_write * r.write_tokens // max(step.num_tokens, 1)
    # per-call events carry a few microseconds of their own: the write's
    # rate comes from the back-to-back region
    res["write_gbs"] = res["write_bytes"] / (t["write_region_ms"] * 1e6) if r.write_tokens else 0.0
    res["write_gbs_single_call_events"] = res["write_bytes"] / (t["write_ms"] * 1e6) if r.write_tokens else 0.0
    if mixed:
        res["decode_bytes"] = decode_bytes(step)
        res["prefill_flops"] = prefill_flops(step)
        del r
        import torch
        torch.cuda.empty_cache()
        return step, res
    if r.has_decode:
        res["decode_bytes"] = decode_bytes(step) + (step_write - res["write_bytes"])
        res["decode_gbs"] = res["decode_bytes"] / (t["decode_ms"] * 1e6)
        res["decode_frac_hbm"] = res["decode_gbs"] / HBM_PEAK_GBS
    if r.has_prefill:
        res["prefill_flops"] = prefill_flops(step)
        # as for the write: the rate comes from the back-to-back region (events
        # around single calls read the prefill about a tenth slower than the
        # kernel trace does)
        res["prefill_tflops"] = res["prefill_flops"] / (t["prefill_region_ms"] * 1e9)
        res["prefill_tflops_single_call_events"] = res["prefill_flops"] / (t["prefill_ms"] * 1e9)
        res["prefill_frac_mfma"] = res["prefill_tflops"] / BF16_PEAK_TFLOPS
    del r
    import torch
    torch.cuda.empty_cache()
    return step, res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# ---------------------------------------------------------------------------


def _threads():
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - reporting only
        blas = 1
    return blas, len(os.sched_getaffinity(0))


def cpu_baseline_decode(step, min_seconds=10.0):
    """The oracle's decode of whole sequences of the step, over the caches
    after the step's write (made before timing), one sequence after another
    until about ten seconds of CPU work; GB/s of the sequences' algorithmic
    decode bytes."""
    from oracle import paged
    blas, cores = _threads()
    kc, vc = paged.kv_cache_write(step.k_new, step.v_new, step.k_cache, step.v_cache, step.slot_map,
                                  step.q_dtype, step.cache_dtype, step.k_scale, step.v_scale)
    d = step.decode_inputs()
    nseq = len(d["seq_ids"])
    row = 2 * step.num_kv_heads * step.head_dim * ELT[step.cache_dtype]
    done, nbytes, keys, t0 = 0, 0, 0, time.perf_counter()
    while True:
        sel = [done % nseq]
        n = int(d["cache_seqlens"][sel[0]])
        paged.paged_decode(d["q"][sel], step.q_dtype, kc, vc, step.cache_dtype, d["block_table"][sel],
                           d["cache_seqlens"][sel], step.scale, step.k_scale, step.v_scale)
        nbytes += n * row + 2 * step.num_heads * step.head_dim * ELT[step.q_dtype] + 4 + 4 * -(-n // step.block_size)
        keys += n
        done += 1
        secs = time.perf_counter() - t0
        if secs >= min_seconds:
            break
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": min(cores, blas), "kind": "oracle",
            "sample": (f"{done} whole sequence{'s' if done != 1 else ''} ({keys} keys, all {step.num_heads} q heads) of the {step.name} "
                       f"decode, oracle paged_decode over the caches after the step's write, fp64 numpy, "
                       f"{secs:.1f} s; BLAS threads {blas}, host CPUs available {cores}")}


def cpu_baseline_prefill(step, min_seconds=10.0, rows_per_call=64):
    """The oracle's prefill of consecutive blocks of query rows of the step
    (64 rows a call, requests in order), over the caches after the step's
    write, until about ten seconds of CPU work; GFLOP/s of the rows' useful
    flops (4 Hq D per visible (query, key) pair)."""
    from oracle import paged
    blas, cores = _threads()
    kc, vc = paged.kv_cache_write(step.k_new, step.v_new, step.k_cache, step.v_cache, step.slot_map,
                                  step.q_dtype, step.cache_dtype, step.k_scale, step.v_scale)
    p = step.prefill_inputs()
    cu_q, cu_k = p["cu_seqlens_q"].astype(np.int64), p["cu_seqlens_k"].astype(np.int64)
    total = int(cu_q[-1])
    flops, nrows, r0, t0 = 0, 0, 0, time.perf_counter()
    while True:
        b = int(np.searchsorted(cu_q, r0, side="right") - 1)
        r1 = min(r0 + rows_per_call, int(cu_q[b + 1]))
        rows = np.arange(r0, r1)
        paged.varlen_prefill(p["q"], step.q_dtype, kc, vc, step.cache_dtype, p["cu_seqlens_q"], p["cu_seqlens_k"],
                             step.scale, True, block_table=p["block_table"], k_scale=step.k_scale,
                             v_scale=step.v_scale, rows=rows)
        lq, lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        visible = (rows - cu_q[b]) + (lk - lq) + 1
        flops += 4 * step.num_heads * step.head_dim * int(np.clip(visible, 0, lk).sum())
        nrows += len(rows)
        r0 = r1 % total
        secs = time.perf_counter() - t0
        if secs >= min_seconds:
            break
    return {"value": round(flops / secs / 1e9, 4), "unit": "GFLOP/s", "cores": min(cores, blas), "kind": "oracle",
            "sample": (f"{nrows} query rows (blocks of up to {rows_per_call} rows, requests in order) of the "
                       f"{step.name} prefill, all {step.num_heads} q heads, oracle varlen_prefill over the caches "
                       f"after the step's write, fp64 numpy, {secs:.1f} s; BLAS threads {blas}, host CPUs "
                       f"available {cores}")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import paged_kv_cache_map_amd as pkv
    pkv.library()

    if args.only:
        print(f"[bench] {args.only} (diagnostic)", flush=True)
        overrides = {}
        for item in args.set:
            key, val = item.split("=", 1)
            overrides[key] = int(val) if val.lstrip("-").isdigit() else val
        _, res = measure(args.only, args.steps, args.warmup, args.split_keys, args.append, args.mixed,
                         **overrides)
        if args.copy_probe:
            res["copy_probe"] = copy_probe()
        print(json.dumps({"diagnostic": args.only, "overrides": overrides,
                          **{k: (round(v, 5) if isinstance(v, float) else v) for k, v in res.items()}}),
              flush=True)
        return

    # The headline step: the largest decode workload of one GPU, done by the
    # appending decode (one call for the 8 new rows and the attention); the
    # same step as two calls, and the 8B-shaped decode both ways, beside it.
    head = "llama70b_long_decode"
    print(f"[bench] {head} (appending decode)", flush=True)
    step, main_res = measure(head, args.steps, args.warmup, args.split_keys, append=True)
    step_bytes = main_res["write_bytes"] + main_res["decode_bytes"]
    value = step_bytes / (main_res["ms_per_step"] * 1e6)
    d = step.decode_inputs()
    achieved = main_res["decode_bytes"] / (main_res["region_ms_per_step"] * 1e6)
    rnd = lambda res: {k: (round(v, 5) if isinstance(v, float) else v) for k, v in res.items()}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, random block permutation)",
        "config": {"workload": "llama70b_long_decode: Llama-3.1-70B-layer-shaped long-context decode step "
                               "(kv write + paged decode of 8 sequences x 131072 cached tokens, one "
                               "appending-decode call)",
                   "batch": int(len(d["seq_ids"])), "num_heads": step.num_heads,
                   "num_kv_heads": step.num_kv_heads, "head_dim": step.head_dim,
                   "block_size": step.block_size,
                   "context": "131072 cached tokens each (+1 new token)",
                   "keys_total": int(d["cache_seqlens"].sum()),
                   "step_bytes": int(step_bytes)},
        # the timed steps are nothing but back-to-back appending-decode calls:
        # HIP events around the whole timed region give the call's average
        "roofline": {"kernel": "paged_decode_append call (stream-K plan on the matrix cores: "
                               "decode_mfma_kernel<append> + stream_merge_kernel); bytes = decode + appended rows",
                     "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic(DECODE_TRAFFIC),
                     "algorithmic_bytes_per_launch": int(main_res["decode_bytes"]),
                     "avg_launch_ms": round(main_res["region_ms_per_step"], 5),
                     "avg_launch_ms_single_call_events": round(main_res["decode_ms"], 5)},
        "kernels": {head: rnd(main_res)},
    }
    print(f"[bench] {head} (slot-map write + plain decode)", flush=True)
    _, sep = measure(head, args.steps, args.warmup, args.split_keys)
    line["kernels"][head + "_separate_calls"] = {**rnd(sep), "step_gbs": round(step_bytes / (sep["ms_per_step"] * 1e6), 2)}
    print("[bench] llama8b_decode (appending decode)", flush=True)
    s8, r8 = measure("llama8b_decode", args.steps, args.warmup, args.split_keys, append=True)
    b8 = r8["write_bytes"] + r8["decode_bytes"]
    line["kernels"]["llama8b_decode"] = {**rnd(r8), "step_gbs": round(b8 / (r8["ms_per_step"] * 1e6), 2),
                                         "call_gbs": round(r8["decode_bytes"] / (r8["region_ms_per_step"] * 1e6), 2)}
    print("[bench] llama8b_decode (slot-map write + plain decode)", flush=True)
    _, s8sep = measure("llama8b_decode", args.steps, args.warmup, args.split_keys)
    line["kernels"]["llama8b_decode_separate_calls"] = {**rnd(s8sep),
                                                        "step_gbs": round(b8 / (s8sep["ms_per_step"] * 1e6), 2)}
    pre_step = None
    if args.configs == "all":
        for name in ("varlen_prefill_prefix", "mixed_fp8", "mixed_int8"):
            print(f"[bench] {name}", flush=True)
            st, res = measure(name, max(5, args.steps // 2), 2, args.split_keys)
            if name == "varlen_prefill_prefix":
                pre_step = st
            line["kernels"][name] = rnd(res)
        for name in ("mixed_fp8", "mixed_int8"):
            print(f"[bench] {name} (one mixed-step call)", flush=True)
            _, res = measure(name, max(3, args.steps // 2), 3, args.split_keys, mixed=True)
            sep_calls = line["kernels"][name]
            line["kernels"][name + "_one_call"] = {
                "ms_per_step": round(res["ms_per_step"], 5), "region_ms_per_step": round(res["region_ms_per_step"], 5),
                "mixed_call_ms": round(res["mixed_call_ms"], 5),
                "separate_calls_ms": round(sep_calls["prefill_ms"] + sep_calls["decode_ms"], 5)}
        pre = line["kernels"]["varlen_prefill_prefix"]
        # a prefill call is its counter-clearing kernel (a few microseconds)
        # and the prefill kernel; its average over back-to-back calls
        line["roofline_prefill"] = {
            "kernel": "prefill_kernel<bf16, D=128, paged> (varlen_prefill_prefix call)",
            "bound": "mfma", "achieved": pre["prefill_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre["prefill_tflops"] / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic(PREFILL_TRAFFIC),
            "algorithmic_flops_per_launch": int(pre["prefill_flops"]),
            "avg_launch_ms": pre["prefill_region_ms"],
            "avg_launch_ms_single_call_events": pre["prefill_ms"]}
        line["secondary"] = {
            "varlen_prefill_tflops": pre["prefill_tflops"],
            "varlen_prefill_frac_mfma": pre["prefill_frac_mfma"],
            "varlen_write_gbs": pre["write_gbs"],
            "llama8b_decode_call_gbs": line["kernels"]["llama8b_decode"]["call_gbs"],
            "llama8b_decode_step_gbs": line["kernels"]["llama8b_decode"]["step_gbs"],
            "mixed_fp8_decode_gbs": line["kernels"]["mixed_fp8"]["decode_gbs"],
            "mixed_fp8_prefill_tflops": line["kernels"]["mixed_fp8"]["prefill_tflops"],
            "mixed_fp8_one_call_ms": line["kernels"]["mixed_fp8_one_call"]["mixed_call_ms"],
            "mixed_int8_decode_gbs": line["kernels"]["mixed_int8"]["decode_gbs"],
            "mixed_int8_prefill_tflops": line["kernels"]["mixed_int8"]["prefill_tflops"],
        }
    print("[bench] write sweep", flush=True)
    line["kernels"]["write_sweep_tokens"] = measure_write_sweep(max(5, args.steps // 2))
    print("[bench] copy_blocks", flush=True)
    line["kernels"]["copy_blocks"] = measure_copy_blocks(max(5, args.steps), 2)
    if args.copy_probe:
        print("[bench] copy probe", flush=True)
        line["kernels"]["copy_probe"] = copy_probe()
    if not args.no_cpu:
        print(f"[bench] cpu baseline (oracle, {head} decode)", flush=True)
        line["cpu_baseline"] = cpu_baseline_decode(step)
        del step
        if pre_step is None:
            import workloads
            pre_step = workloads.config("varlen_prefill_prefix")
        print("[bench] cpu baseline (oracle, varlen_prefill_prefix prefill)", flush=True)
        line["cpu_baseline_prefill"] = cpu_baseline_prefill(pre_step)
        print("[bench] cpu baseline (oracle, llama8b_decode decode)", flush=True)
        line["cpu_baseline_llama8b_decode"] = cpu_baseline_decode(s8)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
