"""GPU parity of block management: the copy-on-write block copy against the
oracle's copy (bit-exact over the whole pool), and forked sequences stepping
through the host block manager, the block copy and the appending decode,
checked against the oracle step by step (caches bit-exact, attention within
the dtype's tolerance)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_map_amd as pkv
from gpu_helpers import TOL, assert_cache_equal, max_err, out_f64, say, to_dev
from oracle import blocks, paged
from workloads import configs

pytestmark = pytest.mark.gpu


def _pool(seed, shape, dtype):
    if dtype == "fp8":
        return configs._fp8_codes(seed, 4, shape), configs._fp8_codes(seed, 5, shape)
    if dtype == "int8":
        return configs._int8_codes(seed, 4, shape), configs._int8_codes(seed, 5, shape)
    return configs._normal(seed, 4, shape, dtype), configs._normal(seed, 5, shape, dtype)


# (num_blocks, block_size, Hkv, D, dtype, pairs)
COPY_CASES = [
    (64, 16, 8, 128, "bf16", 20),
    (300, 16, 8, 128, "fp8", 120),
    (40, 32, 2, 64, "f32", 15),
    (50, 8, 1, 64, "fp8", 20),     # 512-byte blocks: most lanes of a workgroup idle
    (20, 256, 8, 128, "bf16", 8),  # 512 KiB blocks: 32 workgroups per block and cache
    (90, 16, 8, 128, "int8", 40),
]


@pytest.mark.parametrize("nb,bs,hkv,d,dt,npairs", COPY_CASES,
                         ids=[f"{c[4]}_nb{c[0]}_bs{c[1]}_h{c[2]}_d{c[3]}" for c in COPY_CASES])
def test_copy_blocks_bit_exact(nb, bs, hkv, d, dt, npairs):
    rng = np.random.default_rng(nb + bs + d)
    k, v = _pool(nb + d, (nb, bs, hkv, d), dt)
    perm = rng.permutation(nb)
    dst = perm[:npairs]
    src = rng.choice(perm[npairs:], size=npairs)       # sources may repeat, never a target
    pairs = np.stack([src, dst], 1).astype(np.int32)
    bad = np.array([[nb + 3, int(perm[-1])], [int(perm[-2]), -1]], np.int32)  # move nothing
    say("copy_blocks", dt, nb, bs, hkv, d, npairs)
    gk, gv = to_dev(k, dt), to_dev(v, dt)
    pkv.copy_blocks(gk, gv, to_dev(np.concatenate([pairs, bad]), "i32"))
    torch.cuda.synchronize()
    wk, wv = blocks.copy_blocks(k, v, pairs)
    assert_cache_equal(gk, wk, dt, "k_cache")
    assert_cache_equal(gv, wv, dt, "v_cache")


@pytest.mark.parametrize("dt", ["bf16", "fp8", "int8"])
def test_forked_sequences_copy_on_write_then_decode(dt):
    """Prompts written through the block manager's slots; each prompt is
    forked once; both copies then decode three tokens each with the appending
    decode, the manager's copy pairs applied by the block copy first."""
    rng = np.random.default_rng(7)
    hq, hkv, d, bs = 16, 4, 128, 16
    nb, width = 160, 24
    prompts = [5, 16, 33, 70, 1]
    bm = pkv.BlockManager(nb, bs)
    rows, lens = [], []
    slot_map = []
    for n in prompts:
        row = [-1] * width
        for t in range(n):
            slot, copy = bm.append_slot(row, t)
            assert copy is None
            slot_map.append(slot)
        rows.append(row)
        lens.append(n)
    shape = (nb, bs, hkv, d)
    k_pool = np.zeros(shape, {"fp8": np.uint8, "int8": np.int8}.get(dt, np.uint16))
    v_pool = np.zeros_like(k_pool)
    k_new = configs._normal(70, 6, (len(slot_map), hkv, d), "bf16")
    v_new = configs._normal(70, 7, (len(slot_map), hkv, d), "bf16")
    top = {"fp8": 448.0, "int8": 127.0}.get(dt)
    scales = (np.full(hkv, 4.0 / top, np.float32), np.full(hkv, 4.0 / top, np.float32)) if top else (None, None)
    ks, vs = [None if x is None else to_dev(x, "f32") for x in scales]
    gk, gv = to_dev(k_pool, dt), to_dev(v_pool, dt)
    say("fork scenario", dt, "prompt write")
    pkv.kv_cache_write(to_dev(k_new, "bf16"), to_dev(v_new, "bf16"), gk, gv,
                       to_dev(np.array(slot_map, np.int32), "i32"), ks, vs)
    ok, ov = paged.kv_cache_write(k_new, v_new, k_pool, v_pool, np.array(slot_map), "bf16", dt, *scales)
    # fork every prompt: the child shares all of its blocks
    for i in range(len(prompts)):
        rows.append(bm.fork(rows[i], lens[i]))
        lens.append(lens[i])
    for step in range(3):
        copies, cur = [], []
        for i, row in enumerate(rows):
            slot, copy = bm.append_slot(row, lens[i])
            assert slot == paged.slot_of(row, lens[i], bs)
            if copy is not None:
                copies.append(copy)
        # copies only at the first step, one per sequence whose last block is
        # partial and shared (the later writer of a pair owns it by then)
        if step == 0:
            assert len(copies) == sum(1 for n in prompts if n % bs != 0)
        else:
            assert not copies
        table = np.array(rows, np.int32)
        b = len(rows)
        q = configs._normal(100 + step, 3, (b, hq, d), "bf16")
        kn = configs._normal(100 + step, 6, (b, hkv, d), "bf16")
        vn = configs._normal(100 + step, 7, (b, hkv, d), "bf16")
        say("fork scenario", dt, "step", step, "copies", len(copies))
        if copies:
            pkv.copy_blocks(gk, gv, to_dev(np.array(copies, np.int32), "i32"))
            ok, ov = blocks.copy_blocks(ok, ov, copies)
        got = out_f64(pkv.paged_decode_append(to_dev(q, "bf16"), to_dev(kn, "bf16"), to_dev(vn, "bf16"), gk, gv,
                                              to_dev(table, "i32"), to_dev(np.array(lens, np.int32), "i32"),
                                              0.088, ks, vs))
        want, ok, ov = paged.paged_decode_append(q, "bf16", kn, vn, ok, ov, dt, table, np.array(lens), 0.088,
                                                 *scales)
        assert_cache_equal(gk, ok, dt, f"k_cache step {step}")
        assert_cache_equal(gv, ov, dt, f"v_cache step {step}")
        err = max_err(got, want)
        print("fork scenario", dt, "step", step, "max|err|", err, flush=True)
        assert err <= TOL[dt]
        lens = [n + 1 for n in lens]
    # a parent and its child now differ in their last tokens but share every full prompt block
    for i, n in enumerate(prompts):
        shared = n // bs
        assert rows[i][:shared] == rows[len(prompts) + i][:shared]
        for blk in rows[i][:shared]:
            assert bm.refcount(blk) == 2
