"""PKV_VALIDATE=1: each call copies its device metadata to the host and
rejects what would otherwise be unspecified (memory-safe) input, with
PKV_ERR_INVALID and no kernel launched.  These tests only ever launch
kernels on valid input."""

import os

import numpy as np
import pytest
import torch

import paged_kv_cache_map_amd as pkv
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def validate():
    old = os.environ.get("PKV_VALIDATE")
    os.environ["PKV_VALIDATE"] = "1"
    yield
    if old is None:
        del os.environ["PKV_VALIDATE"]
    else:
        os.environ["PKV_VALIDATE"] = old


def _pool(nb=8, bs=16, hkv=2, d=128):
    k = torch.zeros((nb, bs, hkv, d), dtype=torch.bfloat16, device="cuda")
    return k, torch.zeros_like(k)


def _rejects(fn):
    with pytest.raises(pkv.PkvError) as e:
        fn()
    assert e.value.code == pkv.ERR_INVALID
    torch.cuda.synchronize()


def test_write_rejects_duplicate_and_out_of_range_slots(validate):
    kc, vc = _pool()
    new = torch.ones((3, 2, 128), dtype=torch.bfloat16, device="cuda")
    _rejects(lambda: pkv.kv_cache_write(new, new, kc, vc, to_dev(np.array([5, 9, 5], np.int32), "i32")))
    _rejects(lambda: pkv.kv_cache_write(new, new, kc, vc, to_dev(np.array([5, 128, 6], np.int32), "i32")))
    assert int(kc.abs().sum().item()) == 0          # nothing was written
    pkv.kv_cache_write(new, new, kc, vc, to_dev(np.array([5, -1, 6], np.int32), "i32"))  # -1 skips
    torch.cuda.synchronize()
    assert int(kc.float().sum().item()) == 2 * 2 * 128


def test_decode_rejects_bad_block_ids(validate):
    kc, vc = _pool()
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    table = to_dev(np.array([[0, 1], [2, -1]], np.int32), "i32")
    _rejects(lambda: pkv.paged_decode(q, kc, vc, table, to_dev(np.array([20, 17], np.int32), "i32"), 0.1))
    _rejects(lambda: pkv.paged_decode(q, kc, vc, table, to_dev(np.array([33, 3], np.int32), "i32"), 0.1))
    out = pkv.paged_decode(q, kc, vc, table, to_dev(np.array([20, 16], np.int32), "i32"), 0.1)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_append_rejects_no_room_and_shared_slot(validate):
    kc, vc = _pool()
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    new = torch.ones((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    full = to_dev(np.array([[0, 1], [2, 3]], np.int32), "i32")
    _rejects(lambda: pkv.paged_decode_append(q, new, new, kc, vc, full, to_dev(np.array([32, 3], np.int32), "i32"),
                                             0.1))
    shared = to_dev(np.array([[4, 5], [4, 6]], np.int32), "i32")   # both append at block 4, offset 3
    _rejects(lambda: pkv.paged_decode_append(q, new, new, kc, vc, shared,
                                             to_dev(np.array([3, 3], np.int32), "i32"), 0.1))
    assert int(kc.abs().sum().item()) == 0


def test_copy_blocks_rejects_overlapping_pairs(validate):
    kc, vc = _pool()
    _rejects(lambda: pkv.copy_blocks(kc, vc, to_dev(np.array([[0, 1], [1, 2]], np.int32), "i32")))
    _rejects(lambda: pkv.copy_blocks(kc, vc, to_dev(np.array([[0, 3], [1, 3]], np.int32), "i32")))
    _rejects(lambda: pkv.copy_blocks(kc, vc, to_dev(np.array([[0, 8]], np.int32), "i32")))
    pkv.copy_blocks(kc, vc, to_dev(np.array([[0, 3], [0, 4]], np.int32), "i32"))
    torch.cuda.synchronize()


def test_prefill_rejects_bad_cu_seqlens(validate):
    q = torch.zeros((10, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((12, 2, 128), dtype=torch.bfloat16, device="cuda")
    cq = to_dev(np.array([0, 6, 4], np.int32), "i32")       # not monotone
    ck = to_dev(np.array([0, 6, 12], np.int32), "i32")
    _rejects(lambda: pkv.varlen_prefill(q, k, k, cq, ck, 6, 6, 0.1))
    cq = to_dev(np.array([0, 6, 10], np.int32), "i32")
    _rejects(lambda: pkv.varlen_prefill(q, k, k, cq, ck, 3, 6, 0.1))   # max_seqlen_q below the true 6
    pkv.varlen_prefill(q, k, k, cq, ck, 6, 6, 0.1)
    torch.cuda.synchronize()
