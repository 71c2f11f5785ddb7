"""Seeded workload generators (CPU only)."""

import numpy as np

import workloads
from oracle import paged


def test_tiny_decode_is_the_page_example():
    s = workloads.config("tiny_decode")
    assert s.block_table.tolist() == workloads.configs.PAGE2_DECODE_TABLE
    assert list(s.slot_map) == [94, 32, 198]
    assert s.num_blocks == 8 and s.block_size == 32
    d = s.decode_inputs()
    assert list(d["cache_seqlens"]) == [31, 33, 71]
    assert s.q.shape == (3, 8, 64) and s.k_new.shape == (3, 2, 64)


def test_slot_map_agrees_with_oracle_slot_math():
    s = workloads.config("varlen_prefill_prefix", batch=5, q_hi=300, p_hi=90)
    t = 0
    for i in range(len(s.prefix)):
        for p in range(int(s.prefix[i]), int(s.total[i])):
            assert s.slot_map[t] == paged.slot_of(s.block_table[i], p, s.block_size)
            t += 1
    assert len(set(s.slot_map.tolist())) == len(s.slot_map)


def test_generation_is_deterministic():
    a = workloads.config("llama8b_decode", batch=4, len_lo=20, len_hi=70)
    b = workloads.config("llama8b_decode", batch=4, len_lo=20, len_hi=70)
    for name in ("k_cache", "v_cache", "q", "k_new", "v_new", "slot_map", "block_table"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name


def test_poison_marks_exactly_the_non_history_slots():
    s = workloads.config("llama8b_decode", batch=6, len_lo=1, len_hi=50)
    flat = s.k_cache.reshape(-1, s.num_kv_heads * s.head_dim)
    is_nan = flat[:, 0] == workloads.configs.BF16_NAN
    history = np.zeros(len(flat), bool)
    for i in range(len(s.prefix)):
        history[paged.gather_slots(s.block_table[i], int(s.prefix[i]), s.block_size)] = True
    assert np.array_equal(is_nan, ~history)
    assert np.all(is_nan[s.slot_map])


def test_pool_is_a_permutation_sized_to_fit():
    s = workloads.config("llama8b_decode", batch=7, len_lo=5, len_hi=100)
    used = s.block_table[s.block_table >= 0]
    assert sorted(used.tolist()) == list(range(s.num_blocks))
    for i in range(len(s.prefix)):
        assert int((s.block_table[i] >= 0).sum()) == paged.blocks_needed(int(s.total[i]), 16)


def test_mixed_step_layout():
    s = workloads.config("mixed_fp8", prefill_chunks=2, chunk=40, decode_batch=5, p_hi=100,
                         len_lo=3, len_hi=60)
    assert s.kinds == ["prefill"] * 2 + ["decode"] * 5
    assert s.num_tokens == 85
    assert s.k_cache.dtype == np.uint8 and s.k_scale.shape == (8,)
    p = s.prefill_inputs()
    assert list(p["cu_seqlens_q"]) == [0, 40, 80]
    d = s.decode_inputs()
    assert d["q"].shape == (5, 32, 128)
    assert np.array_equal(d["q"], s.q[80:85])
    # finite history codes only; poison is 0x7F
    flat = s.k_cache.reshape(-1, 8 * 128)
    assert not np.any(flat[flat[:, 0] != 0x7F] == 0xFF)


def test_page2_varlen_example_shapes():
    c = workloads.page2_varlen_example()
    assert list(c.cu_seqlens_q) == [0, 10, 13, 14] and list(c.cu_seqlens_k) == [0, 0, 1, 8]
    assert c.q.shape[0] == 14 and c.k.shape[0] == 8
