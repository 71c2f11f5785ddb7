"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each case copies the oracle's source, changes one expression the way a
plausible bug would (a dropped term, a wrong index, a transposed operand, a
wrong mask alignment ...), loads the copy as a throw-away module and runs the
pins against it.  The real oracle is never modified.
"""

import importlib.util
import pathlib

import numpy as np
import pytest

import oracle_pins as pins

ORACLE = pathlib.Path(__file__).resolve().parent.parent / "oracle"

PAGED_CHECKS = [
    pins.check_varlen_example, pins.check_decode_example, pins.check_write_example,
    pins.check_dense_causal_square, pins.check_dense_noncausal, pins.check_prefix_alignment,
    pins.check_varlen_example_outputs, pins.check_equal_keys_mean,
    pins.check_paged_decode_matches_dense, pins.check_paged_prefill_matches_contig,
    pins.check_decode_is_varlen_with_one_query, pins.check_append_example,
    pins.check_append_to_empty_sequence,
]

# (name, original text, planted text)
PAGED_MUTATIONS = [
    ("gqa_modulo", "g = h // group", "g = h % hkv"),
    ("causal_top_left", "visible = cols <= rows + (lk - chunk)", "visible = cols <= rows"),
    ("causal_strict", "visible = cols <= rows + (lk - chunk)", "visible = cols < rows + (lk - chunk)"),
    ("scale_dropped", "logits = scale * (q[:, h, :] @ k[:, g, :].T)",
     "logits = (q[:, h, :] @ k[:, g, :].T)"),
    ("scale_after_softmax", "logits = scale * (q[:, h, :] @ k[:, g, :].T)",
     "logits = (q[:, h, :] @ k[:, g, :].T) / scale"),
    ("denominator_wrong_axis", "denom = weights.sum(axis=1)", "denom = weights.sum(axis=0)"),
    ("denominator_dropped", "numer / np.where(has_key, denom, 1.0)[:, None]", "numer"),
    ("v_from_k", "numer = weights @ v[:, g, :]", "numer = weights @ k[:, g, :]"),
    ("slot_offset_swapped", "return blocks * block_size + j % block_size",
     "return blocks * block_size + j // block_size"),
    ("slot_no_table", "blocks = np.asarray(block_table_row, dtype=np.int64)[j // block_size]",
     "blocks = j // block_size"),
    ("slot_of_wrong", "return block * block_size + pos % block_size", "return block + pos % block_size"),
    ("cu_no_leading_zero", "return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)",
     "return np.cumsum(lengths).astype(np.int32)"),
    ("request_index_off_by_one", "owner[cu[b]:cu[b + 1]] = b", "owner[cu[b]:cu[b + 1]] = b + 1"),
    ("blocks_needed_floor", "return -(-int(num_tokens) // int(block_size))",
     "return int(num_tokens) // int(block_size)"),
    ("write_k_to_v", "v_out[s] = _store_row(v[t], src_dtype, cache_dtype, v_scale)",
     "v_out[s] = _store_row(k[t], src_dtype, cache_dtype, v_scale)"),
    ("write_wrong_slot", "k_out[s] = _store_row(k[t], src_dtype, cache_dtype, k_scale)",
     "k_out[(s + 1) % num_slots] = _store_row(k[t], src_dtype, cache_dtype, k_scale)"),
    ("varlen_keys_from_q_offsets", "k_rows = k[cu_k[b]:cu_k[b + 1]]", "k_rows = k[cu_q[b]:cu_q[b] + lk]"),
    ("prefill_wrong_table_row", "k_rows = gather(k, block_table[b], lk)",
     "k_rows = gather(k, block_table[0], lk)"),
    ("decode_drops_last_key", "lk = int(cache_seqlens[b])", "lk = int(cache_seqlens[b]) - 1"),
    ("append_after_last_key", "slots = np.array([slot_of(block_table[b], int(lens[b]), bs)",
     "slots = np.array([slot_of(block_table[b], int(lens[b]) - 1, bs)"),
    ("append_not_attended", "out = paged_decode(q, q_dtype, kc, vc, cache_dtype, block_table, lens + 1,",
     "out = paged_decode(q, q_dtype, kc, vc, cache_dtype, block_table, lens,"),
    ("empty_row_not_zero", "out[:, h, :] = np.where(has_key[:, None], numer / np.where(has_key, denom, 1.0)[:, None], 0.0)",
     "out[:, h, :] = numer / np.where(has_key, denom, 1.0)[:, None] + np.where(has_key, 0.0, 1.0)[:, None]"),
]


def _load_mutant(filename, original, planted):
    src = (ORACLE / filename).read_text()
    assert src.count(original) >= 1, f"mutation anchor not found: {original!r}"
    src = src.replace(original, planted)
    spec = importlib.util.spec_from_loader(f"oracle._mutant_{filename[:-3]}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(src, str(ORACLE / filename), "exec"), mod.__dict__)
    return mod


def _some_check_fails(mod, checks):
    for check in checks:
        try:
            with np.errstate(all="ignore"):
                check(mod)
        except Exception:   # an assertion, or a crash the mistake causes
            return True
    return False


def test_real_oracle_passes_every_check():
    from oracle import paged
    assert not _some_check_fails(paged, PAGED_CHECKS)


@pytest.mark.parametrize("name,original,planted", PAGED_MUTATIONS, ids=[m[0] for m in PAGED_MUTATIONS])
def test_planted_mistake_is_caught(name, original, planted):
    mod = _load_mutant("paged.py", original, planted)
    assert _some_check_fails(mod, PAGED_CHECKS), f"mutation {name} survived every pin"


E4M3_MUTATIONS = [
    ("bias_8", "2.0 ** (exp_field - 7)", "2.0 ** (exp_field - 8)"),
    ("subnormal_scale", "(mant / 8.0) * 2.0 ** (1 - 7)", "(mant / 8.0) * 2.0 ** (0 - 7)"),
    ("round_half_up", "rounded = float(np.rint(mag / quantum)) * quantum",
     "rounded = float(np.floor(mag / quantum + 0.5)) * quantum"),
    ("truncate", "rounded = float(np.rint(mag / quantum)) * quantum",
     "rounded = float(np.floor(mag / quantum)) * quantum"),
    ("binade_off", "binade = max(int(exp2) - 1, -6)", "binade = max(int(exp2), -6)"),
    ("no_subnormal_floor", "binade = max(int(exp2) - 1, -6)", "binade = int(exp2) - 1"),
    ("nan_code", "table[code] = np.nan", "table[code] = 480.0"),
]


def _e4m3_checks(mod):
    """The codec pins of test_oracle.py, parametrised by module."""
    import torch
    table = mod.decode_table()

    def spot():
        assert table[0x7E] == 448.0 and table[0x08] == 2.0 ** -6 and table[0x01] == 2.0 ** -9
        assert table[0x38] == 1.0 and np.isnan(table[0x7F])

    def midpoints():
        for c in range(0x7E):
            mid = (table[c] + table[c + 1]) / 2
            assert mod.encode(mid) == (c if c % 2 == 0 else c + 1)

    def library():
        rng = np.random.default_rng(0)
        x = np.concatenate([rng.standard_normal(2000) * s for s in (1e-3, 1.0, 100.0)]).astype(np.float32)
        x = x[np.abs(x) <= 448]
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(mod.encode(x), ref)

    return [lambda _m: spot(), lambda _m: midpoints(), lambda _m: library()]


def test_real_codec_passes():
    from oracle import e4m3
    assert not _some_check_fails(e4m3, _e4m3_checks(e4m3))


@pytest.mark.parametrize("name,original,planted", E4M3_MUTATIONS, ids=[m[0] for m in E4M3_MUTATIONS])
def test_planted_codec_mistake_is_caught(name, original, planted):
    mod = _load_mutant("e4m3.py", original, planted)
    assert _some_check_fails(mod, _e4m3_checks(mod)), f"mutation {name} survived every pin"


INT8_MUTATIONS = [
    ("round_half_away", "codes[finite] = np.clip(np.rint(q[finite]), -127, 127).astype(np.int64)",
     "codes[finite] = np.clip(np.sign(q[finite]) * np.floor(np.abs(q[finite]) + 0.5), -127, 127).astype(np.int64)"),
    ("asymmetric_range", "codes[finite] = np.clip(np.rint(q[finite]), -127, 127).astype(np.int64)",
     "codes[finite] = np.clip(np.rint(q[finite]), -128, 127).astype(np.int64)"),
    ("truncate", "codes[finite] = np.clip(np.rint(q[finite]), -127, 127).astype(np.int64)",
     "codes[finite] = np.clip(np.trunc(q[finite]), -127, 127).astype(np.int64)"),
    ("no_saturation", "codes[finite] = np.clip(np.rint(q[finite]), -127, 127).astype(np.int64)",
     "codes[finite] = np.rint(q[finite]).astype(np.int64)"),
    ("decode_unsigned", "return np.asarray(codes, dtype=np.int8).astype(np.float64)",
     "return np.asarray(codes, dtype=np.int8).view(np.uint8).astype(np.float64)"),
]


def test_real_int8_codec_passes():
    from oracle import int8
    assert not _some_check_fails(int8, pins.int8_checks(int8))


@pytest.mark.parametrize("name,original,planted", INT8_MUTATIONS, ids=[m[0] for m in INT8_MUTATIONS])
def test_planted_int8_mistake_is_caught(name, original, planted):
    mod = _load_mutant("int8.py", original, planted)
    assert _some_check_fails(mod, pins.int8_checks(mod)), f"mutation {name} survived every pin"
