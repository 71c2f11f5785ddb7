"""The oracle against its pins (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle_pins as pins
from oracle import e4m3, int8, kvsize, paged

# ---------------------------------------------------------------------------
# fp8 E4M3 codec
# ---------------------------------------------------------------------------

TABLE = e4m3.decode_table()


def test_e4m3_spot_values():
    # format definition: bias 7, 3 mantissa bits, subnormals m/8 * 2**-6, max 448
    assert TABLE[0x7E] == 448.0 and TABLE[0xFE] == -448.0
    assert TABLE[0x08] == 2.0 ** -6
    assert TABLE[0x01] == 2.0 ** -9
    assert TABLE[0x07] == 7 * 2.0 ** -9
    assert TABLE[0x38] == 1.0
    assert TABLE[0x40] == 2.0 and TABLE[0x3C] == 1.5
    assert TABLE[0x00] == 0.0 and np.signbit(TABLE[0x80])
    assert np.isnan(TABLE[0x7F]) and np.isnan(TABLE[0xFF])
    assert np.sum(np.isnan(TABLE)) == 2


def test_e4m3_monotone_and_symmetric():
    pos = TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(TABLE[0x80:0xFF], -pos)


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(e4m3.encode(TABLE[codes]), codes)
    assert np.array_equal(e4m3.encode_fast(TABLE[codes]), codes)


def test_e4m3_midpoints_round_to_even():
    for c in range(0x7E):
        lo, hi = TABLE[c], TABLE[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert e4m3.encode(mid) == even, hex(c)
        assert e4m3.encode(-mid) == (even | 0x80)
        assert e4m3.encode(np.nextafter(mid, -np.inf)) == c
        assert e4m3.encode(np.nextafter(mid, np.inf)) == c + 1


def test_e4m3_saturation_and_specials():
    # saturation is a reading of the pages (see the codec's header)
    assert e4m3.encode(448.0) == 0x7E
    assert e4m3.encode(464.0) == 0x7E
    assert e4m3.encode(1e30) == 0x7E
    assert e4m3.encode(np.inf) == 0x7E and e4m3.encode(-np.inf) == 0xFE
    assert e4m3.encode(np.nan) == 0x7F
    assert e4m3.encode(2.0 ** -10) == 0x00          # tie between 0 and 2**-9 -> even
    assert e4m3.encode(2.0 ** -10 * 1.0001) == 0x01
    assert e4m3.encode(-(2.0 ** -11)) == 0x80


def test_e4m3_matches_torch_in_range():
    """Library cross-check: torch's float8_e4m3fn conversion (round to nearest
    even) agrees with the oracle codec for every in-range float32 tried."""
    rng = np.random.default_rng(0)
    vals = [rng.standard_normal(200_000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)]
    mids = [(TABLE[c] + TABLE[c + 1]) / 2 for c in range(0x7E)]
    x = np.concatenate(vals + [np.array(mids), -np.array(mids), TABLE[:0x7F]])
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode_fast(x), ref)


def test_e4m3_fast_equals_plain():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(3000) * s for s in (1e-3, 1.0, 100.0, 1e3)] +
                       [np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 448.0, 449.0, 2.0 ** -10])])
    x = x.astype(np.float32)
    assert np.array_equal(e4m3.encode_fast(x), e4m3.encode(x))


# ---------------------------------------------------------------------------
# closed forms printed on the KV-size page
# ---------------------------------------------------------------------------


def test_kv_size_closed_forms():
    g = pins.load_golden("kv_size_closed_forms.json")
    for c in g["cases"]:
        got = kvsize.kv_bytes_total(c["layers"], c["kv_heads"], c["head_dim"], c["bytes"],
                                    c["tokens"], c["requests"])
        # every printed figure, including the ones given as "about", is exact here
        assert got == c["printed_bytes"], c["what"]
    per16 = kvsize.kv_bytes_per_token(32, 8, 128, 2)
    assert kvsize.kv_bytes_per_token(32, 8, 128, 1) * 2 == per16
    assert kvsize.kv_bytes_per_token(32, 32, 128, 2) == 4 * per16
    m = g["mla"]
    mla = kvsize.mla_bytes_per_token(m["layers"], m["latent"], m["rope"], m["bytes"])
    assert abs(mla / 1024 - m["printed_kib_approx"]) < 1.0
    # one layer of the 8B shape, as the decode workloads move it
    assert kvsize.layer_bytes_per_token(8, 128, 2) == 4096


# ---------------------------------------------------------------------------
# index bookkeeping, write, gather, attention
# ---------------------------------------------------------------------------


def test_varlen_example_indexing():
    pins.check_varlen_example(paged)


def test_decode_example_slots():
    pins.check_decode_example(paged)


def test_write_example():
    pins.check_write_example(paged)


def test_dense_causal_square():
    pins.check_dense_causal_square(paged)


def test_dense_noncausal():
    pins.check_dense_noncausal(paged)


def test_prefix_alignment():
    pins.check_prefix_alignment(paged)


def test_varlen_example_outputs():
    pins.check_varlen_example_outputs(paged)


def test_equal_keys_mean():
    pins.check_equal_keys_mean(paged)


def test_paged_decode_matches_dense():
    pins.check_paged_decode_matches_dense(paged)


def test_paged_prefill_matches_contig():
    pins.check_paged_prefill_matches_contig(paged)


def test_decode_is_varlen_with_one_query():
    pins.check_decode_is_varlen_with_one_query(paged)


def test_append_example():
    pins.check_append_example(paged)


def test_append_to_empty_sequence():
    pins.check_append_to_empty_sequence(paged)


def test_write_skip_and_errors():
    kc = np.zeros((2, 4, 1, 8), np.float32)
    vc = np.zeros((2, 4, 1, 8), np.float32)
    k = np.arange(3 * 8, dtype=np.float32).reshape(3, 1, 8) + 1
    v = -k
    k2, v2 = paged.kv_cache_write(k, v, kc, vc, np.array([5, -1, 0], np.int32), "f32", "f32")
    assert np.array_equal(k2.reshape(8, 1, 8)[5], k[0]) and np.array_equal(k2.reshape(8, 1, 8)[0], k[2])
    assert np.count_nonzero(k2) == 16 and np.count_nonzero(v2) == 16
    with pytest.raises(ValueError):
        paged.kv_cache_write(k, v, kc, vc, np.array([1, 1, 2], np.int32), "f32", "f32")
    with pytest.raises(ValueError):
        paged.kv_cache_write(k, v, kc, vc, np.array([0, 8, 2], np.int32), "f32", "f32")


def test_write_fp8_matches_library_quantisation():
    """bf16 -> fp8 write: code = e4m3(fp32(x) / fp32(scale)); cross-checked with
    torch's fp32 division and float8_e4m3fn conversion (values stay in range)."""
    rng = np.random.default_rng(3)
    t, hkv, d = 5, 3, 16
    x = rng.standard_normal((t, hkv, d)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)        # truncation: any bf16 will do
    scale = np.array([0.01, 0.0123, 0.5], np.float32)
    kc = np.zeros((2, 4, hkv, d), np.uint8)
    k2, _ = paged.kv_cache_write(bits, bits, kc, kc, np.arange(t, dtype=np.int32), "bf16", "fp8",
                                 scale, scale)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    ref = (xt / torch.from_numpy(scale)[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(k2.reshape(8, hkv, d)[:t], ref)


def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80], np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(paged.to_f64(bits, "bf16"), want)


def test_fp8_dequant_uses_head_scale():
    codes = np.array([[[0x38, 0x40]], [[0xB8, 0x01]]], np.uint8)    # [2 rows, 1 head, 2]
    got = paged.to_f64(codes, "fp8", np.array([0.25], np.float32))
    assert np.array_equal(got, np.array([[[0.25, 0.5]], [[-0.25, 2.0 ** -11]]]))


def test_empty_sequences():
    q = np.ones((1, 2, 4), np.float32)
    kc = np.full((1, 4, 1, 4), np.nan, np.float32)
    out = paged.paged_decode(q, "f32", kc, kc, "f32", np.array([[-1]], np.int32),
                             np.array([0], np.int32), 1.0)
    assert np.all(out == 0.0)


def test_mqa_and_mha_special_cases():
    """G = Hq (one KV head) and G = 1 both agree with the library routine."""
    rng = np.random.default_rng(5)
    for hq, hkv in [(8, 1), (4, 4)]:
        q = rng.standard_normal((6, hq, 16))
        k = rng.standard_normal((6, hkv, 16))
        v = rng.standard_normal((6, hkv, 16))
        np.testing.assert_allclose(paged.attention(q, k, v, 0.25, True),
                                   pins._sdpa(q, k, v, 0.25, True), rtol=1e-12, atol=1e-12)


def test_scale_is_applied_before_softmax():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((5, 1, 8))
    v = rng.standard_normal((5, 1, 8))
    a = paged.attention(q, k, v, 2.0, False)
    b = paged.attention(2.0 * q, k, v, 1.0, False)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    assert not np.allclose(a, paged.attention(q, k, v, 1.0, False))
    np.testing.assert_allclose(a, pins._sdpa(q, k, v, 2.0, False), rtol=1e-12)
    assert math.isfinite(float(a.sum()))


def test_row_subset_equals_full_computation():
    """Computing selected query rows gives exactly those rows of the full result."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((5 + 9, 4, 8)).astype(np.float32)
    k = rng.standard_normal((7 + 20, 2, 8)).astype(np.float32)
    v = rng.standard_normal((7 + 20, 2, 8)).astype(np.float32)
    cu_q, cu_k = paged.cu_seqlens([5, 9]), paged.cu_seqlens([7, 20])
    full = paged.varlen_prefill(q, "f32", k, v, "f32", cu_q, cu_k, 0.4, True)
    rows = [0, 3, 6, 13]
    part = paged.varlen_prefill(q, "f32", k, v, "f32", cu_q, cu_k, 0.4, True, rows=rows)
    np.testing.assert_array_equal(part[rows], full[rows])
    assert np.all(np.delete(part, rows, axis=0) == 0)


def test_int8_codec_pins():
    for check in pins.int8_checks(int8):
        check(int8)


def test_int8_write_and_decode_use_the_head_scale():
    """An int8 cache stores RNE(x / scale[h]) saturated to 127; decoding gives
    code x scale[h]."""
    k = np.array([[[1.0, -2.0, 3.06, 1000.0]], [[0.5, 0.25, -0.75, 0.0]]], np.float32)  # [2, 1, 4]
    v = -k
    kc = np.zeros((1, 2, 1, 4), np.int8)
    scale = np.array([0.02], np.float32)
    k2, v2 = paged.kv_cache_write(k, v, kc, kc.copy(), np.array([1, 0]), "f32", "int8", scale, scale)
    assert k2[0, 1, 0].tolist() == [50, -100, 127, 127]       # 3.06 / 0.02 = 153 -> 127
    assert k2[0, 0, 0].tolist() == [25, 12, -38, 0]           # 0.25 / 0.02 = 12.5 -> 12 (even)
    assert v2[0, 1, 0].tolist() == [-50, 100, -127, -127]
    vals = paged.to_f64(k2[0], "int8", scale)
    assert vals[1, 0].tolist() == [50 * np.float64(np.float32(0.02)), -100 * np.float64(np.float32(0.02)),
                                   127 * np.float64(np.float32(0.02)), 127 * np.float64(np.float32(0.02))]
