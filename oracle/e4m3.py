"""OCP 8-bit floating point, E4M3 ("FN": finite-only) codec in plain numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages say only that an FP8 (or INT8) KV cache takes exactly half the
memory of a 16-bit one ([ch15] "KV cache / batching / paged attention",
section "KVキャッシュはどれくらいメモリを食う？"; [glossary] "KVキャッシュとは",
section 比較 names cache quantisation).  They fix no format.  The reading
taken here is the OCP OFP8 E4M3 format, the fp8 type gfx950 computes with:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 holds subnormals m/8 * 2**-6;
* no infinities; S.1111.111 is NaN; the largest finite magnitude is 448.

Encoding (reading, not printed on the pages): round to nearest, ties to an
even mantissa, saturate to +-448 (including +-inf), NaN -> 0x7F.
"""

import numpy as np

NAN_CODE = 0x7F
MAX_FINITE = 448.0


def decode_table() -> np.ndarray:
    """Float64 value of each of the 256 codes; NaN at 0x7F and 0xFF.

    Written out from the field layout above, one code at a time.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = np.nan
        elif exp_field == 0:
            table[code] = sign * (mant / 8.0) * 2.0 ** (1 - 7)
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


_TABLE = decode_table()
# magnitude -> code, over the 127 finite non-negative codes 0x00..0x7E
_MAG_TO_CODE = {float(_TABLE[c]): c for c in range(0x7F)}


def decode(codes: np.ndarray) -> np.ndarray:
    """Codes (uint8) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x) -> np.ndarray:
    """Float values (taken exactly, as float64) -> uint8 codes.

    Each magnitude is written as q * quantum, where quantum is the spacing of
    e4m3 values in the binade of |x| (2**(e-3) for a normal binade 2**e with
    e >= -6, and 2**-9 below 2**-6); q is rounded to the nearest integer with
    ties to even (numpy.rint), which for e4m3 is ties to an even mantissa.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, value in enumerate(flat):
        out[i] = _encode_one(float(value))
    return out.reshape(x.shape)


def _encode_one(value: float) -> int:
    if np.isnan(value):
        return NAN_CODE
    sign = 0x80 if np.signbit(value) else 0x00
    mag = abs(value)
    if mag >= MAX_FINITE:
        return sign | _MAG_TO_CODE[MAX_FINITE]
    if mag == 0.0:
        return sign
    _, exp2 = np.frexp(mag)          # mag = f * 2**exp2, 0.5 <= f < 1
    binade = max(int(exp2) - 1, -6)  # mag lies in [2**binade, 2**(binade+1))
    quantum = 2.0 ** (binade - 3)
    rounded = float(np.rint(mag / quantum)) * quantum
    if rounded >= MAX_FINITE:
        rounded = MAX_FINITE
    return sign | _MAG_TO_CODE[rounded]


def encode_fast(x) -> np.ndarray:
    """Vectorised twin of :func:`encode` for large arrays (same arithmetic).

    Used by the bounded CPU timing and by whole-cache oracle writes; the pin
    tests compare it with :func:`encode` code for code.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, exp2 = np.frexp(np.where(mag > 0, mag, 1.0))
    binade = np.maximum(exp2.astype(np.int64) - 1, -6)
    quantum = np.exp2((binade - 3).astype(np.float64))
    rounded = np.rint(mag / quantum) * quantum
    rounded = np.where(np.isfinite(mag), np.minimum(rounded, MAX_FINITE), MAX_FINITE)
    rounded = np.where(mag == 0, 0.0, rounded)
    finite_vals = _TABLE[:0x7F]
    mag_code = np.searchsorted(finite_vals, rounded).astype(np.uint8)
    if not np.array_equal(finite_vals[mag_code], rounded):
        raise AssertionError("e4m3 encode produced a value that is not a code")
    codes = mag_code | np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(NAN_CODE), codes).astype(np.uint8)
