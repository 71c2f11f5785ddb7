"""INT8 KV-cache codec, written from its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[ch15] "KV cache / batching / paged attention", section "KVキャッシュはどれく
らいメモリを食う？": an INT8 (or FP8) cache takes exactly half the memory of a
16-bit one.  The pages fix no encoding; the reading used here is the plain
symmetric one: one fp32 scale per KV head, stored code = the fp32 quotient
x / scale rounded to the nearest integer (ties to even) and saturated to
[-127, 127], NaN stored as 0; value = code x scale.
"""

import numpy as np


def encode(quotient) -> np.ndarray:
    """int8 codes of fp32 quotients x / scale."""
    q = np.asarray(quotient, dtype=np.float32).astype(np.float64)
    codes = np.zeros(q.shape, dtype=np.int64)
    finite = ~np.isnan(q)
    # round half to even on the exact float64 value of each fp32 quotient
    codes[finite] = np.clip(np.rint(q[finite]), -127, 127).astype(np.int64)
    return codes.astype(np.int8)


def decode(codes) -> np.ndarray:
    """Exact float64 value of int8 codes (before the scale)."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64)
