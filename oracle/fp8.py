"""OCP FP8 E4M3 encoding of the cache, float64.  Test infrastructure only.

Source: the pages put an FP8 KV cache on the roadmap ([REPO] future work; [WT] trade-offs), with
no format given.  Reading: OCP 8-bit float E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
bits; subnormals; no infinities; S.1111.111 is NaN, so the largest finite value is 448), written
with round-to-nearest-even and saturation to +-448, the sign of zero kept.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0


def decode_code(c: int) -> float:
    """Value of code c in [0, 256)."""
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return float("nan")
    v = np.ldexp(m / 8.0, -6) if e == 0 else np.ldexp(1.0 + m / 8.0, e - 7)
    return -v if s else v


_POS = np.array([decode_code(c) for c in range(0x7F)])          # codes 0x00..0x7e, increasing


def encode(x) -> np.ndarray:
    """float array -> uint8 codes: nearest finite value, ties to the even code, |x| >= 448 -> 448."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), MAX)
    hi = np.minimum(np.searchsorted(_POS, a), len(_POS) - 1)    # first finite value >= |x|
    lo = np.maximum(hi - 1, 0)                                  # the one below it
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    even = np.where(lo % 2 == 0, lo, hi)                        # neighbouring codes: one is even
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, even)).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


_TABLE = None


def decode(codes) -> np.ndarray:
    global _TABLE
    if _TABLE is None:
        _TABLE = np.array([decode_code(c) for c in range(256)])
    return _TABLE[np.asarray(codes, np.uint8)]


def round_fp8(x) -> np.ndarray:
    """x rounded to the e4m3 values (float64)."""
    return decode(encode(x))
