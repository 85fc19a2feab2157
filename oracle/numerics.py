"""Rounding helpers of the oracle (test infrastructure only).

bfloat16: 1 sign, 8 exponent, 7 stored mantissa bits (the upper half of an
IEEE binary32); rounding is to nearest, ties to even.  E4M3FN (OCP 8-bit
floating point specification): 1 sign, 4 exponent bits with bias 7, 3 mantissa
bits, no infinities, the all-ones pattern (S.1111.111) is NaN, largest finite
magnitude 448.
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = f * 2**e, 0.5 <= |f| < 1
    e = np.maximum(e, -125)                 # below 2**-126 the spacing stays 2**-133
    ulp = np.ldexp(1.0, e - 8)              # 8 significant bits
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(x / ulp) * ulp          # np.rint rounds half to even
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def round_fp32(x) -> np.ndarray:
    """Round float64 values to the nearest binary32, returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3FN codes (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            out[code] = np.nan
        elif exp == 0:
            out[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            out[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return out


_E4M3 = e4m3fn_table()


def decode_e4m3fn(codes) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]
