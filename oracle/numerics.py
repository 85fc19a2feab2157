"""Rounding and decoding helpers of the oracle (test infrastructure only).

bfloat16: 1 sign, 8 exponent, 7 stored mantissa bits (the upper half of an
IEEE binary32); rounding is to nearest, ties to even.  E4M3FN (OCP 8-bit
floating point specification): 1 sign, 4 exponent bits with bias 7, 3 mantissa
bits, no infinities, the all-ones pattern (S.1111.111) is NaN, largest finite
magnitude 448.

MXFP4 (OCP Microscaling Formats (MX) v1.0): blocks of 32 consecutive elements
share one E8M0 scale (an 8-bit biased exponent, bias 127, value 2^(e-127); the
all-ones code is NaN; no sign, no mantissa), and each element is an E2M1 code
(1 sign, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 holds
the subnormals 0 and 0.5; no infinities or NaN; largest magnitude 6).  The
element's value is its E2M1 value times the block scale.  Two codes share a
byte, the element with the even index in the low nibble (the format fixes
no byte packing; this is the reading taken).  This is the MI355X counterpart
of the 4-bit expert weights the pages name (DiffusionGemma深度拆解
(zhichai.net), "MoE 效率：128 专家，8 活跃").

MXFP8 activations (the same MX specification, its conversion of a block of
32 values to a scaled format): the shared exponent is floor(log2(max |v|))
minus the element format's largest exponent (8 for E4M3: 448 = 1.75 * 2^8),
kept in the E8M0 range [-127, 127]; an all-zero block takes code 0.  Each
element v / 2^shared is rounded to E4M3FN, to nearest with ties to even, and
magnitudes past 448 are clamped to 448 (the largest normal; the format has no
infinity).  Used for the routed gate/up inputs of the MXFP4 x MXFP8 variant.
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


def e2m1_table() -> np.ndarray:
    """float64 value of each of the 16 E2M1 codes."""
    out = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        exp = (code >> 1) & 0x3
        man = code & 0x1
        if exp == 0:
            out[code] = sign * (man / 2.0)                      # subnormal: 0 or 0.5
        else:
            out[code] = sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return out


_E2M1 = e2m1_table()


def decode_e8m0(codes) -> np.ndarray:
    """2^(e - 127) for each E8M0 code e; NaN for 255."""
    e = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).astype(np.int64)))


def unpack_fp4(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] E2M1 codes: byte j holds element 2j in its
    low nibble and element 2j + 1 in its high nibble."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def decode_mxfp4(packed, scales) -> np.ndarray:
    """MXFP4 rows [..., K/2] (packed codes) with scales [..., K/32] -> float64 [..., K]."""
    v = _E2M1[unpack_fp4(packed)]
    s = decode_e8m0(scales)
    return v * np.repeat(s, 32, axis=-1)


_E4M3_CODE = {float(v): c for c, v in enumerate(_E4M3[:127]) if np.isfinite(v)}   # non-negative finite values


def round_e4m3(y) -> np.ndarray:
    """Round float64 values to E4M3FN values: nearest, ties to even mantissa,
    magnitudes above 448 clamped to 448."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 448.0)
    _, e = np.frexp(a)                          # a = f 2^e, 0.5 <= f < 1: floor(log2 a) = e - 1
    step = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)   # 3 mantissa bits; subnormal spacing 2^-9
    return np.copysign(np.rint(a / step) * step, y)


def quantize_mxfp8(x):
    """float64 [..., K] (K % 32 == 0) -> (E4M3FN codes uint8 [..., K],
    E8M0 shared-exponent codes uint8 [..., K / 32])."""
    x = np.asarray(x, dtype=np.float64)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    _, e = np.frexp(amax)
    scode = np.where(amax > 0, np.clip(e - 1 - 8 + 127, 0, 254), 0).astype(np.int64)
    q = round_e4m3(blk * np.ldexp(1.0, 127 - scode)[..., None])
    mag = np.vectorize(_E4M3_CODE.__getitem__, otypes=[np.int64])(np.abs(q))
    codes = np.where(np.signbit(q), mag | 0x80, mag).astype(np.uint8)
    return codes.reshape(x.shape), scode.astype(np.uint8)


def decode_mxfp8(codes, scales) -> np.ndarray:
    """MXFP8 codes [..., K] with E8M0 scales [..., K/32] -> float64 [..., K]."""
    return decode_e4m3fn(codes) * np.repeat(decode_e8m0(scales), 32, axis=-1)


def round_mxfp8(x) -> np.ndarray:
    """The MXFP8 value of each element of x [..., K] (float64)."""
    return decode_mxfp8(*quantize_mxfp8(x))
