"""Oracle pins: bfloat16 rounding and E4M3FN decoding against torch's casts."""
import numpy as np
import torch

from oracle.numerics import decode_e4m3fn, round_bf16, round_fp32


def test_bf16_matches_torch_on_binary32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-30, 30, 200000),
        [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40, 1e-45, 65504.0],
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_ties_round_to_even():
    # 1 + 2**-8 lies halfway between 1 and 1 + 2**-7: even mantissa is 1.0.
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3 * 2**-8 lies halfway between 1 + 2**-7 and 1 + 2**-6: rounds up to even.
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert round_bf16(-(1.0 + 2.0 ** -8)) == -1.0
    # just above the midpoint rounds up.
    assert round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7


def test_bf16_overflow_and_nan():
    assert np.isinf(round_bf16(3.4e38))
    assert np.isnan(round_bf16(np.nan))
    assert round_bf16(np.inf) == np.inf


def test_fp32_rounding_is_binary32():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    np.testing.assert_array_equal(round_fp32(x), np.float32(x).astype(np.float64))


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])
    assert np.nanmax(got) == 448.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
