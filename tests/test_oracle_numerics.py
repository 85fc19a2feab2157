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


# ----------------------------------------------------------------------------- MXFP4 (OCP MX v1.0)

def test_e2m1_codes_are_the_spec_values():
    """The E2M1 element table the OCP MX specification prints: magnitudes 0,
    0.5 (the one subnormal), 1 (smallest normal), 1.5, 2, 3, 4, 6 (largest
    normal) for codes 0..7, and the same negated with the sign bit set."""
    from oracle.numerics import e2m1_table
    t = e2m1_table()
    np.testing.assert_array_equal(t[:8], [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    np.testing.assert_array_equal(t[8:], -t[:8])
    assert np.signbit(t[8]) and not np.signbit(t[0])
    # every E2M1 value is exactly an E4M3FN value (2 significant bits, exponents -1..2)
    e4 = torch.from_numpy(t).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(e4, t)


def test_e8m0_all_codes_match_torch():
    from oracle.numerics import decode_e8m0
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_mxfp4_nibble_order_and_block_scale():
    """Byte 0x21 holds element 0 (code 1 = 0.5) in its low nibble and element 1
    (code 2 = 1.0) in its high nibble; a row of 64 elements has two scales."""
    from oracle.numerics import decode_mxfp4
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x21
    packed[0, 16] = 0xF7          # element 32: 6.0, element 33: -6.0
    scales = np.array([[127 + 3, 127 - 2]], dtype=np.uint8)
    v = decode_mxfp4(packed, scales)
    assert v.shape == (1, 64)
    assert v[0, 0] == 0.5 * 8 and v[0, 1] == 1.0 * 8 and not v[0, 2:32].any()
    assert v[0, 32] == 6.0 / 4 and v[0, 33] == -6.0 / 4 and not v[0, 34:].any()


def test_mxfp4_quantize_then_decode():
    """The generator's quantizer and the oracle's decoder agree on the format:
    values already on the grid come back exactly; a random weight comes back
    within half an E2M1 step (at most 2^e, e its block's exponent) when
    |w| <= 6 * 2^e, and saturated to 6 * 2^e above that (the block maximum
    maps into [4, 8) * 2^e); all-zero blocks stay zero."""
    from oracle.numerics import decode_mxfp4
    from workloads.gen import quantize_mxfp4_rows
    rng = np.random.default_rng(7)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    exact = rng.choice(grid, (8, 64)) * rng.choice([1.0, -1.0], (8, 64))
    exact[:, ::32] = 6.0                               # sets each block's scale to 2^0
    exact *= 2.0 ** rng.integers(-20, 5, (8, 1))       # a power of two per row
    q, s = quantize_mxfp4_rows(torch.from_numpy(exact).float())
    np.testing.assert_array_equal(decode_mxfp4(q.numpy(), s.numpy()), exact)
    w = rng.standard_normal((16, 2048)) * 0.02
    w[3, 64:96] = 0.0
    q, s = quantize_mxfp4_rows(torch.from_numpy(w).float())
    dq = decode_mxfp4(q.numpy(), s.numpy())
    step = np.repeat(2.0 ** (s.numpy().astype(np.float64) - 127), 32, axis=-1)
    w32 = w.astype(np.float32).astype(np.float64)
    over = np.abs(w32) > 6 * step
    bound = np.where(over, np.abs(w32) - 6 * step, step)
    assert np.all(np.abs(dq - w32) <= bound * (1 + 1e-6))
    np.testing.assert_array_equal(np.abs(dq[over]), 6 * step[over])
    assert over.any()
    assert not dq[3, 64:96].any() and s.numpy()[3, 2] == 0
    # the largest element of every nonzero block uses the top binade (|code value| >= 4)
    blocks = np.abs(dq).reshape(16, 64, 32).max(-1) / 2.0 ** (s.numpy().astype(np.float64) - 127)
    assert np.all((blocks[s.numpy() > 0] >= 4.0))


# ----------------------------------------------------------------------------- MXFP8 activations

def _e4m3_nearest_brute_force(y: float) -> float:
    """Nearest finite E4M3FN value to y clamped to +-448, by a scan of the 254
    finite codes; on a tie the code with the even mantissa (low bit 0)."""
    from oracle.numerics import e4m3fn_table
    t = e4m3fn_table()
    yc = min(max(y, -448.0), 448.0)
    best = None
    for code in range(256):
        v = t[code]
        if not np.isfinite(v) or (code & 0x80) != (0x80 if np.signbit(yc) else 0):
            continue
        d = abs(v - yc)
        key = (d, code & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def test_e4m3_rounding_matches_a_scan_of_the_code_table():
    """Every bfloat16 value in [-600, 600] (and the tiny ones around the
    subnormal grid) rounds to the nearest E4M3FN value, ties to the even
    mantissa, clamped at 448."""
    from oracle.numerics import round_e4m3
    bits = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    f32 = bits.view(np.float32)
    ys = f32[np.isfinite(f32)].astype(np.float64)          # NaN patterns dropped before widening
    ys = ys[(np.abs(ys) <= 600) & ((np.abs(ys) >= 2.0 ** -12) | (ys == 0))]
    ys = ys[:: max(1, ys.size // 6000)]        # about 6000 values spread over the range
    got = round_e4m3(ys)
    ref = np.array([_e4m3_nearest_brute_force(float(y)) for y in ys])
    np.testing.assert_array_equal(got, ref)


def test_e4m3_rounding_ties_subnormals_and_saturation():
    from oracle.numerics import round_e4m3
    # halfway cases go to the even mantissa: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25
    assert round_e4m3(1.0625) == 1.0 and round_e4m3(1.1875) == 1.25
    # subnormal grid 2^-9: 2^-10 is a tie between 0 and 2^-9 (to 0); 1.5 * 2^-10 rounds up
    assert round_e4m3(2.0 ** -10) == 0.0 and round_e4m3(1.5 * 2.0 ** -10) == 2.0 ** -9
    # 448 is the largest finite value; beyond it the value is clamped
    assert round_e4m3(460.0) == 448.0 and round_e4m3(-511.0) == -448.0
    assert np.signbit(round_e4m3(-1e-9)) and round_e4m3(-1e-9) == 0.0


def test_e4m3_rounding_matches_torch_inside_the_range():
    """torch's float8_e4m3fn cast (round to nearest even) on values within
    +-448, a library cross-check of the same rounding."""
    from oracle.numerics import round_e4m3
    g = np.random.default_rng(7)
    y = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0)])
    y = np.clip(y, -448.0, 448.0).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_e4m3(y), ref)


def test_mxfp8_block_scale_is_the_largest_exponent_less_eight():
    """The shared exponent of a block is floor(log2(max |v|)) - 8, so the
    largest element lands in [256, 512) before rounding: 2^k maps to 256
    exactly, 1.9 * 2^k to 486.4, clamped to 448; an all-zero block takes
    code 0; each block of 32 gets its own scale."""
    from oracle.numerics import quantize_mxfp8, decode_mxfp8, decode_e4m3fn
    x = np.zeros((2, 64))
    x[0, 5] = 2.0 ** 3
    x[0, 40] = -1.9 * 2.0 ** -2
    x[0, 41] = 2.0 ** -2
    codes, scales = quantize_mxfp8(x)
    assert scales.tolist() == [[127 + 3 - 8, 127 - 2 - 8], [0, 0]]
    assert decode_e4m3fn(codes[0, 5]) == 256.0
    assert decode_e4m3fn(codes[0, 40]) == -448.0 and decode_e4m3fn(codes[0, 41]) == 256.0
    assert not codes[1].any()
    v = decode_mxfp8(codes, scales)
    assert v[0, 5] == 8.0 and v[0, 40] == -448.0 * 2.0 ** -10 and v[0, 41] == 0.25


def test_mxfp8_round_trip_and_error_bound():
    """Values on a block's grid come back exactly; random bfloat16 rows come
    back within half a step of the E4M3 grid: at most 2^-4 of the scaled
    element from 2^-6 to 448, an absolute 2^-10 of the scale below 2^-6, and
    the clamp to 448 above it (the block's largest element can map to
    [448, 512))."""
    from oracle.numerics import quantize_mxfp8, decode_mxfp8, round_bf16, e4m3fn_table
    g = np.random.default_rng(11)
    finite = e4m3fn_table()
    finite = finite[np.isfinite(finite)]
    grid = g.choice(finite, size=(4, 64)) * 2.0 ** -5
    grid[:, ::32] = 448.0 * 2.0 ** -5          # fixes every block's scale at 2^-5
    c, s = quantize_mxfp8(grid)
    np.testing.assert_array_equal(decode_mxfp8(c, s), grid)
    x = round_bf16(g.standard_normal((8, 256)) * np.exp(g.uniform(-3, 3, (8, 1))))
    c, s = quantize_mxfp8(x)
    v = decode_mxfp8(c, s)
    X = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=-1)
    y = np.abs(x) / X
    err = np.abs(v - x) / X
    normal = (y >= 2.0 ** -6) & (y <= 448.0)
    assert np.all(err[normal] <= 2.0 ** -4 * y[normal])
    assert np.all(err[y < 2.0 ** -6] <= 2.0 ** -10)
    big = y > 448.0
    np.testing.assert_array_equal(np.abs(v[big]) / X[big], 448.0)
    assert big.any()
