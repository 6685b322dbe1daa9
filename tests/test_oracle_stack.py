"""Pins of the stacked-decode step: bf16 rounding and the chained input.

The rounding is pinned to IEEE round-to-nearest-even by closed forms (halfway
cases between adjacent bf16 values), by every finite bf16 pattern mapping to
itself, and by an independent bit-level construction of both bf16 neighbours
of random fp32 values (the result must be the nearer, the even one on ties)."""

import numpy as np

from oracle import moe as OM


def test_round_bf16_halfway_cases_go_to_even():
    one = 1.0
    u = 2.0 ** -7                                  # bf16 spacing just above 1
    assert OM.round_bf16(one + u / 2) == one          # tie: 1.0 has the even significand
    assert OM.round_bf16(one + 3 * u / 2) == one + 2 * u
    assert OM.round_bf16(one + u / 2 + 2.0 ** -20) == one + u
    assert OM.round_bf16(-(one + 3 * u / 2)) == -(one + 2 * u)
    assert OM.round_bf16(2.0 ** -130) == 2.0 ** -130   # subnormal grid 2^-133
    assert OM.round_bf16(2.0 ** -134) == 0.0           # halfway to the first subnormal: even (0)
    assert OM.round_bf16(3 * 2.0 ** -134) == 2.0 ** -132
    assert OM.round_bf16(OM.BF16_MAX) == OM.BF16_MAX
    assert np.isinf(OM.round_bf16(OM.BF16_MAX + 2.0 ** 119))   # halfway past the top: to infinity


def test_every_finite_bf16_is_a_fixed_point():
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (bits << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(v)
    np.testing.assert_array_equal(OM.round_bf16(v[ok]), v[ok])


def test_nearest_neighbour_by_bit_construction():
    rng = np.random.default_rng(5)
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
                        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-39)])
    u = f.view(np.uint32)
    lo = (u & 0xFFFF0000).view(np.float32).astype(np.float64)              # toward zero
    hi = ((u & 0xFFFF0000) + 0x10000).view(np.float32).astype(np.float64)  # away from zero
    v = f.astype(np.float64)
    dlo, dhi = np.abs(v - lo), np.abs(hi - v)
    lo_even = ((u >> 16) & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo_even, lo, hi)))
    np.testing.assert_array_equal(OM.round_bf16(v), want)


def test_chain_next_adds_in_fp32_then_rounds():
    y = np.array([1.0, 1.0, 3.0e-8, -2.5], np.float32)
    e = np.array([2.0 ** -24, 2.0 ** -8, 1.0, 0.5], np.float32)
    # 1 + 2^-24 rounds to 1 in fp32 before bf16 sees it; 1 + 2^-8 is a bf16 tie -> 1
    np.testing.assert_array_equal(OM.chain_next(y, e), [1.0, 1.0, 1.0, -2.0])


def test_chain_next_bounds_rows_by_a_power_of_two():
    """Rows whose largest |y + eps| is below 4 pass unscaled; a row reaching 4
    is halved; 100 goes to 100 / 32 = 3.125 (floor(log2 100) = 6, s = 5);
    each row has its own power; a NaN or an infinity leaves its row unscaled."""
    z = np.zeros(4, np.float32)
    rows = np.array([[3.99, -1.0, 0.5, 0.25],
                     [4.0, -1.0, 0.5, 0.25],
                     [-100.0, 3.0, 0.5, 1.0],
                     [np.nan, 8.0, 2.0, 1.0],
                     [np.inf, 8.0, 2.0, 1.0]], np.float32)
    out = OM.chain_next(rows, np.zeros_like(rows))
    np.testing.assert_array_equal(out[0], OM.round_bf16(rows[0].astype(np.float64)))
    np.testing.assert_array_equal(out[1], [2.0, -0.5, 0.25, 0.125])
    np.testing.assert_array_equal(out[2], OM.round_bf16(np.array([-3.125, 3 / 32, 0.5 / 32, 1 / 32])))
    assert np.isnan(out[3, 0]) and np.array_equal(out[3, 1:], [8.0, 2.0, 1.0])
    assert np.isinf(out[4, 0]) and np.array_equal(out[4, 1:], [8.0, 2.0, 1.0])
    # a power of two commutes with the rounding: the bound only moves the exponent
    g = np.random.default_rng(2).standard_normal((3, 64)).astype(np.float32) * np.float32(50)
    o = OM.chain_next(g, z[:1].repeat(64)[None, :].repeat(3, 0))
    for r in range(3):
        sh = int(np.floor(np.log2(np.abs(g[r]).max()))) - 1
        np.testing.assert_array_equal(o[r], OM.round_bf16(g[r].astype(np.float64)) / 2.0 ** sh)
        assert 2.0 <= np.abs(o[r]).max() < 4.0
