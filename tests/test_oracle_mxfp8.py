"""Pins of the oracle's MXFP8 activation quantiser (prefill path).

The elementwise rounding is checked exhaustively over every finite bf16 value
against a nearest-value search in the full e4m3 value table, which is built
here bit by bit from the OCP definition (1 sign, 4 exponent bits with bias 7,
3 mantissa bits, subnormals, S.1111.111 = NaN)."""

import numpy as np

from oracle import moe as M


def _e4m3_table():
    vals, mant = [], []
    for code in range(128):
        e, m = code >> 3, code & 7
        if e == 15 and m == 7:
            continue                                    # NaN
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append(v)
        mant.append(m)
    return np.array(vals), np.array(mant)


def test_e4m3_table_limits(golden):
    g = golden("ocp_mx_tables.json")["e4m3"]
    vals, _ = _e4m3_table()
    assert vals.max() == g["max"]
    assert sorted(vals)[1] == g["min_subnormal"]
    assert (1 + 0 / 8) * 2.0 ** -6 == g["min_normal"]


def test_round_e4m3_exhaustive_bf16():
    vals, mant = _e4m3_table()
    bits = np.arange(1 << 16, dtype=np.uint32)
    x32 = (bits << 16).view(np.float32)
    x = x32[np.isfinite(x32)].astype(np.float64)
    a = np.abs(x)
    dist = np.abs(a[:, None] - vals[None, :])
    dmin = dist.min(axis=1, keepdims=True)
    cand = dist == dmin
    # ties: the candidate with even mantissa; beyond the table: saturate at 448
    even = cand & (mant[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    ref = np.copysign(np.where(a >= 448.0, 448.0, vals[pick]), x)
    got = M.round_e4m3(x)
    assert np.array_equal(got, ref)


def test_quant_mxfp8_scale_and_block():
    x = np.zeros((2, 64))
    x[0, :32] = np.linspace(-3, 3, 32)
    x[0, 32:] = 1000.0 * np.sign(np.linspace(-1, 1, 32) + 0.01)
    q, e = M.quant_mxfp8(x)
    assert e[0, 0] == 1 - 8 + 127                       # floor(log2 3) = 1
    assert e[0, 1] == 9 - 8 + 127                       # floor(log2 1000) = 9
    assert e[1, 0] == 0 and not np.any(q[1])            # all-zero block
    # 1000 / 2^(E-127) = 500 lies above the e4m3 maximum: it saturates to 448 * 2
    assert np.all(np.abs(q[0, 32:]) == 896.0)
    rel = np.abs(q[0, :32] - x[0, :32]) / np.maximum(np.abs(x[0, :32]), 1e-30)
    assert np.all(rel[np.abs(x[0, :32]) > 0.25] <= 2.0 ** -4)
