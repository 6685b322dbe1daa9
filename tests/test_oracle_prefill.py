"""Pins of the oracle's prefill path (MXFP8 activations, MXFP4 experts).

The MXFP8 quantiser itself is pinned exhaustively elsewhere; here:
  * on activations that MXFP8 represents exactly, the prefill layer is the
    decode layer's weighted sum (the quantiser is the only difference);
  * otherwise the quantised x stays within the e4m3 half-quantum bound of x
    and the layer output moves, but only slightly;
  * grouping rows by expert changes nothing: a batch equals its rows one at
    a time, each summed over its experts in ascending id with its weights."""

import numpy as np

from oracle import moe as OM


def _expert(rng, H, I, s=0.05):
    return (rng.standard_normal((I, H)) * s, rng.standard_normal((I, H)) * s,
            rng.standard_normal((H, I)) * s)


def _setup(seed, H=64, I=64, E=5, k=2, R=7):
    rng = np.random.default_rng(seed)
    experts = [_expert(rng, H, I) for _ in range(E)]
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(R)])
    w = rng.random((R, k))
    return rng, experts, idx, w


def test_exactly_representable_x_gives_the_decode_layer():
    rng, experts, idx, w = _setup(1)
    x = rng.standard_normal((7, 64))
    xq, _ = OM.quant_mxfp8(x)                       # on the MXFP8 grid by construction
    y = OM.prefill_layer(xq, idx, w, lambda e: experts[e])
    ref = OM.combine(xq, idx, w, lambda e: experts[e])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_quantisation_error_of_x_is_bounded():
    rng, experts, idx, w = _setup(2)
    x = rng.standard_normal((7, 64))
    y = OM.prefill_layer(x, idx, w, lambda e: experts[e])
    ref = OM.combine(x, idx, w, lambda e: experts[e])
    xq, E = OM.quant_mxfp8(x)
    dx = np.abs(x - xq)
    half_q = np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(np.ldexp(1.0, E - 127 - 10), 32, axis=1))
    assert np.all(dx <= half_q * (1 + 1e-12))                    # the e4m3 half-quantum bound
    assert np.max(np.abs(y - ref)) > 0                            # the activations were quantised
    assert np.max(np.abs(y - ref)) < 0.2 * np.max(np.abs(ref))    # and only slightly


def test_prefill_rows_are_independent_and_weighted():
    rng, experts, idx, w = _setup(3)
    x = rng.standard_normal((7, 64))
    y = OM.prefill_layer(x, idx, w, lambda e: experts[e])
    for r in range(7):
        xq, _ = OM.quant_mxfp8(x[r:r + 1])
        want = sum(w[r, j] * OM.expert_ffn(xq, *experts[idx[r, j]])[0] for j in np.argsort(idx[r]))
        np.testing.assert_allclose(y[r], want, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- many-row layer, any format
def test_many_row_layer_without_the_flag_is_the_decode_layer():
    """No MXFP8 activations: the many-row layer is the decode layer's weighted
    sum on the unquantised rows, for every format, shared expert included."""
    rng, experts, idx, w = _setup(4)
    x = rng.standard_normal((7, 64))
    shared = _expert(rng, 64, 64)
    y = OM.many_row_layer(x, idx, w, lambda e: experts[e], lambda e: "MXFP4", False, shared)
    ref = OM.combine(x, idx, w, lambda e: experts[e], shared)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_many_row_layer_all_mxfp4_with_the_flag_is_the_prefill_layer():
    rng, experts, idx, w = _setup(5)
    x = rng.standard_normal((7, 64))
    y = OM.many_row_layer(x, idx, w, lambda e: experts[e], lambda e: "MXFP4", True)
    np.testing.assert_allclose(y, OM.prefill_layer(x, idx, w, lambda e: experts[e]), rtol=1e-12, atol=1e-14)


def test_many_row_layer_mixed_formats_split_by_format():
    """With the flag, a table mixing MXFP4 and other experts is the sum of the
    MXFP4 experts' prefill layer and the other experts' decode layer: split
    the routing by format (zero weight where the other kind is selected)."""
    rng, experts, idx, w = _setup(6, E=6, k=3)
    x = rng.standard_normal((7, 64))
    fmts = ["MXFP4", "Q2_0", "MXFP4", "TERN160", "Q3", "MXFP4"]
    y = OM.many_row_layer(x, idx, w, lambda e: experts[e], lambda e: fmts[e], True)
    is_fp4 = np.vectorize(lambda e: fmts[e] == "MXFP4")(idx)
    part_fp4 = OM.prefill_layer(x, idx, np.where(is_fp4, w, 0.0), lambda e: experts[e])
    part_rest = OM.combine(x, idx, np.where(is_fp4, 0.0, w), lambda e: experts[e])
    np.testing.assert_allclose(y, part_fp4 + part_rest, rtol=1e-12, atol=1e-13)
