"""Pins of oracle.moe: brute force on tiny layers, closed forms, special cases."""

import itertools

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as M
from bit_moe_expert_02_amd import synth


def _tiny(seed=0, e=16, h=32, i=16):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, h))
    wr = (rng.standard_normal((e, h)) * 0.3).astype(np.float32)
    experts = [tuple(rng.standard_normal(s) * 0.2 for s in ((i, h), (i, h), (h, i))) for _ in range(e)]
    return x, wr, experts


# ---------------------------------------------------------------- selection
def test_topk_brute_force_tiny_layer():
    """Top-2 of 16 equals the pair with the largest key sum (every C(16,2) pair)."""
    wl = synth.WORKLOADS["tiny"]
    x = M.bf16_to_f64(synth.x_bf16(wl, 0, 4))
    wr = synth.router(wl, 0)
    logits = M.router_logits(x, wr)
    idx, w, _ = M.select_experts(logits, 2)
    for r in range(4):
        best = max(itertools.combinations(range(16), 2),
                   key=lambda p: (logits[r, p[0]] + logits[r, p[1]], tuple(-v for v in p)))
        assert set(best) == set(idx[r].tolist())
        assert logits[r, idx[r, 0]] >= logits[r, idx[r, 1]]
        # weights: softmax restricted to the pair, written out
        a, b = logits[r, idx[r, 0]], logits[r, idx[r, 1]]
        assert w[r, 0] == pytest.approx(1.0 / (1.0 + np.exp(b - a)), rel=1e-14)


def test_topk_brute_force_with_bias_k3():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((3, 10))
    bias = rng.uniform(-0.6, 1.0, 10)
    idx, w, _ = M.select_experts(logits, 3, bias)
    for r in range(3):
        key = logits[r] + bias
        best = max(itertools.combinations(range(10), 3), key=lambda p: sum(key[list(p)]))
        assert set(best) == set(idx[r].tolist())
        p = np.exp(logits[r, idx[r]])                        # unbiased weights
        assert np.allclose(w[r], p / p.sum(), rtol=1e-14)


def test_zero_router_ties_to_lower_id():
    logits = np.zeros((2, 12))
    idx, w, gap = M.select_experts(logits, 4)
    assert idx.tolist() == [[0, 1, 2, 3]] * 2
    assert np.all(w == 0.25)
    assert np.all(gap == 0.0)


def test_equal_keys_order_lower_id_first():
    logits = np.array([[1.0, 3.0, 2.0, 3.0, 2.0, 0.0]])
    idx, _, _ = M.select_experts(logits, 4)
    assert idx.tolist() == [[1, 3, 2, 4]]


def test_huge_bias_forces_expert_keeps_weight():
    x, wr, _ = _tiny(1)
    logits = M.router_logits(x, wr)
    bias = np.zeros(16)
    bias[11] = 1e6
    idx, w, _ = M.select_experts(logits, 3, bias)
    assert np.all(idx[:, 0] == 11)
    for r in range(4):
        p = np.exp(logits[r, idx[r]] - logits[r].max())
        assert np.allclose(w[r], p / p.sum(), rtol=1e-13)


def test_selected_softmax_equals_full_softmax_renormalised():
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((5, 40)) * 3
    idx, w, _ = M.select_experts(logits, 6)
    for r in range(5):
        z = logits[r, idx[r]]
        sm = np.exp(z - z.max())
        assert np.max(np.abs(w[r] - sm / sm.sum())) < 1e-15


def test_permuting_experts_permutes_idx_not_y():
    x, wr, experts = _tiny(2)
    perm = np.random.default_rng(9).permutation(16)
    bias = np.random.default_rng(10).uniform(-0.6, 1.0, 16)
    a = M.moe_layer(x, wr, 3, lambda e: experts[e], bias=bias)
    b = M.moe_layer(x, wr[perm], 3, lambda e: experts[perm[e]], bias=bias[perm])
    assert np.array_equal(perm[b["idx"]], a["idx"])
    assert np.allclose(a["y"], b["y"], rtol=1e-12, atol=1e-14)


def test_min_gap_reported():
    logits = np.array([[5.0, 4.0, 3.5, 1.0]])
    _, _, gap = M.select_experts(logits, 2)
    assert gap[0] == 0.5


# ---------------------------------------------------------------- experts
def test_expert_ffn_explicit_loops():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 12))
    wg, wu, wd = rng.standard_normal((7, 12)), rng.standard_normal((7, 12)), rng.standard_normal((12, 7))
    a = M.expert_ffn(x, wg, wu, wd)
    b = M.expert_ffn_loops(x, wg, wu, wd)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(b))


def test_silu_closed_forms():
    assert M.silu(np.array(0.0)) == 0.0
    assert M.silu(np.array(1.0)) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-15)
    assert M.silu(np.array(-40.0)) == pytest.approx(-40.0 * np.exp(-40.0), rel=1e-12)
    assert M.silu(np.array(40.0)) == pytest.approx(40.0, rel=1e-15)


def test_single_expert_weight_one_is_plain_ffn():
    x, wr, experts = _tiny(3)
    y = M.combine(x[:1], np.array([[5]]), np.array([[1.0]]), lambda e: experts[e])
    assert np.array_equal(y, M.expert_ffn(x[:1], *experts[5]))


def test_zero_weights_give_zero():
    x, wr, experts = _tiny(4)
    zero = tuple(np.zeros_like(m) for m in experts[0])
    out = M.moe_layer(x, wr, 2, lambda e: zero, shared=zero)
    assert not np.any(out["y"])


def test_dense_special_case():
    """top_k = E, no bias: the sparse path is the full softmax mixture."""
    x, wr, experts = _tiny(5, e=6)
    a = M.moe_layer(x, wr, 6, lambda e: experts[e], shared=experts[0])["y"]
    b = M.dense_moe(x, wr, experts, shared=experts[0])
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


def test_dense_brute_force_masked_mixture():
    """Sparse layer == all experts computed, masked by the selection, weighted."""
    x, wr, experts = _tiny(6)
    out = M.moe_layer(x, wr, 2, lambda e: experts[e])
    dense = np.stack([M.expert_ffn(x, *m) for m in experts])          # [E, R, H]
    y = np.zeros_like(x)
    for r in range(x.shape[0]):
        for s in range(2):
            y[r] += out["w"][r, s] * dense[out["idx"][r, s], r]
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-15)


def test_rows_independent():
    x, wr, experts = _tiny(7)
    full = M.moe_layer(x, wr, 3, lambda e: experts[e], shared=experts[1])
    for r in range(x.shape[0]):
        one = M.moe_layer(x[r:r + 1], wr, 3, lambda e: experts[e], shared=experts[1])
        assert np.array_equal(one["idx"][0], full["idx"][r])
        assert np.allclose(one["y"][0], full["y"][r], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("fmt", ["Q2_0", "Q8", "MXFP4", "TERN160"])
def test_doubling_block_scales_doubles_contribution(fmt):
    """Scaling every block scale by 2 doubles that expert's output exactly."""
    rng = np.random.default_rng(12)
    h, i = 320, 192 if fmt != "TERN160" else 160
    x = rng.standard_normal((2, h))
    mats = [F.pack(fmt, (rng.standard_normal(s) * 0.05).astype(np.float32)) for s in ((i, h), (i, h), (h, i))]
    shapes = ((i, h), (i, h), (h, i))

    def doubled(buf, shape):
        buf = buf.copy()
        n, k = shape
        nb = F.blocks_per_row(fmt, k)
        off = n * nb * F.CODE_BYTES[fmt]
        if fmt == "MXFP4":
            buf[off:] += 1                                    # e8m0 exponent + 1
        else:
            s = buf[off:].view("<f2")
            s *= np.float16(2.0)                               # exact unless overflow
        return buf

    dec = [F.decode(fmt, b, *s) for b, s in zip(mats, shapes)]
    # double only the down matrix: the expert output is linear in W_down
    dd = F.decode(fmt, doubled(mats[2], shapes[2]), *shapes[2])
    assert np.array_equal(dd, 2 * dec[2])
    a = M.expert_ffn(x, *dec)
    b = M.expert_ffn(x, dec[0], dec[1], dd)
    assert np.allclose(b, 2 * a, rtol=1e-13, atol=0)


def test_tiny_layer_from_packed_q2_0():
    """The tiny workload end to end in the oracle: shapes, weights sum, finite y."""
    wl = synth.WORKLOADS["tiny"]
    x = M.bf16_to_f64(synth.x_bf16(wl, 0, 4))
    wr = synth.router(wl, 0)

    def expert(e):
        g, u, d = synth.expert_weights(wl, 0, e)
        return (F.decode("Q2_0", F.pack("Q2_0", g), 256, 512),
                F.decode("Q2_0", F.pack("Q2_0", u), 256, 512),
                F.decode("Q2_0", F.pack("Q2_0", d), 512, 256))

    out = M.moe_layer(x, wr, 2, expert, shared=expert(16))
    assert out["idx"].shape == (4, 2) and out["y"].shape == (4, 512)
    assert np.allclose(out["w"].sum(axis=1), 1.0, rtol=1e-15)
    assert np.all(np.isfinite(out["y"]))
    assert np.all(out["min_gap"] > 1e-9)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F], np.uint16)
    v = M.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0
    assert v[4] == 3.140625
    assert v[5] == (2 - 2 ** -7) * 2.0 ** 127


def test_zipf_routing_input_shape_and_skew():
    """The prefill routing input: distinct ids per row, weights summing to 1,
    popularity falling with rank (the most popular expert far above the mean)."""
    from bit_moe_expert_02_amd import synth
    wl = synth.WORKLOADS["fp4_stack20"]
    idx, w = synth.zipf_routing(wl, 0, 2048)
    assert idx.shape == (2048, 6) and w.shape == (2048, 6)
    assert all(len(set(r)) == 6 for r in idx.tolist())
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    counts = np.bincount(idx.reshape(-1), minlength=384)
    assert counts.max() > 20 * counts.mean() and counts.mean() == 32


# ---------------------------------------------------------------- router GEMV
def test_router_logits_hand_worked(golden):
    """Logits of small integer / power-of-two inputs equal the sums worked by
    hand in the fixture (pins the x . Wr^T orientation: a transposed operand
    would score expert e with column e)."""
    g = golden("router_worked.json")["small"]
    got = M.router_logits(np.array(g["x"]), np.array(g["w_router"], np.float32))
    assert got.shape == (3, 3)
    assert np.array_equal(got, np.array(g["logits"]))


def test_router_logits_one_hot_rows_read_one_router_column():
    """x = unit vector at h gives logits[e] = Wr[e, h] exactly, for every h."""
    rng = np.random.default_rng(3)
    wr = (rng.standard_normal((16, 24)) * 0.02).astype(np.float32)
    x = np.eye(24)
    assert np.array_equal(M.router_logits(x, wr), wr.T.astype(np.float64))


def test_router_logits_accumulate_beyond_fp32(golden):
    """The sums are fp64: a logit that needs 31 significant bits comes out
    exact, and a sum of 2^24, 1, 1, -2^24 is 2.  The same inputs summed in
    fp32 (the slip this pin is meant to catch) give 1.0 and 0.0."""
    g = golden("router_worked.json")
    for case in ("beyond_fp32", "cancellation"):
        x = np.array(g[case]["x"])
        wr = np.array(g[case]["w_router"], np.float32)
        assert M.router_logits(x, wr)[0, 0] == g[case]["logit"]
        # a planted mistake: the same sum accumulated left to right in fp32
        acc = np.float32(0.0)
        for xv, wv in zip(x[0].astype(np.float32), wr[0]):
            acc = np.float32(acc + np.float32(xv * wv))
        assert float(acc) != g[case]["logit"]
