"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar: expert indices bit-exact; mixing weights within 1e-6 relative; layer
output within 1e-3 relative L2 per row.  Real-shape layers materialise only
the experts the checked rows select (every other slot is an all-zero expert;
a wrong selection would therefore also show up in y)."""

import numpy as np
import pytest

from tests import gpu_util as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from bit_moe_expert_02_amd import _lib as L          # noqa: E402
from bit_moe_expert_02_amd import layer as LY        # noqa: E402
from bit_moe_expert_02_amd import synth              # noqa: E402
from oracle import moe as OM                         # noqa: E402


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L.lib()


# ------------------------------------------------------------------ tiny layer
@pytest.mark.parametrize("rows,stream", [(4, 0), (1, 1), (2, 2), (5, 3), (8, 4)])
def test_tiny_layer(rows, stream):
    wl = synth.WORKLOADS["tiny"]
    _say("tiny layer rows", rows, "x stream", stream)
    xbits = synth.x_bf16(wl, 0, rows, stream)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    gi, gw, gy, _ = G.run_layer(dl, G.device_inputs(wl, 0, xbits), rows)
    G.check_routing(gi, gw, idx, w, gap, logits)
    ref = G.oracle_y(wl, 0, x, idx, w, list(range(rows)))
    err = G.rel_l2_rows(gy, ref)
    _say("  rel L2 per row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)


def test_tiny_repeated_rows_share_experts():
    """Identical rows select identical experts: each expert serves 5 rows
    (more than one staging batch)."""
    wl = synth.WORKLOADS["tiny"]
    xbits = np.repeat(synth.x_bf16(wl, 0, 1, 7), 5, axis=0)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    gi, gw, gy, _ = G.run_layer(dl, G.device_inputs(wl, 0, xbits), 5)
    G.check_routing(gi, gw, idx, w, gap, logits)
    ref = G.oracle_y(wl, 0, x, idx, w, list(range(5)))
    assert np.all(G.rel_l2_rows(gy, ref) <= G.REL_L2_TOL)
    assert np.array_equal(gy[0], gy[4])


def test_tiny_deterministic_and_workspace_reuse():
    """One zero-filled workspace serves calls of different row counts in turn
    (the fused launch's hand-off words are tagged per call, so words left by
    earlier calls must never be taken); equal inputs give bitwise equal y."""
    wl = synth.WORKLOADS["tiny"]
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    ys = []
    ws = LY.workspace(dl.dims, 8)
    for rows, stream in [(8, 10), (3, 11), (8, 12), (8, 10), (1, 13)]:
        xbits = synth.x_bf16(wl, 0, rows, stream)
        xd = G.device_inputs(wl, 0, xbits)
        idx = torch.zeros((rows, 2), dtype=torch.int32, device="cuda")
        wts = torch.zeros((rows, 2), dtype=torch.float32, device="cuda")
        y = torch.zeros((rows, wl.hidden), dtype=torch.float32, device="cuda")
        L.moe_layer(dl.dims, xd, rows, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                    idx, wts, y, ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
        x, ri, rw, logits, gap = G.oracle_route(wl, 0, xbits)
        assert np.array_equal(idx.cpu().numpy(), ri)
        ref = G.oracle_y(wl, 0, x, ri, rw, list(range(rows)))
        assert np.all(G.rel_l2_rows(ys[-1], ref) <= G.REL_L2_TOL)
    assert np.array_equal(ys[0], ys[3])            # bitwise reproducible


def test_given_up_waits_give_nan_and_the_next_call_recovers():
    """Failure path of the fused launch, forced from the host: with the spin
    limit at 0 every hand-off wait gives up at once, yet the launch drains
    and y is all NaN; the next call at the default limit, on the same
    workspace, is bitwise the call before."""
    wl = synth.WORKLOADS["tiny"]
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    ws = LY.workspace(dl.dims, 4)
    xd = G.device_inputs(wl, 0, synth.x_bf16(wl, 0, 4, 21))

    def run():
        idx = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
        wts = torch.zeros((4, 2), dtype=torch.float32, device="cuda")
        y = torch.zeros((4, wl.hidden), dtype=torch.float32, device="cuda")
        L.moe_layer(dl.dims, xd, 4, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                    idx, wts, y, ws)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    y_ok = run()
    assert np.all(np.isfinite(y_ok))
    assert L.moe_workspace_status(ws) == L.MOE_OK
    prev = L.moe_set_spin_limit(0)
    try:
        y_fail = run()
    finally:
        L.moe_set_spin_limit(prev)
    _say("NaN fraction with spin limit 0:", float(np.isnan(y_fail).mean()))
    assert np.all(np.isnan(y_fail))
    assert L.moe_workspace_status(ws) == L.MOE_ETIMEOUT      # reported once, then cleared
    assert L.moe_workspace_status(ws) == L.MOE_OK
    assert np.array_equal(run(), y_ok)
    assert L.moe_workspace_status(ws) == L.MOE_OK


def test_route_only_and_ffn_only_match_layer():
    wl = synth.WORKLOADS["tiny"]
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    xbits = synth.x_bf16(wl, 0, 3, 5)
    xd = G.device_inputs(wl, 0, xbits)
    ws = LY.workspace(dl.dims, 3)
    idx = torch.zeros((3, 2), dtype=torch.int32, device="cuda")
    wts = torch.zeros((3, 2), dtype=torch.float32, device="cuda")
    L.moe_route(dl.dims, xd, 3, dl.router, dl.bias, idx, wts, ws)
    y = torch.zeros((3, wl.hidden), dtype=torch.float32, device="cuda")
    L.moe_expert_ffn(dl.dims, xd, 3, idx, wts, dl.weights, dl.experts, dl.shared, y, ws)
    torch.cuda.synchronize()
    gi, gw, gy, _ = G.run_layer(dl, xd, 3)
    assert np.array_equal(idx.cpu().numpy(), gi)
    assert np.array_equal(wts.cpu().numpy(), gw)
    np.testing.assert_allclose(y.cpu().numpy(), gy, rtol=1e-6, atol=1e-7)


def test_tiny_topk_max():
    """top_k = 8 of 16 (the largest the selection kernel takes), no shared expert."""
    base = synth.WORKLOADS["tiny"]
    wl = synth.Workload("tiny_k8", 11, 512, 256, 16, 8, "Q2_0", None, rows=(2,))
    xbits = synth.x_bf16(wl, 0, 8, 0)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    dl = LY.DeviceLayer(wl, 0, materialize=range(16))
    gi, gw, gy, _ = G.run_layer(dl, G.device_inputs(wl, 0, xbits), 8)
    G.check_routing(gi, gw, idx, w, gap, logits)
    assert np.all(G.rel_l2_rows(gy, G.oracle_y(wl, 0, x, idx, w, list(range(8)))) <= G.REL_L2_TOL)
    del base


def test_tiny_selection_limits():
    """The selection and its hand-off at their limits: 500 experts (a ragged
    last lane group of the 8 per lane), top_k = 8, 8 rows (64 entries, every
    word of a published copy), mixed formats, a Q8 shared expert and a bias."""
    wl = synth.Workload("tiny_limits", 12, 512, 256, 500, 8, "MIX", "Q8", use_bias=True, rows=(8,))
    xbits = synth.x_bf16(wl, 0, 8, 0)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    need = sorted(set(idx.reshape(-1).tolist()))
    _say("tiny limits: experts", len(need))
    dl = LY.DeviceLayer(wl, 0, materialize=need)
    gi, gw, gy, _ = G.run_layer(dl, G.device_inputs(wl, 0, xbits), 8)
    G.check_routing(gi, gw, idx, w, gap, logits)
    err = G.rel_l2_rows(gy, G.oracle_y(wl, 0, x, idx, w, list(range(8))))
    _say("  rel L2 per row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)


def test_selection_exact_ties_and_lower_half_order():
    """Keys that tie exactly, and keys equal in their upper 32 bits that
    differ only below: a zero router (every logit 0) and a crafted bias, so
    key = bias exactly.  Expected from the rules alone: equal keys go to the
    lower id, so experts 5, 69, 133 (one lane of the selection wave, bias 2)
    come first, then 10, 11, 300 (bias 1 + 3 * 2^-23, three lanes), then 21
    (1 + 2 * 2^-23) and 20 (1 + 2^-23), whose keys differ only in their lower
    32 bits; weights are all 1/8 (the unbiased logits are equal).  Through the
    fused layer and the split route, 1 and 8 rows."""
    wl = synth.Workload("tiny_ties", 13, 512, 256, 384, 8, "Q2_0", None, use_bias=True, rows=(8,))
    bias = np.full(384, -1.0, np.float32)
    bias[[5, 69, 133]] = 2.0
    u = np.float32(2.0 ** -23)
    bias[[10, 11, 300]] = np.float32(1.0) + 3 * u
    bias[21] = np.float32(1.0) + 2 * u
    bias[20] = np.float32(1.0) + u
    want = [5, 69, 133, 10, 11, 300, 21, 20]
    dl = LY.DeviceLayer(wl, 0, materialize=want)
    dl.router.zero_()
    dl.bias.copy_(torch.from_numpy(bias))
    for rows in (1, 8):
        xbits = synth.x_bf16(wl, 0, rows, 0)
        oi, ow, _ = OM.select_experts(np.zeros((rows, 384)), 8, bias)
        assert all(list(r) == want for r in oi)                     # the oracle agrees with the rules
        gi, gw, gy, _ = G.run_layer(dl, G.device_inputs(wl, 0, xbits), rows)
        assert np.array_equal(gi, oi), gi
        np.testing.assert_array_equal(gw, np.full((rows, 8), 0.125, np.float32))
        ref = G.oracle_y(wl, 0, OM.bf16_to_f64(xbits), oi, ow, list(range(rows)))
        assert np.all(G.rel_l2_rows(gy, ref) <= G.REL_L2_TOL)
        ws = LY.workspace(dl.dims, rows)
        idx = torch.zeros((rows, 8), dtype=torch.int32, device="cuda")
        wts = torch.zeros((rows, 8), dtype=torch.float32, device="cuda")
        L.moe_route(dl.dims, G.device_inputs(wl, 0, xbits), rows, dl.router, dl.bias, idx, wts, ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), oi)


# ------------------------------------------------------------------ real shapes
def _real_case(wl, rows, stream, check_rows):
    xbits = synth.x_bf16(wl, 0, rows, stream)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    need = sorted(set(idx[check_rows].reshape(-1).tolist()))
    _say(f"{wl.name}: rows {rows}, checking rows {check_rows}, experts {need}")
    dl = LY.DeviceLayer(wl, 0, materialize=need)
    gi, gw, gy, _ = G.run_layer(dl, G.device_inputs(wl, 0, xbits), rows)
    G.check_routing(gi, gw, idx, w, gap, logits)
    ref = G.oracle_y(wl, 0, x, idx, w, check_rows)
    err = G.rel_l2_rows(gy[check_rows], ref)
    _say("  rel L2 per checked row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)
    return gy


def test_decode_q2_layer_one_row():
    _real_case(synth.WORKLOADS["decode_q2"], 1, 0, [0])


def _every_row_case(wl, rows, stream, twice=True):
    """A real-shape layer holding exactly the experts the rows select, every
    row checked against the oracle; with `twice`, a second call on the same
    workspace must give bitwise the same y, idx and weights."""
    xbits = synth.x_bf16(wl, 0, rows, stream)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    _say(f"{wl.name}: rows {rows}, {len(np.unique(idx))} distinct experts, every row checked")
    dl, ref = G.materialized_layer_and_oracle(wl, 0, x, idx, w)
    xd = G.device_inputs(wl, 0, xbits)
    gi, gw, gy, ws = G.run_layer(dl, xd, rows)
    G.check_routing(gi, gw, idx, w, gap, logits)
    err = G.rel_l2_rows(gy, ref)
    _say("  rel L2 per row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)
    if twice:
        idx2 = torch.zeros((rows, wl.top_k), dtype=torch.int32, device="cuda")
        wts2 = torch.zeros((rows, wl.top_k), dtype=torch.float32, device="cuda")
        y2 = torch.zeros((rows, wl.hidden), dtype=torch.float32, device="cuda")
        L.moe_layer(dl.dims, xd, rows, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                    idx2, wts2, y2, ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx2.cpu().numpy(), gi)
        assert np.array_equal(wts2.cpu().numpy(), gw)
        assert np.array_equal(y2.cpu().numpy(), gy), "a second identical call changed y"
        assert L.moe_workspace_status(ws) == L.MOE_OK


@pytest.mark.parametrize("rows", [1, 5, 8])
def test_mixed_verify_layer_every_row(rows):
    """The mixed-format verify layer with its selection bias (ternary / Q2_0 /
    Q3 experts, a Q8 shared expert) at rows 1, 5 and 8: every row."""
    _every_row_case(synth.WORKLOADS["mixed_verify"], rows, rows)


@pytest.mark.parametrize("rows", [1, 8])
def test_fp4_layer_fused_every_row(rows):
    """MXFP4 experts through the fused launch (moe_layer), one layer of the
    FP4 stack (no shared expert), at rows 1 and 8: every row."""
    _every_row_case(synth.WORKLOADS["fp4_stack20"], rows, 40 + rows)


def test_many_row_call_then_fused_call_share_a_workspace():
    """A many-row call writes its pair lists and chunk tables into the
    workspace; a fused decode call on the same workspace right after must not
    take any of those words for its own hand-off words (the tagged area sits
    apart from everything else).  55 rows then 1 row, real shape."""
    wl = synth.WORKLOADS["fp4_stack20"]
    xb1 = synth.x_bf16(wl, 0, 1, 77)
    x1, idx1, w1, logits, gap = G.oracle_route(wl, 0, xb1)
    dl, ref = G.materialized_layer_and_oracle(wl, 0, x1, idx1, w1, flags=L.MOE_ACT_MXFP8)
    ws = torch.zeros(max(L.workspace_bytes(dl.dims, 55), L.workspace_bytes(dl.dims, 1)),
                     dtype=torch.uint8, device="cuda")
    ri, rw = synth.zipf_routing(wl, 0, 55)
    y55 = torch.zeros((55, wl.hidden), dtype=torch.float32, device="cuda")
    L.moe_expert_ffn(dl.dims, G.device_inputs(wl, 0, synth.x_bf16(wl, 0, 55, 78)), 55,
                     torch.from_numpy(ri).cuda(), torch.from_numpy(rw).cuda(), dl.weights,
                     dl.experts, None, y55, ws)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(y55.cpu().numpy()))
    idx = torch.zeros((1, wl.top_k), dtype=torch.int32, device="cuda")
    wts = torch.zeros((1, wl.top_k), dtype=torch.float32, device="cuda")
    y = torch.zeros((1, wl.hidden), dtype=torch.float32, device="cuda")
    L.moe_layer(dl.dims, G.device_inputs(wl, 0, xb1), 1, dl.router, dl.bias, dl.weights,
                dl.experts, dl.shared, idx, wts, y, ws)
    torch.cuda.synchronize()
    G.check_routing(idx.cpu().numpy(), wts.cpu().numpy(), idx1, w1, gap, logits)
    err = G.rel_l2_rows(y.cpu().numpy(), ref)
    _say("  rel L2", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)
    assert L.moe_workspace_status(ws) == L.MOE_OK


@pytest.mark.parametrize("fmt", ["TERN160", "Q2_0", "Q3", "MXFP4", "Q8"])
def test_expert_ffn_each_format_real_shape(fmt):
    """moe_expert_ffn with given routing, every routed expert in one format."""
    wl = synth.Workload(f"single_{fmt}", 20 + L.FMT[fmt], 5120, 2304, 384, 6, fmt, None, rows=(2,))
    rows = 2
    xbits = synth.x_bf16(wl, 0, rows, 0)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    idx = idx[:, :2].copy()                              # two experts per row keeps this quick
    w = w[:, :2] / w[:, :2].sum(axis=1, keepdims=True)
    w32 = w.astype(np.float32)
    need = sorted(set(idx.reshape(-1).tolist()))
    dl = LY.DeviceLayer(wl, 0, materialize=need)
    d = L.dims(wl.hidden, wl.inter, wl.n_experts, 2)
    ws = LY.workspace(d, rows)
    y = torch.zeros((rows, wl.hidden), dtype=torch.float32, device="cuda")
    L.moe_expert_ffn(d, G.device_inputs(wl, 0, xbits), rows,
                     torch.from_numpy(idx.astype(np.int32)).cuda(), torch.from_numpy(w32).cuda(),
                     dl.weights, dl.experts, None, y, ws)
    torch.cuda.synchronize()
    ref = G.oracle_y(wl, 0, x, idx, w32.astype(np.float64), list(range(rows)))
    err = G.rel_l2_rows(y.cpu().numpy(), ref)
    _say(f"  {fmt}: rel L2 per row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)


@pytest.mark.parametrize("rows", [2, 5])
def test_fused_layer_matches_split_calls_real_shape(rows):
    """moe_layer (fused launch) against moe_route + moe_expert_ffn (one launch
    per step) on the mixed-format verify layer: same ids, same y.  With
    several rows the shared workers run the shared expert's down tiles before
    their routed items; a down tile overwrites the staged x row, so a later
    gate/up item of that row must stage x again (the last row came out NaN
    when it did not)."""
    wl = synth.WORKLOADS["mixed_verify"]
    xbits = synth.x_bf16(wl, 0, rows, 21)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    need = sorted(set(idx.reshape(-1).tolist()))
    dl = LY.DeviceLayer(wl, 0, materialize=need)
    xd = G.device_inputs(wl, 0, xbits)
    gi, gw, gy, _ = G.run_layer(dl, xd, rows)
    ws = LY.workspace(dl.dims, rows)
    idx2 = torch.zeros((rows, wl.top_k), dtype=torch.int32, device="cuda")
    wts2 = torch.zeros((rows, wl.top_k), dtype=torch.float32, device="cuda")
    L.moe_route(dl.dims, xd, rows, dl.router, dl.bias, idx2, wts2, ws)
    y2 = torch.zeros((rows, wl.hidden), dtype=torch.float32, device="cuda")
    L.moe_expert_ffn(dl.dims, xd, rows, idx2, wts2, dl.weights, dl.experts, dl.shared, y2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), gi)
    assert np.array_equal(wts2.cpu().numpy(), gw)
    assert not np.isnan(gy).any(), f"NaN rows of the fused y: {sorted(set(np.where(np.isnan(gy))[0]))}"
    np.testing.assert_allclose(y2.cpu().numpy(), gy, rtol=1e-6, atol=1e-6)
    G.check_routing(gi, gw, idx, w, gap, logits)


# ------------------------------------------------------------------ workloads of the next steps
@pytest.mark.parametrize("rows", [1, 5])
def test_draft_layer_every_row(rows):
    """The draft model's MoE layer: 128 experts, top-3, a Q2_0 shared expert."""
    _every_row_case(synth.WORKLOADS["draft128"], rows, 60 + rows)


@pytest.mark.parametrize("scale,rows", [(0.5, 7), (1.0, 1)])
def test_residency_policy_bias_every_row(scale, rows):
    """The mixed layer under the residency-style selection bias (+1.0 fast /
    -0.6 slow tier, times the scale): ids exact, weights the unbiased softmax."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["policy_stack40"], layers=1, extra={"policy_scale": scale})
    _every_row_case(wl, rows, 70 + rows, twice=False)


def test_correlated_verify_window_every_row():
    """A verify window of 7 correlated rows (rho 0.9): rows share experts, so
    slots serve several rows; every row checked."""
    wl = synth.WORKLOADS["verify_correlated"]
    rows = 7
    xbits = synth.correlated_x(wl, 0, rows, 0.9, 5)
    x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
    _say(f"correlated window: {len(np.unique(idx))} distinct experts for {rows} rows")
    assert len(np.unique(idx)) < rows * wl.top_k
    dl, ref = G.materialized_layer_and_oracle(wl, 0, x, idx, w)
    gi, gw, gy, ws = G.run_layer(dl, G.device_inputs(wl, 0, xbits), rows)
    G.check_routing(gi, gw, idx, w, gap, logits)
    err = G.rel_l2_rows(gy, ref)
    _say("  rel L2 per row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)
