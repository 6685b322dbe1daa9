"""GPU parity of the stacked decode (moe_stack_decode), teacher-forced: the
oracle's layer l takes exactly the bf16 x_l the GPU consumed, so a 1-ulp
difference in one layer cannot grow into a routing change downstream.

Per layer: expert ids bit-exact, mixing weights to 1e-6, y within 1e-3
relative L2 per checked row, and the next input x_{l+1} equal bit for bit to
the oracle's bf16(y_l + noise_l) of the GPU's own fp32 y_l."""

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


def _run_stack(wl, layers, rows, stream=0):
    H, k, n = wl.hidden, wl.top_k, len(layers)
    x_all = torch.zeros((n + 1, rows, H), dtype=torch.int16, device="cuda")
    x_all[0] = torch.from_numpy(synth.x_bf16(wl, 0, rows, stream).view(np.int16).copy()).cuda()
    noise = torch.from_numpy(np.stack([synth.noise(wl, l, rows) for l in range(n)])).cuda()
    y_all = torch.zeros((n, rows, H), dtype=torch.float32, device="cuda")
    idx_all = torch.zeros((n, rows, k), dtype=torch.int32, device="cuda")
    wts_all = torch.zeros((n, rows, k), dtype=torch.float32, device="cuda")
    ws = LY.workspace(layers[0].dims, rows)
    L.moe_stack_decode(layers[0].dims, L.layer_weights(layers), rows, x_all, noise, y_all,
                       idx_all, wts_all, ws)
    torch.cuda.synchronize()
    return (x_all.cpu().numpy().view(np.uint16), noise.cpu().numpy(), y_all.cpu().numpy(),
            idx_all.cpu().numpy(), wts_all.cpu().numpy())


def _check_layers(wl, layers, rows, check_rows, stream=0, parallel=False):
    xs, noise, ys, idxs, wtss = _run_stack(wl, layers, rows, stream)
    for l, dl in enumerate(layers):
        x, idx, w, logits, gap = G.oracle_route(wl, l, xs[l])
        G.check_routing(idxs[l], wtss[l], idx, w, gap, logits)
        if parallel:
            ref = G.oracle_y_parallel(dl, x[check_rows], idx[check_rows], w[check_rows])
        else:
            ref = G.oracle_y_for(dl, x, idx, w, check_rows)
        err = G.rel_l2_rows(ys[l][check_rows], ref)
        _say(f"  layer {l}: rel L2 {G.fmt_err(err)}")
        assert np.all(err <= G.REL_L2_TOL)
        nxt = OM.chain_next(ys[l], noise[l])
        np.testing.assert_array_equal(OM.bf16_to_f64(xs[l + 1]), nxt)


@pytest.mark.parametrize("rows", [1, 7])
def test_tiny_stack_chained(rows):
    wl = synth.WORKLOADS["tiny_stack"]
    _say(f"tiny stack: {wl.layers} layers, rows {rows}")
    layers = [LY.DeviceLayer(wl, l, materialize=range(wl.n_experts)) for l in range(wl.layers)]
    _check_layers(wl, layers, rows, list(range(rows)), stream=rows)


def test_mixed_stack_real_shape_three_layers():
    """Three layers of the 40-layer mixed stack at rows 7, every row of every
    layer; slots are pool-filled, every selected expert's weights are
    regenerated for the oracle."""
    base = synth.WORKLOADS["stack40_mixed"]
    rows, n = 7, 3
    _say(f"mixed stack: {n} layers of {base.name}, rows {rows}")
    pool = LY.make_pool(base, 0, ["TERN160", "Q2_0", "Q3"], 8)
    layers = [LY.DeviceLayer(base, l, materialize=(), pool=pool) for l in range(n)]
    _check_layers(base, layers, rows, list(range(rows)), stream=3, parallel=True)


@pytest.mark.parametrize("rows", [1, 8])
def test_fp4_stack_real_shape_three_layers(rows):
    """Three layers of the FP4 stack (MXFP4 experts, no shared expert) chained
    through moe_stack_decode at rows 1 and 8, every row of every layer."""
    base = synth.WORKLOADS["fp4_stack20"]
    n = 3
    _say(f"fp4 stack: {n} layers of {base.name}, rows {rows}")
    pool = LY.make_pool(base, 0, ["MXFP4"], 12)
    layers = [LY.DeviceLayer(base, l, materialize=(), pool=pool) for l in range(n)]
    _check_layers(base, layers, rows, list(range(rows)), stream=50 + rows, parallel=True)
