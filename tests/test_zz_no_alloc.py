"""moe_layer_noalloc (the fused layer on the library's fixed per-GPU
workspace) against moe_layer on a caller workspace: the same kernels, so the
same ids, weights and y bit for bit; two calls in a row, the second with
fewer rows, and the oracle as the reference for both."""

import numpy as np
import pytest

from tests import gpu_util as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from bit_moe_expert_02_amd import _lib as L          # noqa: E402
from bit_moe_expert_02_amd import layer as LY        # noqa: E402
from bit_moe_expert_02_amd import synth              # noqa: E402


def _say(*a):
    print(*a, flush=True)


def _both(dl, xbits, rows):
    wl = dl.wl
    xd = G.device_inputs(wl, 0, xbits)
    gi, gw, gy, _ = G.run_layer(dl, xd, rows)
    idx = torch.zeros((rows, wl.top_k), dtype=torch.int32, device="cuda")
    wts = torch.zeros((rows, wl.top_k), dtype=torch.float32, device="cuda")
    y = torch.full((rows, wl.hidden), float("nan"), dtype=torch.float32, device="cuda")
    L.moe_layer_noalloc(dl.dims, xd, rows, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                        idx, wts, y)
    torch.cuda.synchronize()
    return (gi, gw, gy), (idx.cpu().numpy(), wts.cpu().numpy(), y.cpu().numpy())


@pytest.mark.parametrize("name,rows_seq", [("tiny", (8, 3)), ("mixed_verify", (8, 1))])
def test_noalloc_matches_moe_layer(name, rows_seq):
    wl = synth.WORKLOADS[name]
    for n, rows in enumerate(rows_seq):
        _say(f"{name}: call {n + 1}, rows {rows}")
        xbits = synth.x_bf16(wl, 0, rows, 300 + rows)
        x, idx, w, logits, gap = G.oracle_route(wl, 0, xbits)
        if name == "tiny":
            dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
            ref = G.oracle_y(wl, 0, x, idx, w, list(range(rows)))
        else:
            dl, ref = G.materialized_layer_and_oracle(wl, 0, x, idx, w)
        (gi, gw, gy), (ni, nw, ny) = _both(dl, xbits, rows)
        G.check_routing(ni, nw, idx, w, gap, logits)
        assert np.array_equal(ni, gi) and np.array_equal(nw, gw)
        assert np.array_equal(ny, gy), "moe_layer_noalloc differs from moe_layer"
        err = G.rel_l2_rows(ny, ref)
        _say("  rel L2 per row", G.fmt_err(err))
        assert np.all(err <= G.REL_L2_TOL)


def test_noalloc_argument_errors_and_null_routing_outputs():
    wl = synth.WORKLOADS["tiny"]
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    xd = G.device_inputs(wl, 0, synth.x_bf16(wl, 0, 4, 310))
    y = torch.zeros((9, wl.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(L.MoeError) as e:
        L.moe_layer_noalloc(dl.dims, xd, 9, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                            None, None, y)
    assert e.value.status == L.MOE_ESHAPE
    L.moe_layer_noalloc(dl.dims, xd, 0, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                        None, None, y)                   # rows 0: nothing launched
    L.moe_layer_noalloc(dl.dims, xd, 4, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                        None, None, y)                   # routing outputs not wanted
    torch.cuda.synchronize()
    _, _, gy, _ = G.run_layer(dl, xd, 4)
    assert np.array_equal(y[:4].cpu().numpy(), gy)
