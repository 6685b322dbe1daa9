"""GPU parity of the stack-larger-than-HBM path ([P1 §3C, §5], [P3 §五.2]).

  * moe_expert_ffn with pairs marked -1 (served elsewhere): they add nothing,
    on the decode path and on the many-row path; an id outside [-1, E) makes
    only its own row NaN;
  * the offloaded tiny stack (routed experts in pinned host memory, 5 device
    slots for 64 experts) at copy shares 0, 0.5 and 1, two passes each so
    that slots hit: teacher-forced against the oracle layer by layer (ids
    exact, y within 1e-3 relative L2 per row, x_{l+1} the bf16 of the GPU's
    own y_l + noise bit for bit)."""

import numpy as np
import pytest

from tests import gpu_util as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from bit_moe_expert_02_amd import _lib as L          # noqa: E402
from bit_moe_expert_02_amd import layer as LY        # noqa: E402
from bit_moe_expert_02_amd import offload as OFL     # noqa: E402
from bit_moe_expert_02_amd import synth              # noqa: E402
from oracle import moe as OM                         # noqa: E402


def _say(*a):
    print(*a, flush=True)


def _ffn(dl, xbits, idx, w, rows, flags=0):
    wl = dl.wl
    d = L.dims(wl.hidden, wl.inter, wl.n_experts, wl.top_k, flags)
    ws = LY.workspace(d, rows)
    y = torch.zeros((rows, wl.hidden), dtype=torch.float32, device="cuda")
    L.moe_expert_ffn(d, G.device_inputs(wl, 0, xbits), rows, torch.from_numpy(idx).cuda(),
                     torch.from_numpy(w).cuda(), dl.weights, dl.experts, dl.shared, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _oracle_skipping(wl, dl, xbits, idx, w):
    """The oracle with every -1 pair given weight 0 on expert 0 (0 * a finite
    output adds exactly nothing)."""
    idx2 = np.where(idx < 0, 0, idx)
    w2 = np.where(idx < 0, 0.0, w.astype(np.float64))
    x = OM.bf16_to_f64(xbits)
    shared = G.oracle_expert(wl, 0, wl.n_experts) if wl.shared_fmt else None
    return OM.combine(x, idx2, w2, lambda e: G.oracle_expert(wl, 0, e), shared)


@pytest.mark.parametrize("rows", [4, 8, 12])
def test_skipped_pairs_add_nothing(rows):
    wl = synth.Workload("tiny_skip", 40, 512, 256, 16, 2, "MIX", "Q8", rows=(rows,))
    xbits = synth.x_bf16(wl, 0, rows)
    idx, w = synth.zipf_routing(wl, 0, rows)
    idx = idx.copy()
    idx[::2, 1] = -1                       # every other row serves its second pair elsewhere
    idx[rows - 1, :] = -1                  # one row with no routed pair at all
    _say(f"skip: {rows} rows ({'decode' if rows <= 8 else 'many-row'} path), idx\n{idx}")
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    y = _ffn(dl, xbits, idx, w, rows)
    ref = _oracle_skipping(wl, dl, xbits, idx, w)
    err = G.rel_l2_rows(y, ref)
    _say("  rel L2 per row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)


def test_invalid_id_poisons_only_its_row():
    wl = synth.Workload("tiny_badid", 41, 512, 256, 16, 2, "Q2_0", None, rows=(4,))
    rows = 4
    xbits = synth.x_bf16(wl, 0, rows)
    idx, w = synth.zipf_routing(wl, 0, rows)
    idx = idx.copy()
    idx[1, 0] = wl.n_experts               # past the table
    idx[2, 1] = -5
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    y = _ffn(dl, xbits, idx, w, rows)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))
    good = [0, 3]
    ref = _oracle_skipping(wl, dl, xbits[good], idx[good], w[good])
    err = G.rel_l2_rows(y[good], ref)
    _say("  rel L2 of the valid rows", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)


def _tiny_offload_stack(wl, n_slots, share):
    H, I, E = wl.hidden, wl.inter, wl.n_experts
    fmts = [synth.format_map(wl, li) for li in range(wl.layers)]

    def fill(li, e, dst):
        f = fmts[li][e]
        g, u, d = synth.expert_weights(wl, li, e)
        g0, u0, d0, _ = OFL.blob_layout(f, H, I)
        for o, m in zip((g0, u0, d0), (g, u, d)):
            b = L.pack(f, m)
            dst[o:o + b.size] = b

    shared = []
    for li in range(wl.layers):
        g, u, d = synth.expert_weights(wl, li, E)
        shared.append((wl.shared_fmt, L.pack(wl.shared_fmt, g), L.pack(wl.shared_fmt, u),
                       L.pack(wl.shared_fmt, d)))
    routers = [torch.from_numpy(synth.router(wl, li)).cuda() for li in range(wl.layers)]
    biases = [None if synth.bias(wl, li) is None else torch.from_numpy(synth.bias(wl, li)).cuda()
              for li in range(wl.layers)]
    return OFL.OffloadStack(H, I, E, wl.top_k, routers, biases, shared, fmts, fill, n_slots,
                            copy_share=share, cpu_threads=4)


@pytest.mark.parametrize("share,n_slots", [(0.0, 5), (0.5, 5), (1.0, 5), (1.0, 48)])
@pytest.mark.parametrize("rows", [1, 7])
def test_offloaded_tiny_stack_teacher_forced(share, n_slots, rows):
    """Two passes over the same x: with 48 slots (more than a pass touches)
    the second pass hits every expert; with 5 slots experts are evicted
    within a pass and misses beyond the slots fall back to the CPU."""
    wl = synth.WORKLOADS["tiny_stack"]
    st = _tiny_offload_stack(wl, n_slots=n_slots, share=share)
    noise_np = np.stack([synth.noise(wl, li, rows) for li in range(wl.layers)])
    noise = torch.from_numpy(noise_np).cuda()
    try:
        for rep in range(2):
            x0 = torch.from_numpy(synth.x_bf16(wl, 0, rows, 60).view(np.int16).copy()).cuda()
            x_all, y_all, idx_all = st.decode(x0, rows, noise)
            torch.cuda.synchronize()
            xa = x_all.cpu().numpy().view(np.uint16)
            ya = y_all.cpu().numpy()
            ia = idx_all.cpu().numpy()
            _say(f"offload share {share} rows {rows} pass {rep}: {st.stats}")
            for li in range(wl.layers):
                x, idx, w, logits, gap = G.oracle_route(wl, li, xa[li])
                assert np.array_equal(ia[li], idx), (li, ia[li], idx)
                ref = G.oracle_y(wl, li, x, idx, w, list(range(rows)))
                err = G.rel_l2_rows(ya[li], ref)
                assert np.all(err <= G.REL_L2_TOL), (li, err)
                nxt = OM.chain_next(ya[li], noise_np[li])
                assert np.array_equal(OM.bf16_to_f64(xa[li + 1]), nxt), li
        s = st.stats
        if share == 0.0:
            assert s["copies"] == 0 and s["hits"] == 0 and s["cpu"] > 0
        if share == 1.0 and n_slots == 48:
            assert s["cpu"] == 0 and s["hits"] == s["copies"] > 0   # pass 2 hits all of pass 1's
        if share == 0.5:
            assert s["copies"] > 0 and s["cpu"] > 0
    finally:
        st.close()
