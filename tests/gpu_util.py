"""Helpers for the GPU parity tests: oracle references built from the seeded
inputs, device layers built with the library's packer, and comparisons.

The oracle never sees anything the HIP path produced: it packs and decodes the
same seeded fp32 weights with its own code, and routes the same bf16 x."""

import numpy as np

from bit_moe_expert_02_amd import _lib as L
from bit_moe_expert_02_amd import layer as LY
from bit_moe_expert_02_amd import synth
from oracle import formats as OF
from oracle import moe as OM

REL_L2_TOL = 1e-3     # per row, against the fp64 oracle
W_RTOL = 1e-6         # mixing weights (fp32 on the device)
NEAR_TIE = 1e-9       # relative key gap below which an index mismatch would be a tie


def oracle_expert(wl, layer, e):
    """Decoded fp64 (gate, up, down) of routed expert e, or the shared one (e == n_experts)."""
    fmt = wl.shared_fmt if e == wl.n_experts else synth.format_map(wl, layer)[e]
    g, u, d = synth.expert_weights(wl, layer, e)
    return (OF.decode(fmt, OF.pack(fmt, g), wl.inter, wl.hidden),
            OF.decode(fmt, OF.pack(fmt, u), wl.inter, wl.hidden),
            OF.decode(fmt, OF.pack(fmt, d), wl.hidden, wl.inter))


def oracle_route(wl, layer, xbits):
    x = OM.bf16_to_f64(xbits)
    idx, w, logits, gap = OM.route(x, synth.router(wl, layer), wl.top_k, synth.bias(wl, layer))
    return x, idx, w, logits, gap


def oracle_y(wl, layer, x, idx, w, rows):
    """Oracle y for the given rows (list of row numbers)."""
    cache = {}

    def ex(e):
        if e not in cache:
            cache[e] = oracle_expert(wl, layer, e)
        return cache[e]

    shared = ex(wl.n_experts) if wl.shared_fmt is not None else None
    return OM.combine(x[rows], idx[rows], w[rows], ex, shared)


def rel_l2_rows(got, ref):
    got = np.asarray(got, np.float64)
    return np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)


def device_inputs(wl, layer, xbits):
    import torch
    x = torch.from_numpy(xbits.view(np.int16).copy()).cuda()
    return x


def run_layer(dl, x, rows):
    import torch
    ws = LY.workspace(dl.dims, rows)
    idx = torch.zeros((rows, dl.wl.top_k), dtype=torch.int32, device="cuda")
    wts = torch.zeros((rows, dl.wl.top_k), dtype=torch.float32, device="cuda")
    y = torch.zeros((rows, dl.wl.hidden), dtype=torch.float32, device="cuda")
    L.moe_layer(dl.dims, x, rows, dl.router, dl.bias, dl.weights, dl.experts, dl.shared,
                idx, wts, y, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wts.cpu().numpy(), y.cpu().numpy(), ws


def check_routing(idx_gpu, w_gpu, idx_ref, w_ref, gap, logits):
    scale = np.max(np.abs(logits), axis=1)
    assert np.all(gap > NEAR_TIE * scale), "near-tie in the selection keys: inputs are ambiguous"
    assert np.array_equal(idx_gpu, idx_ref)
    np.testing.assert_allclose(w_gpu, w_ref, rtol=W_RTOL, atol=0)


def oracle_y_for(dl, x, idx, w, rows):
    """Oracle y for the given rows of a device layer whose routed slots may come
    from a pool: each slot's weights are regenerated from dl.source."""
    wl = dl.wl
    cache = {}

    def ex(e):
        if e not in cache:
            if e == wl.n_experts:
                cache[e] = oracle_expert(wl, dl.layer, e)
            else:
                src = dl.source[e]
                assert src is not None, f"slot {e} of layer {dl.layer} holds no weights"
                fmt = dl.fmts[e]
                g, u, d = synth.expert_weights(wl, src[0], src[1])
                cache[e] = (OF.decode(fmt, OF.pack(fmt, g), wl.inter, wl.hidden),
                            OF.decode(fmt, OF.pack(fmt, u), wl.inter, wl.hidden),
                            OF.decode(fmt, OF.pack(fmt, d), wl.hidden, wl.inter))
        return cache[e]

    shared = ex(wl.n_experts) if wl.shared_fmt is not None else None
    return OM.combine(x[rows], idx[rows], w[rows], ex, shared)


# ----------------------------------------------------------------------------
# Every row of a real-shape layer: experts regenerated, packed and run through
# the oracle in parallel worker processes (fresh interpreters: none of them
# touches the GPU).
# ----------------------------------------------------------------------------
def n_workers():
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _expert_job(job):
    """One expert, from its seed: (moe_pack bytes for the device or None, the
    oracle's expert output for the given rows or None).  The two come from the
    same fp32 weights through independent code: the library's packer for the
    device, the oracle's own packer and decoder for the reference."""
    wl, src_layer, src_expert, fmt, x_rows, pack_for_device = job
    g, u, d = synth.expert_weights(wl, src_layer, src_expert)
    dev = (L.pack(fmt, g), L.pack(fmt, u), L.pack(fmt, d)) if pack_for_device else None
    o = None
    if x_rows is not None and len(x_rows):
        mats = (OF.decode(fmt, OF.pack(fmt, g), wl.inter, wl.hidden),
                OF.decode(fmt, OF.pack(fmt, u), wl.inter, wl.hidden),
                OF.decode(fmt, OF.pack(fmt, d), wl.hidden, wl.inter))
        o = OM.expert_ffn(x_rows, *mats)
    return dev, o


def run_jobs(jobs, label):
    """Runs _expert_job over the jobs in a pool of spawned processes, printing
    progress; results in job order."""
    import multiprocessing as mp
    import time
    from concurrent.futures import ProcessPoolExecutor
    t0 = time.time()
    out = []
    print(f"  {label}: {len(jobs)} expert jobs on {n_workers()} processes", flush=True)
    with ProcessPoolExecutor(max_workers=n_workers(), mp_context=mp.get_context("spawn")) as ex:
        for i, r in enumerate(ex.map(_expert_job, jobs)):
            out.append(r)
            if (i + 1) % 8 == 0 or i + 1 == len(jobs):
                print(f"    {i + 1}/{len(jobs)} done ({time.time() - t0:.0f} s)", flush=True)
    return out


def materialized_layer_and_oracle(wl, layer, x, idx, w, xin_for=None, flags=0):
    """A device layer holding exactly the experts idx selects (every other slot
    all-zero) and the oracle's y for every row.  xin_for(e) -> the activations
    expert e sees (default x); the shared expert always sees x."""
    fm = synth.format_map(wl, layer)
    experts = sorted(set(int(v) for v in np.asarray(idx).reshape(-1)))
    jobs = []
    for e in experts:
        rows, _ = np.nonzero(idx == e)
        xe = x if xin_for is None else xin_for(e)
        jobs.append((wl, layer, e, fm[e], xe[rows], True))
    if wl.shared_fmt is not None:
        jobs.append((wl, layer, wl.n_experts, wl.shared_fmt, x, True))
    res = run_jobs(jobs, f"{wl.name} layer {layer}")
    packed = {e: r[0] for e, r in zip(experts, res)}
    outs = {e: r[1] for e, r in zip(experts, res)}
    shared_out = None
    if wl.shared_fmt is not None:
        packed[wl.n_experts] = res[-1][0]
        shared_out = res[-1][1]
    dl = LY.DeviceLayer(wl, layer, packed=packed, flags=flags)
    y = OM.combine_outputs(x.shape, idx, w, outs, shared_out)
    return dl, y


def oracle_y_parallel(dl, x, idx, w):
    """The oracle's y for every row of x on a device layer whose slots may come
    from a pool (weights regenerated from dl.source)."""
    wl = dl.wl
    experts = sorted(set(int(v) for v in np.asarray(idx).reshape(-1)))
    jobs = []
    for e in experts:
        src = dl.source[e]
        assert src is not None, f"slot {e} of layer {dl.layer} holds no weights"
        rows, _ = np.nonzero(idx == e)
        jobs.append((wl, src[0], src[1], dl.fmts[e], x[rows], False))
    if wl.shared_fmt is not None:
        jobs.append((wl, dl.layer, wl.n_experts, wl.shared_fmt, x, False))
    res = run_jobs(jobs, f"{wl.name} layer {dl.layer} oracle")
    outs = {e: r[1] for e, r in zip(experts, res)}
    shared_out = res[-1][1] if wl.shared_fmt is not None else None
    return OM.combine_outputs(x.shape, idx, w, outs, shared_out)


def fmt_err(err):
    """Per-row errors in scientific notation (a fixed-point print would round
    the real margins to zero)."""
    return "[" + ", ".join(f"{v:.2e}" for v in np.asarray(err).reshape(-1)) + "]"
