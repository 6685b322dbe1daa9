#!/usr/bin/env python3
"""Benchmark: MoE-layer decode tokens/s and achieved HBM GB/s on one MI355X.

One step = one full pass of the layer's hot path through the C ABI (moe_layer:
router GEMV + top-6 with the selection-only bias, shared-expert gate/up,
routed gate/up + SwiGLU, down + combine) over one batch of rows, on the
mixed-format verify layer: hidden 5120, intermediate 2304, 384 routed experts
(164 ternary / 151 Q2_0 / 69 Q3), top-6, an int8 shared expert, a bias
U(-0.6, 1.0).  The headline is rows 1; rows 5 and 8 (verify windows) are
timed beside it, and the same series runs on the all-Q2_0 layer and on one
MXFP4 layer of the FP4 stack (no shared expert).

Inputs are synthetic and seeded, and resident in HBM before timing starts.
Each timed step uses a different copy of the layer (8 copies of a 3.85 GB
layer, 4 of the 7.2 GB FP4 layer, so neither the 256 MB Infinity Cache nor the
L2s can serve a step from a previous one) and a fresh activation batch.
Routed slots are filled from a pool of distinct packed experts per format
(bandwidth does not depend on the values).

Other workloads print their own line (--workload): the 40-layer mixed stack,
the 20-layer FP4 stack, the FP4 prefill layer, verify windows of correlated
rows on the mixed stack, the mixed stack under the residency-style bias
policy, and the draft model's 128-expert top-3 layer.

Prints one JSON line (fields described in the repository's design notes).
"""

import argparse
import ctypes
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
METRIC = "MoE-layer decode tokens/s + achieved HBM GB/s (% of peak), rows=1..8"
NEV = 2                       # events per layer pass: before and after its one launch
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--rows", type=int, default=1, help="headline row count")
    p.add_argument("--copies", type=int, default=8)
    p.add_argument("--pool", type=int, default=16)
    p.add_argument("--sweep", default="1,5,8", help="row counts timed beside the headline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="headline workload only (no decode_q2 / fp4_layer series)")
    p.add_argument("--cpu-rows", type=int, default=1)
    p.add_argument("--workload", default="mixed_verify",
                   choices=["mixed_verify", "decode_q2", "fp4_layer", "draft128", "stack40_mixed",
                            "fp4_stack20", "fp4_prefill", "verify_correlated", "policy_stack40",
                            "alloc_stack40", "offload_fp4"])
    p.add_argument("--offload-layers", type=int, default=4,
                   help="offload_fp4: FP4 layers whose routed experts live in pinned host memory")
    p.add_argument("--offload-slots", type=int, default=384,
                   help="offload_fp4: device expert slots (default: one layer's worth)")
    p.add_argument("--offload-share", type=float, default=-1.0,
                   help="offload_fp4: share of misses copied; negative: measured (moe_copy_share)")
    p.add_argument("--stack-rows", default="",
                   help="stack workloads: row counts to time (default: the workload's own)")
    p.add_argument("--copy-calib-mb", type=int, default=0,
                   help="run one device copy of this many MiB first (a known-size reference "
                        "for hardware byte counters)")
    return p.parse_args()


def say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def ms(self, a, b):
        v = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(v), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return float(v.value)

    def record(self, e, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def measured_traffic(name):
    """HBM bytes per launch from a committed counter record (profiles/traffic_<name>.json),
    or None when it is missing or the kernel sources changed since it was taken."""
    from bit_moe_expert_02_amd import profile_summary
    try:
        with open(os.path.join(PROFILES, f"traffic_{name}.json")) as f:
            d = json.load(f)
    except OSError:
        return None
    if d.get("source_sha256") != profile_summary.source_hash():
        return None
    return int(d["traffic_bytes_per_launch"])


def expert_bytes(wl, fmt):
    from bit_moe_expert_02_amd import _lib as L
    return 2 * L.packed_bytes(fmt, wl.inter, wl.hidden) + L.packed_bytes(fmt, wl.hidden, wl.inter)


def layer_bytes(wl, fmts_unique, rows):
    """Algorithmic bytes of one pass: router + distinct selected experts + shared + x/y."""
    router = 4 * wl.n_experts * wl.hidden
    routed = sum(expert_bytes(wl, f) for f in fmts_unique)
    shared = expert_bytes(wl, wl.shared_fmt) if wl.shared_fmt else 0
    return router + routed + shared + rows * wl.hidden * (2 + 4)


def build_copies(wl, copies, pool_n):
    from bit_moe_expert_02_amd import layer as LY
    from bit_moe_expert_02_amd import synth
    fmts = sorted(set(synth.format_map(wl, 0)))
    pool = LY.make_pool(wl, 0, fmts, pool_n)
    out = []
    for c in range(copies):
        out.append(LY.DeviceLayer(wl, c, materialize=(), pool=pool))
    return out


def run_steps(torch, L, LY, layers, xs, rows, steps, warmup, events=None, hev=None):
    """warmup + steps layer passes, rotating the layer copies; returns (seconds,
    per-step launch ms or None, idx of the timed steps)."""
    wl = layers[0].wl
    ws = LY.workspace(layers[0].dims, rows)
    idx = torch.zeros((steps + warmup, rows, wl.top_k), dtype=torch.int32, device="cuda")
    wts = torch.zeros((steps + warmup, rows, wl.top_k), dtype=torch.float32, device="cuda")
    y = torch.zeros((rows, wl.hidden), dtype=torch.float32, device="cuda")
    evs = hev.create(NEV * steps) if events else None

    def one(i, timed_slot=None):
        dl = layers[i % len(layers)]
        if timed_slot is None:
            L.moe_layer(dl.dims, xs[i], rows, dl.router, dl.bias, dl.weights, dl.experts,
                        dl.shared, idx[i], wts[i], y, ws)
        else:
            L.moe_layer_profiled(dl.dims, xs[i], rows, dl.router, dl.bias, dl.weights,
                                 dl.experts, dl.shared, idx[i], wts[i], y, ws,
                                 evs[NEV * timed_slot: NEV * timed_slot + NEV])

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        one(warmup + s, s if events else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert L.moe_workspace_status(ws) == L.MOE_OK, "a hand-off wait of the fused launch gave up"
    per = None
    if events:
        per = np.array([hev.ms(evs[NEV * s], evs[NEV * s + 1]) for s in range(steps)])
        hev.destroy(evs)
    return t1 - t0, per, idx[warmup:].cpu().numpy()


def decode_series(torch, L, LY, synth, hev, wl, layers, rows_list, steps, warmup, x_for=None):
    """Per row count: wall-clock step time, per-launch event times, distinct
    experts and algorithmic bytes per step."""
    res = {}
    fm = layers[0].fmts
    for rows in rows_list:
        n = steps + warmup
        xs = [torch.from_numpy((x_for(rows, i) if x_for else synth.x_bf16(wl, 0, rows, 10_000 * rows + i))
                               .view(np.int16).copy()).cuda() for i in range(n)]
        secs, _, idx = run_steps(torch, L, LY, layers, xs, rows, steps, warmup)
        _, per, _ = run_steps(torch, L, LY, layers, xs, rows, steps, warmup, events=True, hev=hev)
        uniq = [np.unique(i) for i in idx]
        by = np.array([layer_bytes(wl, [fm[e] for e in u], rows) for u in uniq], np.float64)
        launch_ms = float(per.mean())
        res[rows] = dict(secs=secs, per=per, uniq=float(np.mean([len(u) for u in uniq])),
                         bytes=float(by.mean()), launch_ms=launch_ms)
        say(f"{wl.name} rows {rows}: {secs / steps * 1e6:.1f} us/step, launch {launch_ms * 1e3:.2f} us, "
            f"{np.mean([len(u) for u in uniq]):.1f} experts, {by.mean() / (launch_ms * 1e-3) / 1e9:.0f} GB/s")
    return res


def series_json(res, steps):
    out = {}
    for k, v in res.items():
        ach = v["bytes"] / (v["launch_ms"] * 1e-3) / 1e9
        out[str(k)] = {"tokens_per_s": round(k * steps / v["secs"], 1),
                       "us_per_step": round(v["secs"] / steps * 1e6, 2),
                       "kernel_us": round(v["launch_ms"] * 1e3, 3),
                       "kernel_us_p10_p50_p90": [round(float(q) * 1e3, 3)
                                                 for q in np.percentile(v["per"], [10, 50, 90])],
                       "unique_experts": round(v["uniq"], 2),
                       "bytes_per_step": int(v["bytes"]),
                       "layer_GBps": round(v["bytes"] / (v["secs"] / steps) / 1e9, 1),
                       "kernel_GBps": round(ach, 1),
                       "frac_of_hbm_peak": round(ach / HBM_PEAK_GBPS, 4)}
    return out


def stream_read_ceiling(torch, L):
    """The device's streaming-read rate (GB/s): the best of a few launch
    shapes of the library's plain read kernel over 4 GiB, timed with events."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = 0.0
    for grid, unroll in ((1024, 2), (2048, 4), (4096, 8), (8192, 8)):
        sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        for _ in range(3):
            L.moe_stream_read(buf, nbytes, sink, grid, unroll)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        n = 10
        for _ in range(n):
            L.moe_stream_read(buf, nbytes, sink, grid, unroll)
        b.record()
        b.synchronize()
        best = max(best, nbytes * n / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return best


# ----------------------------------------------------------------------------- oracle baseline
def _oracle_layer_time(wl, layer, xbits, limit):
    """Seconds the oracle takes for one layer on the given rows (BLAS threads
    capped at `limit`): route, then decode and run every selected expert and
    the shared expert in fp64."""
    from threadpoolctl import threadpool_limits

    from bit_moe_expert_02_amd import synth
    from oracle import formats as OF
    from oracle import moe as OM

    fm = synth.format_map(wl, layer)

    def expert(e):
        f = wl.shared_fmt if e == wl.n_experts else fm[e]
        g, u, d = synth.expert_weights(wl, layer, e)
        return (OF.decode(f, OF.pack(f, g), wl.inter, wl.hidden), OF.decode(f, OF.pack(f, u), wl.inter, wl.hidden),
                OF.decode(f, OF.pack(f, d), wl.hidden, wl.inter))

    with threadpool_limits(limits=limit):
        t0 = time.perf_counter()
        x = OM.bf16_to_f64(xbits)
        OM.moe_layer(x, synth.router(wl, layer), wl.top_k, expert,
                     shared=expert(wl.n_experts) if wl.shared_fmt else None, bias=synth.bias(wl, layer))
        return time.perf_counter() - t0


def cpu_baseline(wl, rows, layers_in_pass=1, label=None):
    """The oracle, as it stands, on `rows` row(s) of one layer: BLAS on one
    thread, then on every allowed core.  For a stack the one layer's time is
    multiplied by the layers in a pass (an extrapolation, said so)."""
    from bit_moe_expert_02_amd import synth
    xbits = synth.x_bf16(wl, 0, rows, 999)
    t1 = _oracle_layer_time(wl, 0, xbits, 1)
    ncores = len(os.sched_getaffinity(0))
    tn = _oracle_layer_time(wl, 0, xbits, ncores)
    what = label or f"{rows} row(s) of one {wl.name} layer"
    sample = (f"{what}: route + decode of the selected experts and the shared expert + fp64 math, "
              f"{t1:.2f} s with BLAS on 1 thread")
    if layers_in_pass > 1:
        sample += f"; x{layers_in_pass} layers per pass (extrapolated from one layer)"
    return dict(value=round(rows / (t1 * layers_in_pass), 5), unit="tokens/s", cores=1, kind="oracle",
                sample=sample, all_cores=dict(value=round(rows / (tn * layers_in_pass), 5), cores=ncores,
                                              seconds=round(tn, 2)))


# ----------------------------------------------------------------------------- single-layer decode
WORKLOAD_TEXT = {
    "mixed_verify": "mixed_verify: hidden 5120, moe_intermediate 2304, 384 routed experts (164 ternary "
                    "TERN160 / 151 Q2_0 / 69 Q3 by seeded draw), top-6, selection bias U(-0.6,1.0), "
                    "1 shared expert int8 (per-32 fp16 scale), one layer",
    "decode_q2": "decode_q2: hidden 5120, moe_intermediate 2304, 384 routed Q2_0 experts, top-6, "
                 "1 shared expert int8 (per-32 fp16 scale), one layer",
    "fp4_layer": "fp4_layer: one layer of the FP4 stack: hidden 5120, moe_intermediate 2304, 384 MXFP4 "
                 "experts (e2m1 + per-32 e8m0), top-6, no shared expert",
    "draft128": "draft128: the draft model's MoE layer: hidden 5120, moe_intermediate 2304, 128 routed "
                "Q2_0 experts, top-3, 1 shared Q2_0 expert",
}


def single_layer(args, torch, L, LY, synth, hev, name, copies, rows_list):
    wl = synth.WORKLOADS["fp4_stack20" if name == "fp4_layer" else name]
    say(f"building {copies} layer copies of {name}")
    layers = build_copies(wl, copies, args.pool)
    torch.cuda.synchronize()
    res = decode_series(torch, L, LY, synth, hev, wl, layers, rows_list, args.steps, args.warmup)
    del layers
    torch.cuda.empty_cache()
    return wl, res


def main_decode(args, torch, L, LY, synth):
    hev = HipEvents()
    name = args.workload
    sweep = sorted(set([args.rows] + [int(r) for r in args.sweep.split(",") if r]))
    if name == "draft128":
        sweep = sorted(set([args.rows, 1, 5]))
    copies = 4 if name == "fp4_layer" else args.copies
    wl, res = single_layer(args, torch, L, LY, synth, hev, name, copies, sweep)
    extra = {}
    if name == "mixed_verify" and not args.no_extra:
        for sub, cp, rl in (("decode_q2", args.copies, [1, 8]), ("fp4_layer", 4, [1, 8])):
            swl, sres = single_layer(args, torch, L, LY, synth, hev, sub, cp, rl)
            extra[sub] = {"workload": WORKLOAD_TEXT[sub], "rows": series_json(sres, args.steps)}
    ceiling = stream_read_ceiling(torch, L)
    say(f"streaming-read ceiling {ceiling:.0f} GB/s")
    r = res[args.rows]
    ms_step = r["secs"] / args.steps * 1e3
    value = args.rows * args.steps / r["secs"]
    achieved = r["bytes"] / (r["launch_ms"] * 1e-3) / 1e9
    layer_gbps = r["bytes"] / (ms_step * 1e-3) / 1e9
    traffic_name = f"k_layer_{name}_rows{args.rows}"
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "low-bit codes (ternary/2-bit/3-bit/int8/e2m1) x f16 -> f32, router f64",
        "data": "synthetic (seeded N(0,0.02) weights packed RTN, bf16 N(0,1) rows; routed slots from a "
                "pool of distinct packed experts per format)",
        "config": {
            "workload": WORKLOAD_TEXT[name],
            "rows": args.rows,
            "layer_copies_rotated": copies,
            "layer_bytes_per_step": int(r["bytes"]),
            "layer_GBps": round(layer_gbps, 1),
            "layer_frac_of_hbm_peak": round(layer_gbps / HBM_PEAK_GBPS, 4),
            "stream_read_ceiling_GBps": round(ceiling, 1),
            "layer_frac_of_stream_ceiling": round(layer_gbps / ceiling, 4),
            "rows_sweep": series_json(res, args.steps),
            "expert_bytes": {f: expert_bytes(wl, f) for f in sorted(set(layers_fmts(synth, wl)))},
            **({"other_layers": extra} if extra else {}),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(traffic_name),
            "kernel": "k_layer (the whole layer in one launch)",
            "bytes_per_launch": int(r["bytes"]),
            "avg_launch_us": round(r["launch_ms"] * 1e3, 3),
            "stream_ceiling": round(ceiling, 1),
            "frac_of_stream_ceiling": round(achieved / ceiling, 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        say("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    print(json.dumps(out), flush=True)


def layers_fmts(synth, wl):
    f = list(synth.format_map(wl, 0))
    return f + ([wl.shared_fmt] if wl.shared_fmt else [])


# ----------------------------------------------------------------------------- FP4 prefill layer
def bench_prefill(args, torch, L, LY, synth):
    """One FP4 layer at the prefill shape: 2048 Zipf-routed rows through
    moe_expert_ffn with MOE_ACT_MXFP8 (MXFP8 x MXFP4 gate/up and f16 x MXFP4
    down on the matrix cores)."""
    wl = synth.WORKLOADS["fp4_stack20"]
    R = 2048
    copies = 2
    pool = LY.make_pool(wl, 0, ["MXFP4"], args.pool)
    layers = [LY.DeviceLayer(wl, c, materialize=(), pool=pool, flags=L.MOE_ACT_MXFP8) for c in range(copies)]
    idx, w = synth.zipf_routing(wl, 0, R)
    used = np.unique(idx)
    wbytes = len(used) * expert_bytes(wl, "MXFP4")
    flops = 2.0 * 3 * wl.hidden * wl.inter * R * wl.top_k
    xs = [torch.from_numpy(synth.x_bf16(wl, 0, R, 900 + i).view(np.int16).copy()).cuda() for i in range(2)]
    it, wt = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    y = torch.zeros((R, wl.hidden), dtype=torch.float32, device="cuda")
    ws = LY.workspace(layers[0].dims, R)
    hev = HipEvents()
    ev = hev.create(2)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        dl = layers[i % copies]
        L.moe_expert_ffn(dl.dims, xs[i % 2], R, it, wt, dl.weights, dl.experts, None, y, ws)
    torch.cuda.synchronize()
    times = []
    for i in range(args.steps):
        dl = layers[i % copies]
        hev.record(ev[0], stream)
        L.moe_expert_ffn(dl.dims, xs[i % 2], R, it, wt, dl.weights, dl.experts, None, y, ws)
        hev.record(ev[1], stream)
        torch.cuda.synchronize()
        times.append(hev.ms(ev[0], ev[1]))
    hev.destroy(ev)
    ms = float(np.median(times))
    gbps = wbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    say(f"fp4 prefill {R} rows: {ms:.3f} ms/layer, {gbps:.0f} GB/s of expert weights, {tflops:.0f} TFLOP/s")
    line = {
        "metric": "FP4 prefill-layer tokens/s (2048 Zipf-routed rows, MXFP4 experts on the matrix cores)",
        "value": round(R / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8 x mxfp4 (gate/up), f16 x mxfp4 (down) -> f32",
        "data": "synthetic (seeded; Zipf s=1.1 routing; experts filled from a pool of distinct packed experts)",
        "config": {"workload": "fp4 prefill: hidden 5120, moe_intermediate 2304, 384 MXFP4 experts, "
                               "top-6, 2048 rows", "experts_touched": int(len(used)),
                   "weight_bytes": int(wbytes), "flop": flops, "TFLOPs": round(tflops, 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": sum_or_none([measured_traffic("k_gateup_prefill_fp4_rows2048"),
                                             measured_traffic("k_down_prefill_fp4_rows2048")]),
                     "kernel": "whole prefill call (quant, dispatch, gate/up, down, combine); traffic: "
                               "k_gateup + k_down"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        say("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline_prefill(wl, idx, w)
    print(json.dumps(line), flush=True)


def sum_or_none(vals):
    return None if any(v is None for v in vals) else int(sum(vals))


def cpu_baseline_prefill(wl, idx, w, rows=1):
    """The oracle's prefill layer on the first `rows` row(s) of the routing."""
    from threadpoolctl import threadpool_limits

    from bit_moe_expert_02_amd import synth
    from oracle import formats as OF
    from oracle import moe as OM

    def expert(e):
        g, u, d = synth.expert_weights(wl, 0, e)
        return (OF.decode("MXFP4", OF.pack("MXFP4", g), wl.inter, wl.hidden),
                OF.decode("MXFP4", OF.pack("MXFP4", u), wl.inter, wl.hidden),
                OF.decode("MXFP4", OF.pack("MXFP4", d), wl.hidden, wl.inter))

    xbits = synth.x_bf16(wl, 0, rows, 900)
    res = {}
    for limit in (1, len(os.sched_getaffinity(0))):
        with threadpool_limits(limits=limit):
            t0 = time.perf_counter()
            OM.prefill_layer(OM.bf16_to_f64(xbits), idx[:rows], w[:rows].astype(np.float64), expert)
            res[limit] = time.perf_counter() - t0
    n = max(res)
    return dict(value=round(rows / res[1], 5), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{rows} row(s) of the 2048-row FP4 prefill layer (MXFP8 x, {wl.top_k} MXFP4 experts "
                       f"decoded in fp64), {res[1]:.2f} s with BLAS on 1 thread",
                all_cores=dict(value=round(rows / res[n], 5), cores=n, seconds=round(res[n], 2)))


# ----------------------------------------------------------------------------- stacks
def build_stack(args, torch, LY, synth, wl, pool_layer=0):
    fmts = sorted({f for l in range(wl.layers) for f in synth.format_map(wl, l)})
    say(f"building {wl.layers} layers of {wl.name} (pool of {args.pool} per format)")
    pool = LY.make_pool(wl, pool_layer, fmts, args.pool)
    layers = []
    for l in range(wl.layers):
        layers.append(LY.DeviceLayer(wl, l, materialize=(), pool=pool))
        if l % 10 == 9:
            say(f"  {l + 1} layers resident")
    torch.cuda.synchronize()
    return layers


def stack_passes(args, torch, L, LY, synth, hev, wl, layers, rows, x0_for, noise):
    """Times whole chained passes (moe_stack_decode, one launch per layer);
    returns (mean ms per pass, mean algorithmic bytes, mean distinct experts
    per layer, per-pass ms list)."""
    H, k, n = wl.hidden, wl.top_k, wl.layers
    lw = L.layer_weights(layers)
    x_all = torch.zeros((n + 1, rows, H), dtype=torch.int16, device="cuda")
    noise_d = torch.from_numpy(noise).cuda()
    y_all = torch.zeros((n, rows, H), dtype=torch.float32, device="cuda")
    idx_all = torch.zeros((n, rows, k), dtype=torch.int32, device="cuda")
    ws = LY.workspace(layers[0].dims, rows)
    x0 = [torch.from_numpy(x0_for(i).view(np.int16).copy()).cuda() for i in range(args.steps + args.warmup)]
    ev = hev.create(2)
    stream = torch.cuda.current_stream().cuda_stream
    times, byts, uniq = [], [], []
    for i in range(args.steps + args.warmup):
        x_all[0].copy_(x0[i])
        if i >= args.warmup:
            hev.record(ev[0], stream)
        L.moe_stack_decode(layers[0].dims, lw, rows, x_all, noise_d, y_all, idx_all, None, ws)
        if i >= args.warmup:
            hev.record(ev[1], stream)
            torch.cuda.synchronize()
            times.append(hev.ms(ev[0], ev[1]))
            ids = idx_all.cpu().numpy()
            b, u = 0, 0
            for l in range(n):
                ue = np.unique(ids[l])
                b += layer_bytes(wl, [layers[l].fmts[e] for e in ue], rows)
                u += len(ue)
            byts.append(b)
            uniq.append(u / n)
    hev.destroy(ev)
    assert L.moe_workspace_status(ws) == L.MOE_OK, "a hand-off wait of the fused launch gave up"
    return float(np.mean(times)), float(np.mean(byts)), float(np.mean(uniq)), times


def stack_line(args, wl, out_rows, metric, extra_cfg=None, cpu=None, traffic=None):
    r0 = min(out_rows)
    return {
        "metric": metric,
        "value": out_rows[r0]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": out_rows[r0]["ms_per_pass"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "low-bit codes x f16 -> f32 (router f64)",
        "data": "synthetic (seeded; routed slots filled from a pool of distinct packed experts)",
        "config": {"workload": wl.name, "layers": wl.layers, "rows": out_rows, **(extra_cfg or {})},
        "roofline": {"bound": "hbm", "achieved": out_rows[r0]["GBps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": out_rows[r0]["frac_of_hbm_peak"], "traffic": traffic,
                     "kernel": "whole pass (one fused launch per layer)"},
        "cpu_baseline": cpu,
    }


def bench_stack(args, torch, L, LY, synth):
    """Chained decode passes through a whole stack (every layer resident in HBM)."""
    wl = synth.WORKLOADS[args.workload]
    layers = build_stack(args, torch, LY, synth, wl)
    hev = HipEvents()
    out_rows = {}
    row_counts = [int(r) for r in args.stack_rows.split(",")] if args.stack_rows else wl.rows
    for rows in [r for r in row_counts if 1 <= r <= 8]:
        noise = np.stack([synth.noise(wl, l, rows) for l in range(wl.layers)])
        ms, b, u, _ = stack_passes(args, torch, L, LY, synth, hev, wl, layers, rows,
                                   lambda i: synth.x_bf16(wl, 0, rows, 50_000 + i), noise)
        gbps = b / (ms * 1e-3) / 1e9
        out_rows[rows] = dict(ms_per_pass=round(ms, 4), tokens_per_s=round(rows / (ms * 1e-3), 2),
                              pass_bytes=int(b), unique_experts_per_layer=round(u, 2), GBps=round(gbps, 1),
                              frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4))
        say(f"{wl.name} rows {rows}: {ms:.3f} ms/pass, {gbps:.0f} GB/s, {u:.1f} experts/layer")
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, 1, wl.layers)
    traffic = measured_traffic(f"k_layer_{wl.name}_rows1")
    print(json.dumps(stack_line(args, wl, out_rows,
                                f"{wl.name} chained decode tokens/s (one pass = {wl.layers} layers)",
                                cpu=cpu, traffic=None if traffic is None else traffic * wl.layers)),
          flush=True)


# ----------------------------------------------------------------------------- verify windows
PAGES_TOKENS_PER_PASS = 3.39   # accepted tokens per verify pass ([P1 §3B])


def tune_rho(torch, L, LY, synth, wl, layer0, rows=7, target=25.2, windows=48):
    """rho of the correlated verify window at which `rows` rows select `target`
    distinct experts per layer on average (bisection, routing through moe_route
    on layer 0 of the stack)."""
    ws = LY.workspace(layer0.dims, rows)
    idx = torch.zeros((rows, wl.top_k), dtype=torch.int32, device="cuda")
    wts = torch.zeros((rows, wl.top_k), dtype=torch.float32, device="cuda")

    def mean_unique(rho):
        u = []
        for s in range(windows):
            x = torch.from_numpy(synth.correlated_x(wl, 0, rows, rho, 70_000 + s).view(np.int16).copy()).cuda()
            L.moe_route(layer0.dims, x, rows, layer0.router, layer0.bias, idx, wts, ws)
            u.append(len(np.unique(idx.cpu().numpy())))
        return float(np.mean(u))

    lo, hi = 0.0, 1.0        # unique experts fall as rho grows
    for _ in range(10):
        mid = 0.5 * (lo + hi)
        if mean_unique(mid) > target:
            lo = mid
        else:
            hi = mid
    rho = 0.5 * (lo + hi)
    return rho, mean_unique(rho)


def bench_verify_correlated(args, torch, L, LY, synth):
    """Verify windows of correlated rows on the mixed stack: pass time against
    rows, distinct experts per layer, and the fitted pass-time law."""
    base = synth.WORKLOADS["verify_correlated"]
    layers = build_stack(args, torch, LY, synth, base)
    hev = HipEvents()
    rho, u7 = tune_rho(torch, L, LY, synth, base, layers[0])
    say(f"rho {rho:.4f}: {u7:.1f} distinct experts per layer at 7 rows")
    out_rows, pts = {}, []
    for rows in range(1, 9):
        noise = np.stack([synth.correlated_noise(base, l, rows, rho) for l in range(base.layers)])
        ms, b, u, times = stack_passes(args, torch, L, LY, synth, hev, base, layers, rows,
                                       lambda i: synth.correlated_x(base, 0, rows, rho, 80_000 + i), noise)
        gbps = b / (ms * 1e-3) / 1e9
        out_rows[rows] = dict(ms_per_pass=round(ms, 4), tokens_per_s=round(rows / (ms * 1e-3), 2),
                              pass_bytes=int(b), unique_experts_per_layer=round(u, 2), GBps=round(gbps, 1),
                              frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4))
        pts.append((rows, u, ms))
        say(f"correlated rows {rows}: {ms:.3f} ms/pass, {u:.1f} experts/layer, {gbps:.0f} GB/s")
    a = np.array(pts)
    # pass ms = c0 + c1 * rows (the pages' form without its miss terms), and
    # pass ms = d0 + d1 * distinct experts per layer (what the bytes follow)
    c = np.polyfit(a[:, 0], a[:, 2], 1)
    d = np.polyfit(a[:, 1], a[:, 2], 1)
    r2 = lambda x, y, p: 1.0 - np.sum((np.polyval(p, x) - y) ** 2) / np.sum((y - y.mean()) ** 2)
    t67 = float(np.polyval(c, 6.7))
    cfg = {"rho": round(rho, 4), "unique_experts_at_7_rows": round(u7, 2),
           "law_ms": {"intercept": round(float(c[1]), 4), "per_row": round(float(c[0]), 4),
                      "r2": round(float(r2(a[:, 0], a[:, 2], c)), 4)},
           "law_ms_by_experts": {"intercept": round(float(d[1]), 4), "per_expert_per_layer": round(float(d[0]), 5),
                                 "r2": round(float(r2(a[:, 1], a[:, 2], d)), 4)},
           "pass_ms_at_6_7_rows": round(t67, 4),
           "tokens_per_s_at_3_39_accepted_per_pass": round(PAGES_TOKENS_PER_PASS / (t67 * 1e-3), 1)}
    cpu = None if args.no_cpu_baseline else cpu_baseline(base, 1, base.layers)
    line = stack_line(args, base, out_rows, "verify-window decode: pass time vs rows on the 40-layer mixed stack "
                      "(correlated rows)", extra_cfg=cfg, cpu=cpu)
    line["value"] = cfg["tokens_per_s_at_3_39_accepted_per_pass"]
    line["unit"] = "tokens/s (3.39 accepted tokens per pass at 6.7 rows)"
    print(json.dumps(line), flush=True)


def bench_policy(args, torch, L, LY, synth):
    """The mixed stack under the residency-style selection bias at scales 0,
    0.25, 0.5 and 1.0: distinct experts per layer and pass time at rows 1 and 7."""
    base = synth.WORKLOADS["policy_stack40"]
    layers = build_stack(args, torch, LY, synth, base)
    hev = HipEvents()
    per_scale = {}
    for scale in (0.0, 0.25, 0.5, 1.0):
        wl = dataclasses.replace(base, extra={"policy_scale": scale})
        for dl in layers:
            dl.bias.copy_(torch.from_numpy(synth.bias(wl, dl.layer)))
        torch.cuda.synchronize()
        rows_out = {}
        for rows in (1, 7):
            noise = np.stack([synth.noise(wl, l, rows) for l in range(wl.layers)])
            ms, b, u, _ = stack_passes(args, torch, L, LY, synth, hev, wl, layers, rows,
                                       lambda i: synth.x_bf16(wl, 0, rows, 90_000 + i), noise)
            gbps = b / (ms * 1e-3) / 1e9
            rows_out[rows] = dict(ms_per_pass=round(ms, 4), tokens_per_s=round(rows / (ms * 1e-3), 2),
                                  pass_bytes=int(b), unique_experts_per_layer=round(u, 2), GBps=round(gbps, 1),
                                  frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4))
            say(f"policy x{scale} rows {rows}: {ms:.3f} ms/pass, {u:.1f} experts/layer")
        per_scale[str(scale)] = rows_out
    cpu = None if args.no_cpu_baseline else cpu_baseline(base, 1, base.layers)
    line = stack_line(args, base, per_scale["0.5"], "policy_stack40 chained decode tokens/s (residency bias x0.5)",
                      extra_cfg={"by_scale": per_scale, "tiers_per_layer": list(synth.POLICY_TIERS),
                                 "tier_bias": list(synth.POLICY_BIAS)}, cpu=cpu)
    print(json.dumps(line), flush=True)


def bench_alloc(args, torch, L, LY, synth):
    """The mixed stack with formats chosen per expert by moe_allocate_formats
    (budget: the stack in Q2_0) from synthetic held-out errors, instead of the
    seeded draw: the allocation's cost against all-Q2_0, its format shares, and
    chained decode passes over the allocated stack."""
    base = synth.WORKLOADS["stack40_mixed"]
    err, tokens, energy = synth.alloc_inputs(base)
    nb = [expert_bytes(base, f) for f in ("TERN160", "Q2_0", "Q3")]
    t0 = time.perf_counter()
    names, cost, nbytes = L.allocate_formats(err, tokens, energy, nb)
    t_alloc = time.perf_counter() - t0
    # the same cost of the all-Q2_0 stack, for the ratio reported beside it:
    # held-out error / layer energy, the first 2 and last 3 layers doubled
    n_l = err.shape[0]
    w_l = np.array([2.0 if (li < 2 or li >= n_l - 3) else 1.0 for li in range(n_l)])
    q2_cost = float((w_l[:, None] * err[:, :, 1] / energy[:, None]).sum())
    budget = base.layers * base.n_experts * nb[1]
    shares = {f: round(float((names == f).mean()), 4) for f in ("TERN160", "Q2_0", "Q3")}
    say(f"allocation: cost {cost / q2_cost:.3f} of all-Q2_0, bytes {nbytes / budget:.5f} of budget, {shares}")
    fmts = sorted(set(names.reshape(-1)))
    pool = LY.make_pool(base, 0, fmts, args.pool)
    layers = [LY.DeviceLayer(base, l, materialize=(), pool=pool, fmts=list(names[l])) for l in range(base.layers)]
    torch.cuda.synchronize()
    hev = HipEvents()
    out_rows = {}
    for rows in (1, 7):
        noise = np.stack([synth.noise(base, l, rows) for l in range(base.layers)])
        ms, b, u, _ = stack_passes(args, torch, L, LY, synth, hev, base, layers, rows,
                                   lambda i: synth.x_bf16(base, 0, rows, 95_000 + i), noise)
        gbps = b / (ms * 1e-3) / 1e9
        out_rows[rows] = dict(ms_per_pass=round(ms, 4), tokens_per_s=round(rows / (ms * 1e-3), 2),
                              pass_bytes=int(b), unique_experts_per_layer=round(u, 2), GBps=round(gbps, 1),
                              frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4))
        say(f"allocated stack rows {rows}: {ms:.3f} ms/pass, {gbps:.0f} GB/s")
    cpu, t_oracle = None, None
    if not args.no_cpu_baseline:
        from oracle import alloc as OA
        t1 = time.perf_counter()
        OA.allocate(err, tokens, energy, nb)
        t_oracle = time.perf_counter() - t1
        cpu = cpu_baseline(base, 1, base.layers)
    cfg = {"allocation": {"cost_vs_all_q2": round(cost / q2_cost, 4), "bytes": int(nbytes), "budget": int(budget),
                          "oracle_seconds": None if t_oracle is None else round(t_oracle, 2),
                          "shares": shares, "max_ternary_share_per_layer":
                              round(float((names == "TERN160").mean(axis=1).max()), 4),
                          "library_seconds": round(t_alloc, 3)}}
    line = stack_line(args, base, out_rows, "alloc_stack40 chained decode tokens/s (per-expert allocated formats)",
                      extra_cfg=cfg, cpu=cpu)
    print(json.dumps(line), flush=True)


def bench_offload(args, torch, L, LY, synth):
    """FP4 layers of the real shape whose routed experts live in pinned host
    memory, decoded through a device slot cache that holds a fraction of them
    (default: 384 slots for 4 x 384 experts): per layer step the route, the
    plan, the copies over PCIe and / or the host FFN, the device FFN and the
    add.  Wall-clock time per chained pass (the step synchronises on the
    selection)."""
    from bit_moe_expert_02_amd import offload as OFL
    base = synth.WORKLOADS["fp4_stack20"]
    H, I, E, k = base.hidden, base.inter, base.n_experts, base.top_k
    n_layers = args.offload_layers
    fmt = "MXFP4"
    lay = OFL.blob_layout(fmt, H, I)
    t0 = time.perf_counter()
    blobs = []
    for i in range(8):   # distinct packed experts; slot e of layer l holds item (l * E + e) % 8
        b = np.zeros(lay[3], np.uint8)
        for o, m in zip(lay[:3], synth.expert_weights(base, LY.pool_layer(0, fmt), i)):
            pk = L.pack(fmt, m)
            b[o:o + pk.size] = pk
        blobs.append(b)

    def fill(li, e, dst):
        dst[:] = blobs[(li * E + e) % len(blobs)]

    routers = [torch.from_numpy(synth.router(base, li)).cuda() for li in range(n_layers)]
    share = None if args.offload_share < 0 else args.offload_share
    st = OFL.OffloadStack(H, I, E, k, routers, [None] * n_layers, [None] * n_layers,
                          [[fmt] * E for _ in range(n_layers)], fill, args.offload_slots,
                          copy_share=share, cpu_threads=0)
    say(f"offload: {n_layers} layers, {st.store.numel() / 1e9:.1f} GB pinned, {st.n_slots} slots "
        f"({st.n_slots * st.slot_bytes / 1e9:.1f} GB), share {st.copy_share:.3f}, rates {st.rates}, "
        f"set-up {time.perf_counter() - t0:.1f} s")
    passes, warm = min(args.steps, 16), min(args.warmup, 2)
    out_rows = {}
    for rows in (1, 8):
        noise = torch.from_numpy(np.stack([synth.noise(base, li, rows) for li in range(n_layers)])).cuda()
        ws = LY.workspace(st.dims, rows)
        times = []
        for i in range(warm + passes):
            x0 = torch.from_numpy(synth.x_bf16(base, 0, rows, 70_000 + i).view(np.int16).copy()).cuda()
            if i == warm:
                before = dict(st.stats)
            torch.cuda.synchronize()
            ta = time.perf_counter()
            st.decode(x0, rows, noise, ws)
            torch.cuda.synchronize()
            if i >= warm:
                times.append(time.perf_counter() - ta)
        d = {key: st.stats[key] - before[key] for key in st.stats}
        ms = float(np.mean(times)) * 1e3
        steps = max(d["steps"], 1)
        touched = d["hits"] + d["copies"] + d["cpu"]
        out_rows[rows] = dict(
            ms_per_pass=round(ms, 3), tokens_per_s=round(rows / (ms * 1e-3), 2),
            p10_ms=round(float(np.percentile(times, 10)) * 1e3, 3),
            p90_ms=round(float(np.percentile(times, 90)) * 1e3, 3),
            experts_per_layer_step=round(touched / steps, 2),
            hit_rate=round(d["hits"] / max(touched, 1), 4),
            copies_per_layer_step=round(d["copies"] / steps, 2),
            cpu_per_layer_step=round(d["cpu"] / steps, 2),
            copy_GBps_over_pass=round(d["copy_bytes"] / (sum(times)) / 1e9, 2),
            cpu_seconds_per_pass=round(d["cpu_seconds"] / passes, 4))
        say(f"offload rows {rows}: {ms:.2f} ms/pass, {out_rows[rows]}")
    cpu = None if args.no_cpu_baseline else cpu_baseline(base, 1, n_layers)
    r0 = out_rows[1]
    line = {
        "metric": f"offloaded FP4 stack chained decode tokens/s ({n_layers} layers, experts in pinned host memory)",
        "value": r0["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": passes, "warmup": warm,
        "ms_per_step": r0["ms_per_pass"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4 codes x f16 -> f32 (router f64); host FFN f64",
        "data": "synthetic (seeded; expert slots filled from 8 distinct packed experts)",
        "config": {"workload": "offload_fp4", "layers": n_layers, "experts": n_layers * E,
                   "store_GB": round(st.store.numel() / 1e9, 2), "slots": st.n_slots,
                   "slot_GB": round(st.n_slots * st.slot_bytes / 1e9, 2),
                   "copy_share": round(st.copy_share, 4),
                   "measured_rates_GBps": None if st.rates is None else
                   {key: round(v / 1e9, 3) for key, v in st.rates.items()},
                   "rows": out_rows},
        "roofline": {"bound": "pcie", "achieved": r0["copy_GBps_over_pass"],
                     "peak": None if st.rates is None else round(st.rates["pcie_bytes_per_s"] / 1e9, 2),
                     "unit": "GB/s", "frac": None if st.rates is None else
                     round(r0["copy_GBps_over_pass"] * 1e9 / st.rates["pcie_bytes_per_s"], 4),
                     "traffic": None, "kernel": "pinned host -> device copies over the pass "
                                                "(peak: the measured pinned copy rate)"},
        "cpu_baseline": cpu,
    }
    st.close()
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is described in the design notes, not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    from bit_moe_expert_02_amd import _lib as L
    from bit_moe_expert_02_amd import layer as LY
    from bit_moe_expert_02_amd import synth

    assert torch.cuda.is_available(), "bench.py needs the MI355X"
    L.lib()
    if args.copy_calib_mb:
        src = torch.ones(args.copy_calib_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "fp4_prefill":
        return bench_prefill(args, torch, L, LY, synth)
    if args.workload in ("stack40_mixed", "fp4_stack20"):
        return bench_stack(args, torch, L, LY, synth)
    if args.workload == "verify_correlated":
        return bench_verify_correlated(args, torch, L, LY, synth)
    if args.workload == "policy_stack40":
        return bench_policy(args, torch, L, LY, synth)
    if args.workload == "alloc_stack40":
        return bench_alloc(args, torch, L, LY, synth)
    if args.workload == "offload_fp4":
        return bench_offload(args, torch, L, LY, synth)
    return main_decode(args, torch, L, LY, synth)


if __name__ == "__main__":
    main()
