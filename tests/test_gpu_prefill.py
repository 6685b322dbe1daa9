"""GPU parity of the many-row path: moe_expert_ffn with more than 8 rows.

With MOE_ACT_MXFP8, MXFP4 experts run on the matrix cores: gate/up with
MXFP8 x on the scaled fp8 x fp4 instruction, down with f16 h; the oracle
quantises x the same way (oracle.moe.prefill_layer / many_row_layer) and
computes the rest in fp64.  Every other expert (any format, and MXFP4 without
the flag) and the shared expert run the decode tiles on unquantised x.

Bar: the MXFP8 quantiser bit-exact; y within 1e-3 relative L2 per row."""

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


def e4m3_value(code):
    """Value of OCP e4m3 (finite-only variant) codes; 0x7F / 0xFF are NaN."""
    c = np.asarray(code, np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def test_e4m3_decoder_matches_the_oracle_grid():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    v = e4m3_value(codes)
    np.testing.assert_array_equal(OM.round_e4m3(v), v)          # every code is on the grid
    assert len(set(v[codes < 0x80].tolist())) == 127              # and distinct (0 .. 448)
    assert e4m3_value(0x7E) == 448.0 and e4m3_value(0x01) == 2.0 ** -9


def test_quant_mxfp8_bit_exact():
    rng = np.random.default_rng(3)
    R, K = 64, 512
    x = rng.standard_normal((R, K)).astype(np.float32)
    blk = x.reshape(R, K // 32, 32)
    blk[0::7] *= np.float32(1e-30)                                 # tiny blocks
    blk[1::7] *= np.float32(1e30)                                  # huge blocks
    blk[2::7] = 0.0                                                # all-zero blocks
    blk[3::7, :, 5] = np.float32(3.0e38)                           # a near-max element
    xbits = synth.f32_to_bf16_bits(blk.reshape(R, K))
    xd = torch.from_numpy(xbits.view(np.int16).copy()).cuda()
    codes = torch.zeros((R, K), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((R, K // 32), dtype=torch.uint8, device="cuda")
    L.moe_quant_mxfp8(xd, R, K, codes, scales)
    torch.cuda.synchronize()
    want, E = OM.quant_mxfp8(OM.bf16_to_f64(xbits))
    got_e = scales.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(got_e, E)
    got = e4m3_value(codes.cpu().numpy()) * np.repeat(np.ldexp(1.0, got_e - 127), 32, axis=1)
    np.testing.assert_array_equal(got, want)


def _prefill(dl, xbits, idx, w, rows, flags=L.MOE_ACT_MXFP8, shared=None, misaligned=False):
    """y of a many-row call; with `misaligned`, y starts 4 bytes past a
    16-byte boundary (the combine then writes one float per thread), and the
    float before it must stay untouched."""
    wl = dl.wl
    d = L.dims(wl.hidden, wl.inter, wl.n_experts, wl.top_k, flags)
    ws = LY.workspace(d, rows)
    n = rows * dl.wl.hidden
    flat = torch.zeros(n + 2, dtype=torch.float32, device="cuda")
    y = flat[1:n + 1].view(rows, dl.wl.hidden) if misaligned else flat[:n].view(rows, dl.wl.hidden)
    L.moe_expert_ffn(d, G.device_inputs(dl.wl, 0, xbits), rows, torch.from_numpy(idx).cuda(),
                     torch.from_numpy(w).cuda(), dl.weights, dl.experts, shared, y, ws)
    torch.cuda.synchronize()
    if misaligned:
        assert y.data_ptr() % 16 == 4
        assert flat[0].item() == 0.0 and flat[n + 1].item() == 0.0   # nothing written outside y
    return y.cpu().numpy()


def test_tiny_prefill_every_row():
    """Tiny MXFP4 layer, 256 Zipf-routed rows: experts see 1..~100 rows, so
    chunks of one to several 16-row tiles and several chunks per expert occur."""
    wl = synth.Workload("tiny_fp4", 30, 512, 256, 16, 2, "MXFP4", None, rows=(256,))
    R = 256
    xbits = synth.x_bf16(wl, 0, R)
    idx, w = synth.zipf_routing(wl, 0, R)
    counts = np.bincount(idx.reshape(-1), minlength=16)
    _say("rows per expert", counts.tolist())
    assert counts.max() > 64                                       # an expert spans several chunks
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    y = _prefill(dl, xbits, idx, w, R)
    ref = OM.prefill_layer(OM.bf16_to_f64(xbits), idx, w.astype(np.float64),
                           lambda e: G.oracle_expert(wl, 0, e))
    err = G.rel_l2_rows(y, ref)
    _say("max rel L2", f"{err.max():.2e}")
    assert np.all(err <= G.REL_L2_TOL)
    assert np.array_equal(y, _prefill(dl, xbits, idx, w, R))      # bitwise reproducible
    # a y that is not 16-byte aligned takes the one-wide combine: same bits
    assert np.array_equal(y, _prefill(dl, xbits, idx, w, R, misaligned=True))


def test_real_shape_prefill_sampled_rows():
    """One layer of the FP4 stack, 2048 Zipf-routed rows (the prefill shape);
    rows checked against the oracle: the first, the last, and one routed to
    the most popular expert."""
    wl = synth.WORKLOADS["fp4_stack20"]
    R = 2048
    xbits = synth.x_bf16(wl, 0, R, 7)
    idx, w = synth.zipf_routing(wl, 0, R)
    top = np.bincount(idx.reshape(-1)).argmax()
    check = sorted({0, R - 1, int(np.nonzero((idx == top).any(axis=1))[0][0])})
    need = sorted(set(idx[check].reshape(-1).tolist()))
    _say(f"fp4 prefill: {R} rows, top expert {top} with {(idx == top).sum()} rows, checking {check}")
    pool = LY.make_pool(wl, 0, ["MXFP4"], 8)
    dl = LY.DeviceLayer(wl, 0, materialize=need, pool=pool)
    y = _prefill(dl, xbits, idx, w, R)
    assert np.all(np.isfinite(y))
    x = OM.bf16_to_f64(xbits)
    ref = OM.prefill_layer(x[check], idx[check], w[check].astype(np.float64),
                           lambda e: G.oracle_expert(wl, 0, e))
    err = G.rel_l2_rows(y[check], ref)
    _say("rel L2 per checked row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)


def _tiny_many_rows(name, key, fmt, rows, flags, shared_fmt):
    wl = synth.Workload(name, key, 512, 256, 16, 2, fmt, shared_fmt, rows=(rows,))
    xbits = synth.x_bf16(wl, 0, rows)
    idx, w = synth.zipf_routing(wl, 0, rows)
    dl = LY.DeviceLayer(wl, 0, materialize=range(wl.n_experts))
    fm = synth.format_map(wl, 0)
    _say(f"{name}: {rows} rows, formats {sorted(set(fm))}, flags {flags}, shared {shared_fmt}")
    y = _prefill(dl, xbits, idx, w, rows, flags, dl.shared)
    shared = G.oracle_expert(wl, 0, wl.n_experts) if shared_fmt else None
    ref = OM.many_row_layer(OM.bf16_to_f64(xbits), idx, w.astype(np.float64),
                            lambda e: G.oracle_expert(wl, 0, e), lambda e: fm[e],
                            bool(flags & L.MOE_ACT_MXFP8), shared)
    err = G.rel_l2_rows(y, ref)
    _say("  max rel L2", f"{err.max():.2e}")
    assert np.all(err <= G.REL_L2_TOL)
    assert np.array_equal(y, _prefill(dl, xbits, idx, w, rows, flags, dl.shared))   # bitwise again


def test_tiny_many_rows_generic_mixed_formats_with_shared():
    """Ternary / Q2_0 / Q3 experts and a Q8 shared expert, 40 rows: every pair
    runs the decode tiles (entries of up to 8 pairs of one expert)."""
    _tiny_many_rows("tiny_mix_many", 32, "MIX", 40, 0, "Q8")


def test_tiny_many_rows_all_formats_with_the_flag():
    """All five formats mixed, 96 rows, MOE_ACT_MXFP8: MXFP4 experts on the
    matrix cores (quantised x), the others and the shared expert on the
    decode tiles (unquantised x), one combine in ascending expert id."""
    _tiny_many_rows("tiny_all_many", 33, "MIXALL", 96, L.MOE_ACT_MXFP8, "Q2_0")


def test_tiny_many_rows_mxfp4_without_the_flag_is_exact():
    """MXFP4 experts without the flag: the decode tiles on unquantised x."""
    _tiny_many_rows("tiny_fp4_generic", 34, "MXFP4", 24, 0, None)


def test_real_shape_many_rows_generic_sampled():
    """The mixed-format layer (with its Q8 shared expert) at 24 rows on the
    generic path; the first, a middle and the last row checked."""
    wl = synth.WORKLOADS["mixed_verify"]
    R = 24
    xbits = synth.x_bf16(wl, 0, R, 9)
    idx, w = synth.zipf_routing(wl, 0, R)
    check = [0, 11, R - 1]
    x = OM.bf16_to_f64(xbits)
    dl, ref = G.materialized_layer_and_oracle(wl, 0, x[check], idx[check], w[check].astype(np.float64))
    y = _prefill(dl, xbits, idx, w, R, 0, dl.shared)
    err = G.rel_l2_rows(y[check], ref)
    _say("rel L2 per checked row", G.fmt_err(err))
    assert np.all(err <= G.REL_L2_TOL)
