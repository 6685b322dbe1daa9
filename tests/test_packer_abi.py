"""CPU checks of the C-ABI library: exported symbols, host packer vs the oracle's
packer (bit-exact bytes), unpack vs the oracle's decoders, host-side error paths.
No device call is made here."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import formats as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from bit_moe_expert_02_amd import _lib
    _lib.lib()
    return _lib


def test_exports_match_header(L):
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    declared = set(re.findall(r"^\s*(?:const char\*|size_t|int32_t|int|void|double)\s+(moe_\w+)\s*\(", hdr, re.M))
    assert declared == set(L.EXPORTS)
    for name in declared:
        assert hasattr(L.lib(), name), name


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert L.status_string(st) != "unknown status"
    assert L.status_string(-99) == "unknown status"


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("shape", [(7, 2304), (3, 5120), (2, 512), (4, 256)])
def test_pack_matches_oracle_bytes(L, fmt, shape):
    n, k = shape
    rng = np.random.default_rng(abs(hash((fmt, shape))) % 2**32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0                                  # all-zero blocks
    w[1, 3] = -w[1, :64].__abs__().max()             # ties in |w|
    w[1, 7] = -w[1, 3]
    w[-1, 10:20] = 1e-30                             # subnormal-scale blocks
    w[-1, k - 5:] *= 1e4                             # large values (fp16 range)
    assert L.packed_bytes(fmt, n, k) == F.packed_bytes(fmt, n, k)
    got = L.pack(fmt, w, nthreads=3)
    assert np.array_equal(got, F.pack(fmt, w))
    dec = L.unpack(fmt, got, n, k, nthreads=2)
    assert np.array_equal(dec.astype(np.float64), F.decode(fmt, got, n, k))


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_unpack_random_valid_bytes(L, fmt):
    rng = np.random.default_rng(3)
    n, k = 3, (768 if fmt == "Q3" else 640)
    buf = rng.integers(0, 256, F.packed_bytes(fmt, n, k), dtype=np.uint8)
    nb = F.blocks_per_row(fmt, k)
    if fmt == "TERN160":
        codes = buf[: n * nb * 32]
        codes %= 243
    if fmt == "MXFP4":
        sc = buf[n * nb * 16:]
        sc[sc > 250] = 250                               # keep 6 * 2^(E-127) inside fp32
    if fmt in ("Q2_0", "TERN160", "Q8"):                 # finite fp16 scales
        s = buf[n * nb * F.CODE_BYTES[fmt]:].view("<u2")
        s &= 0xBBFF
    if fmt == "Q3":
        s = buf[n * nb * 96: n * nb * 98].view("<u2")
        s &= 0xBBFF
    got = L.unpack(fmt, buf, n, k)
    assert np.array_equal(got.astype(np.float64), F.decode(fmt, buf, n, k))


def test_unpack_rejects_invalid_codes(L):
    buf = np.zeros(F.packed_bytes("TERN160", 1, 160), np.uint8)
    buf[5] = 243
    with pytest.raises(L.MoeError) as e:
        L.unpack("TERN160", buf, 1, 160)
    assert e.value.status == L.MOE_ECODE
    buf = np.zeros(17, np.uint8)
    buf[16] = 255
    with pytest.raises(L.MoeError) as e:
        L.unpack("MXFP4", buf, 1, 32)
    assert e.value.status == L.MOE_ECODE


def test_pack_errors(L):
    lib = L.lib()
    w = np.zeros((2, 64), np.float32)
    out = np.zeros(64, np.uint8)
    assert lib.moe_pack(99, w.ctypes.data, 2, 64, out.ctypes.data, 64, 1) == L.MOE_EFORMAT
    assert lib.moe_pack(2, None, 2, 64, out.ctypes.data, 64, 1) == L.MOE_EINVAL
    assert lib.moe_pack(2, w.ctypes.data, 2, 60, out.ctypes.data, 64, 1) == L.MOE_ESHAPE
    assert lib.moe_pack(2, w.ctypes.data, 2, 64, out.ctypes.data, 10, 1) == L.MOE_EINVAL
    assert L.packed_bytes("Q2_0", 2, 60) == 0
    assert L.packed_bytes("TERN160", 1, 300) == 68


def test_workspace_and_dims_validation(L):
    d = L.dims(5120, 2304, 384, 6)
    ws = L.workspace_bytes(d, 8)
    assert ws > 0 and ws % 256 == 0
    # above the decode row limit: the prefill path's workspace, which holds
    # MXFP8 x, the dispatch, MXFP8 h and the fp32 per-pair partials
    wp = L.workspace_bytes(d, 2048)
    assert wp >= 2048 * 6 * (5120 * 4 + 2304) + 2048 * 5120 and wp % 256 == 0
    assert L.workspace_bytes(d, 8193) == 0                # above the prefill row limit
    assert L.workspace_bytes(L.dims(4096, 2304, 384, 6), 1) == 0
    assert L.workspace_bytes(L.dims(5120, 2304, 384, 9), 1) == 0
    assert L.workspace_bytes(L.dims(512, 256, 16, 2), 4) > 0


def test_entry_points_reject_bad_args_on_host(L):
    lib = L.lib()
    d = L.dims(5120, 2304, 384, 6)
    bad = L.dims(5000, 2304, 384, 6)
    dp = ctypes.byref(d)
    fake = ctypes.c_void_p(0x1000)                       # never dereferenced: errors come first
    ws_need = L.workspace_bytes(d, 1)
    # null dims / negative rows / unsupported shape
    assert lib.moe_route(None, fake, 1, fake, None, fake, fake, fake, ws_need, None) == L.MOE_EINVAL
    assert lib.moe_route(dp, fake, -1, fake, None, fake, fake, fake, ws_need, None) == L.MOE_EINVAL
    assert lib.moe_route(ctypes.byref(bad), fake, 1, fake, None, fake, fake, fake, ws_need, None) == L.MOE_ESHAPE
    assert lib.moe_route(dp, fake, 9, fake, None, fake, fake, fake, ws_need, None) == L.MOE_ESHAPE
    # missing outputs, missing router, small workspace
    assert lib.moe_route(dp, fake, 1, fake, None, None, fake, fake, ws_need, None) == L.MOE_EINVAL
    assert lib.moe_route(dp, fake, 1, None, None, fake, fake, fake, ws_need, None) == L.MOE_EINVAL
    assert lib.moe_route(dp, fake, 1, fake, None, fake, fake, fake, ws_need - 1, None) == L.MOE_EWORKSPACE
    # expert ffn without routing inputs / weights
    assert lib.moe_expert_ffn(dp, fake, 1, None, fake, fake, fake, None, fake, fake, ws_need, None) == L.MOE_EINVAL
    assert lib.moe_expert_ffn(dp, fake, 1, fake, fake, None, fake, None, fake, fake, ws_need, None) == L.MOE_EINVAL
    # rows == 0 is a no-op
    assert lib.moe_layer(dp, fake, 0, fake, None, fake, fake, None, fake, fake, fake, fake, ws_need, None) == L.MOE_OK
    # profiled needs two events
    assert lib.moe_layer_profiled(dp, fake, 1, fake, None, fake, fake, None, fake, fake, fake, fake,
                                  ws_need, None, None, 0) == L.MOE_EINVAL
    evs = (ctypes.c_void_p * 1)()
    assert lib.moe_layer_profiled(dp, fake, 1, fake, None, fake, fake, None, fake, fake, fake, fake,
                                  ws_need, None, evs, 1) == L.MOE_EINVAL


def test_check_experts(L):
    from bit_moe_expert_02_amd import layer, synth
    wl = synth.WORKLOADS["mixed_verify"]
    d = L.dims(wl.hidden, wl.inter, wl.n_experts, wl.top_k)
    table, shared, total = layer.plan(synth.format_map(wl, 0), "Q8", wl.hidden, wl.inter)
    assert L.check_experts(d, table, total) == L.MOE_OK
    assert L.check_experts(d, shared, total) == L.MOE_OK
    t = table.copy()
    t[3]["fmt"] = 9
    assert L.check_experts(d, t, total) == L.MOE_EFORMAT
    t = table.copy()
    t[5]["gate"] += 8
    assert L.check_experts(d, t, total) == L.MOE_EINVAL
    end = int(shared[0]["down"]) + L.packed_bytes("Q8", wl.hidden, wl.inter)
    assert L.check_experts(d, shared, end) == L.MOE_OK
    assert L.check_experts(d, shared, end - 1) == L.MOE_EINVAL
    t = table.copy()
    t[0]["reserved"] = 1
    assert L.check_experts(d, t, total) == L.MOE_EINVAL


def test_plan_offsets_and_sizes():
    from bit_moe_expert_02_amd import layer
    table, shared, total = layer.plan(["Q2_0", "TERN160", "Q3"], "Q8", 5120, 2304)
    assert table["gate"][0] == 0
    for r in list(table) + list(shared):
        assert r["gate"] % 256 == 0 and r["up"] % 256 == 0 and r["down"] % 256 == 0
    assert total >= 9_953_280 + 7_624_704 + 15_206_400 + 37_601_280


def test_spin_limit_setter(L):
    """The hand-off spin limit is a process-wide host setting: the setter
    returns the previous value and rejects a negative one (no device use)."""
    lib = L.lib()
    prev = lib.moe_set_spin_limit(1000)
    try:
        assert prev >= 0
        assert lib.moe_set_spin_limit(-1) == -1          # MOE_EINVAL, limit unchanged
        assert lib.moe_set_spin_limit(1000) == 1000
    finally:
        lib.moe_set_spin_limit(prev)
