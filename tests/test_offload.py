"""Stacks larger than HBM ([P1 §3C, §5], [P2 §六], [P3 §五.2]): the device
slot cache's plan (moe_cache_plan) against the oracle's plain LRU
(oracle/offload.py), step for step; the oracle pinned by a hand-worked
sequence and by invariants; the copy share; and the library's host expert FFN
(moe_cpu_expert_ffn) against the oracle's fp64 expert.  No GPU."""

import numpy as np
import pytest

from bit_moe_expert_02_amd import _lib as L
from oracle import formats as F
from oracle import moe as M
from oracle import offload as OO


def _lib_plan(cache, layer, idx, share):
    p = cache.plan(layer, np.asarray(idx, np.int32), share)
    return list(p["slot_of"]), p["copies"], p["cpu"], p["idx_gpu"].tolist()


# --------------------------------------------------------------------- the oracle, pinned
def test_oracle_hand_worked_sequence():
    """Worked by hand from the rules in oracle/offload.py: one layer, 8 experts,
    3 slots."""
    c = OO.SlotCache(1, 8, 3)
    # step 1: counts 1:1, 2:2, 5:1; misses by (most pairs, lower id): 2, 1, 5;
    # all copied into the free slots 0, 1, 2
    slot_of, copies, cpu, idx_gpu = c.plan(0, [[1, 2], [2, 5]], 1.0)
    assert copies == [(2, 0), (1, 1), (5, 2)] and cpu == []
    assert slot_of == [-1, 1, 0, -1, -1, 2, -1, -1]
    # step 2: 2 hits slot 0; 7 misses; slots 1 and 2 were last used at step 1,
    # so the lower index (slot 1, expert 1) is evicted
    slot_of, copies, cpu, idx_gpu = c.plan(0, [[2, 7]], 1.0)
    assert copies == [(7, 1)] and cpu == [] and slot_of[1] == -1 and slot_of[7] == 1
    # step 3, share 0.5: 5 hits slot 2; misses 1, 3, 4 (one pair each); m f =
    # 1.5, and q = 1 or q = 2 both leave the slower channel at one expert's
    # time (max(0.5, 1) = max(1, 0.5)), so the larger: 1 and 3 are copied,
    # 4 goes to the CPU.
    # For 1: slots 0 and 1 were last used at step 2 -> slot 0 (expert 2 out);
    # for 3: slot 1 (expert 7 out), slots 0 and 2 are in use by this step
    slot_of, copies, cpu, idx_gpu = c.plan(0, [[1, 5], [3, 4]], 0.5)
    assert copies == [(1, 0), (3, 1)] and cpu == [4]
    assert idx_gpu == [[1, 5], [3, -1]]
    assert slot_of == [-1, 0, -1, 1, -1, 2, -1, -1]


def test_oracle_share_zero_never_copies():
    c = OO.SlotCache(2, 16, 4)
    for step in range(5):
        slot_of, copies, cpu, idx_gpu = c.plan(step % 2, [[step, step + 1]], 0.0)
        assert copies == [] and cpu == [step, step + 1]
        assert all(s == -1 for s in slot_of)


def test_oracle_too_few_slots_falls_back_to_cpu():
    c = OO.SlotCache(1, 32, 2)
    slot_of, copies, cpu, idx_gpu = c.plan(0, [[0, 1, 2, 3]], 1.0)
    assert copies == [(0, 0), (1, 1)] and cpu == [2, 3]
    # the next step's hits pin both slots: the miss cannot evict them
    slot_of, copies, cpu, idx_gpu = c.plan(0, [[0, 1, 9]], 1.0)
    assert copies == [] and cpu == [9] and idx_gpu == [[0, 1, -1]]


def test_oracle_invariants_random():
    rng = np.random.default_rng(3)
    L_, E, S = 3, 24, 10
    c = OO.SlotCache(L_, E, S)
    resident = {}
    for step in range(300):
        layer = int(rng.integers(L_))
        rows, k = int(rng.integers(1, 5)), 3
        idx = [list(rng.choice(E, k, replace=False)) for _ in range(rows)]
        share = float(rng.choice([0.0, 0.3, 0.5, 1.0]))
        slot_of, copies, cpu, idx_gpu = c.plan(layer, idx, share)
        sel = sorted({e for row in idx for e in row})
        for e in sel:   # every selected expert is on the device after the step or on the CPU
            assert (slot_of[e] >= 0) != (e in cpu)
        assert sorted(e for e, _ in copies) == sorted(e for e in sel if e not in cpu and
                                                      resident.get((layer, e)) is None)
        assert [[(-1 if e in cpu else e) for e in row] for row in idx] == idx_gpu
        misses = len(copies) + len(cpu)
        assert len(copies) <= int(np.ceil(misses * share))
        for e, s in copies:
            resident = {k2: v for k2, v in resident.items() if v != s}
            resident[(layer, e)] = s
        owned = [k2 for k2 in resident]
        assert len(set(resident.values())) == len(resident) <= S and len(owned) == len(resident)
        for e in range(E):
            assert slot_of[e] == resident.get((layer, e), -1)


def _count_copied(m, f):
    c = OO.SlotCache(1, m, m)
    _, copies, cpu, _ = c.plan(0, [list(range(m))], f)
    return len(copies)


def test_oracle_copied_count_balances_the_channels():
    """The number copied, worked by hand: q next to m f minimising
    max(q (1 - f), (m - q) f)."""
    # m f = 44.28: q = 44 leaves one expert on the CPU (time 0.984 of an
    # expert), q = 45 leaves the copies at 45 * 0.016 = 0.72: copy all
    assert _count_copied(45, 0.984) == 45
    # the share one engine's profile chose ([P1 §3C], 14.7 %): m = 10 ->
    # q = 1 (max(0.853, 1.323)) beats q = 2 (max(1.706, 1.176))
    assert _count_copied(10, 0.147) == 1
    assert _count_copied(4, 0.5) == 2 and _count_copied(7, 0.0) == 0 and _count_copied(7, 1.0) == 7
    for m in range(0, 30):
        for f in (0.05, 0.3, 0.5, 0.77, 0.95):
            q = _count_copied(m, f)
            best = min(max(c * (1 - f), (m - c) * f) for c in range(m + 1))
            assert max(q * (1 - f), (m - q) * f) == pytest.approx(best, abs=1e-12)


def test_copy_share_balance():
    for bp, bc in [(50e9, 1e9), (13.1e9, 38e9), (1.0, 1.0), (0.0, 5.0)]:
        f = OO.copy_share(bp, bc)
        if bc > 0 and f < 1:
            assert f / (1 - f) == pytest.approx(bp / bc, rel=1e-12)
        # both channels finish together: f m / B_P == (1 - f) m / B_C
        if bp > 0:
            assert f / bp == pytest.approx((1 - f) / bc, rel=1e-12)
    assert OO.copy_share(0, 0) == 0.0
    # the page's first-order form m * B_P / B_H for B_P << B_H
    assert OO.copy_share(1e6, 1e12) == pytest.approx(1e6 / 1e12, rel=1e-5)


# --------------------------------------------------------------------- library == oracle
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_library_plan_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    L_, E = 4, int(rng.choice([16, 64, 384]))
    S = int(rng.integers(2, 40))
    lib_c, ora_c = L.SlotCache(L_, E, S), OO.SlotCache(L_, E, S)
    try:
        for step in range(400):
            layer = int(rng.integers(L_))
            rows, k = int(rng.integers(1, 9)), int(rng.integers(1, 7))
            k = min(k, E)
            idx = [list(map(int, rng.choice(E, k, replace=False))) for _ in range(rows)]
            share = float(rng.choice([0.0, 0.147, 0.33, 0.5, 0.9, 1.0]))
            assert _lib_plan(lib_c, layer, idx, share) == ora_c.plan(layer, idx, share)
    finally:
        lib_c.close()


def test_library_plan_rejects_bad_input_unchanged():
    lib_c, ora_c = L.SlotCache(1, 8, 2), OO.SlotCache(1, 8, 2)
    try:
        assert _lib_plan(lib_c, 0, [[1, 2]], 1.0) == ora_c.plan(0, [[1, 2]], 1.0)
        for bad_idx, share in (([[1, 8]], 1.0), ([[-1, 2]], 1.0), ([[3, 4]], 1.5), ([[3, 4]], -0.1)):
            with pytest.raises(L.MoeError) as ei:
                lib_c.plan(0, np.asarray(bad_idx, np.int32), share)
            assert ei.value.status == L.MOE_EINVAL
        # the failed calls changed nothing: the next step matches the oracle's
        assert _lib_plan(lib_c, 0, [[3, 1]], 1.0) == ora_c.plan(0, [[3, 1]], 1.0)
    finally:
        lib_c.close()
    with pytest.raises(L.MoeError):
        L.SlotCache(1, 8, 0)


def test_library_copy_share():
    for bp, bc in [(50e9, 1e9), (13.1e9, 38e9), (0.0, 0.0), (3.0, 0.0), (-1.0, 2.0)]:
        assert L.copy_share(bp, bc) == OO.copy_share(bp, bc)


# --------------------------------------------------------------------- host expert FFN
@pytest.mark.parametrize("fmt", ["Q2_0", "TERN160", "Q3", "MXFP4", "Q8"])
def test_cpu_expert_ffn_matches_oracle(fmt):
    """[P1 §3C] the CPU tier computes missed experts: the library's host FFN on
    the packed bytes against the oracle's fp64 decode and expert (512 x 256,
    a row subset with weights, accumulated into a non-zero y)."""
    rng = np.random.default_rng(11)
    H, I, R = 512, 256, 5
    mats = [rng.normal(0, 0.02, (I, H)).astype(np.float32), rng.normal(0, 0.02, (I, H)).astype(np.float32),
            rng.normal(0, 0.02, (H, I)).astype(np.float32)]
    packed = [F.pack(fmt, m) for m in mats]
    dec = [F.decode(fmt, p, *m.shape) for p, m in zip(packed, mats)]
    xb = (rng.normal(0, 1, (R, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = M.bf16_to_f64(xb)
    rows = np.array([3, 0, 4], np.int32)
    w = np.array([0.5, 0.25, 1.0], np.float32)
    y0 = rng.normal(0, 1, (R, H)).astype(np.float32)
    y = y0.copy()
    L.cpu_expert_ffn(L.dims(H, I, 16, 2), fmt, *[np.ascontiguousarray(p) for p in packed], xb, rows, w, y)
    want = y0.astype(np.float64)
    for r, wr in zip(rows, w):
        want[r] += float(wr) * M.expert_ffn(x[r], *dec)
    untouched = [1, 2]
    assert np.array_equal(y[untouched], y0[untouched])
    err = np.abs(y.astype(np.float64) - want).max() / np.abs(want).max()
    assert err < 1e-6, err


def test_cpu_expert_ffn_errors():
    d = L.dims(512, 256, 16, 2)
    z = np.zeros(1 << 20, np.uint8)
    x = np.zeros((1, 512), np.uint16)
    y = np.zeros((1, 512), np.float32)
    with pytest.raises(L.MoeError) as ei:
        L.cpu_expert_ffn(d, 9, z, z, z, x, [0], [1.0], y)
    assert ei.value.status == L.MOE_EFORMAT
    bad = np.full(1 << 20, 255, np.uint8)      # ternary bytes > 242 are invalid codes
    with pytest.raises(L.MoeError) as ei:
        L.cpu_expert_ffn(d, "TERN160", bad, bad, bad, x, [0], [1.0], y)
    assert ei.value.status == L.MOE_ECODE
