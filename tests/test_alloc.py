"""Per-expert format allocation ([P3 §五.1]): the library's moe_allocate_formats
against the oracle (oracle/alloc.py), decision for decision, and the oracle
pinned by the guardrails, a closed form and brute force on tiny instances."""

import itertools

import numpy as np
import pytest

from bit_moe_expert_02_amd import _lib as L
from bit_moe_expert_02_amd import synth
from oracle import alloc as OA

NBYTES = (7_624_704, 9_953_280, 15_206_400)   # TERN160, Q2_0, Q3 expert at 5120 / 2304


def _small(L_=6, E=48, seed=0):
    wl = synth.Workload("alloc_small", 90 + seed, 512, 256, E, 6, "MIX", None, layers=L_)
    return synth.alloc_inputs(wl, heldout_tokens=2_000)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_library_matches_oracle(seed):
    err, tokens, energy = _small(seed=seed)
    want, cost, nbytes, budget = OA.allocate(err, tokens, energy, NBYTES)
    got, gcost, gbytes = L.allocate_formats(err, tokens, energy, NBYTES)
    assert np.array_equal(got, want)
    assert gbytes == nbytes and gcost == pytest.approx(cost, rel=1e-12)


def test_guardrails_and_budget():
    err, tokens, energy = _small(L_=8, E=64, seed=4)
    tokens[3, :10] = 3                              # ten experts seen by fewer than 8 tokens
    names, cost, nbytes, budget = OA.allocate(err, tokens, energy, NBYTES)
    assert nbytes <= budget == 8 * 64 * NBYTES[1]
    assert np.all((names == "TERN160").sum(axis=1) <= 32)
    assert np.all(names[3, :10] == "Q2_0")
    assert cost < OA.costs(err, energy)[:, :, 1].sum()     # better than all Q2_0 at the same budget
    assert len(set(names.reshape(-1))) == 3


def test_equal_errors_keep_every_expert_q2():
    """Formats of equal error: at multiplier 0 every value ties and Q2_0 wins
    the tie; all-Q2_0 fits the budget exactly, and no upgrade saves cost."""
    err, tokens, energy = _small(seed=5)
    err = np.repeat(err[:, :, 1:2], 3, axis=2)
    names, cost, nbytes, budget = OA.allocate(err, tokens, energy, NBYTES)
    assert np.all(names == "Q2_0") and nbytes == budget


def test_edge_layers_count_double():
    err = np.ones((6, 2, 3))
    c = OA.costs(err, np.ones(6))
    assert c[:, 0, 0].tolist() == [2, 2, 1, 2, 2, 2]


def test_lagrangian_choice_is_optimal_for_its_bytes():
    """Brute force over all 3^6 assignments of a one-layer, six-expert problem
    (no binding guardrail): no assignment of at most the Lagrangian choice's
    bytes costs less, at several multipliers."""
    rng = np.random.default_rng(11)
    nb = [float(b) for b in NBYTES]
    for _ in range(5):
        cost = rng.random((1, 6, 3))
        locked = np.zeros((1, 6), bool)
        for lam in (0.0, 1e-8, 5e-8, 2e-7):
            f = OA.lagrangian_choice(cost, locked, nb, lam, cap=6)[0]
            fb = sum(nb[c] for c in f)
            fc = sum(cost[0, e, c] for e, c in enumerate(f))
            for a in itertools.product(range(3), repeat=6):
                if sum(nb[c] for c in a) <= fb:
                    assert sum(cost[0, e, c] for e, c in enumerate(a)) >= fc - 1e-12


def test_greedy_fill_leaves_no_affordable_upgrade():
    err, tokens, energy = _small(seed=6)
    names, cost, nbytes, budget = OA.allocate(err, tokens, energy, NBYTES)
    c = OA.costs(err, energy)
    idx = {n: i for i, n in enumerate(OA.FORMATS)}
    left = budget - nbytes
    for l in range(names.shape[0]):
        for e in range(names.shape[1]):
            if tokens[l, e] < 8:
                continue
            cur = idx[names[l, e]]
            for to in range(3):
                if NBYTES[to] > NBYTES[cur] and c[l, e, to] < c[l, e, cur]:
                    assert NBYTES[to] - NBYTES[cur] > left


def test_argument_errors():
    err, tokens, energy = _small(seed=7)
    with pytest.raises(L.MoeError):
        L.allocate_formats(err, tokens, energy, (NBYTES[1], NBYTES[0], NBYTES[2]))
    bad = energy.copy()
    bad[0] = 0.0
    with pytest.raises(L.MoeError):
        L.allocate_formats(err, tokens, bad, NBYTES)
