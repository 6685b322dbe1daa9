"""Oracle: per-expert format allocation (ternary / Q2_0 / Q3) for a stack.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[P3 §五.1] allocates a format to every routed expert:
  * budget: exactly the bytes of the whole stack in Q2_0 (budget neutral);
  * Lagrangian relaxation (bisection on the multiplier), then a greedy fill of
    the bytes left over;
  * cost of an expert's format = its held-out output error / its layer's
    routed output energy (every layer weighs the same), doubled for the first
    2 and the last 3 layers;
  * guardrails: at most 50 % ternary experts per layer; an expert seen by
    fewer than 8 held-out tokens stays Q2_0.

Readings where the page is silent (each also in the design notes):
  * per expert the multiplier picks the format of least cost + lam * bytes;
    equal values go to Q2_0 first, then ternary, then Q3;
  * the ternary cap per layer is floor(0.5 * E); when more experts pick
    ternary, those whose best other value is closest to their ternary value go
    to that other format (equal differences: the higher expert id first);
  * the bisection keeps the smallest multiplier found whose choice fits: if
    the choice at 0 fits it is taken as is; otherwise the upper end doubles
    from 1 until it fits, then 200 halvings at most;
  * greedy fill: the upgrades to a larger format of lower cost, largest cost
    saving per extra byte first (ties: lower expert index, then lower format
    index), each taken when it still fits.
"""

import heapq

import numpy as np

FORMATS = ("TERN160", "Q2_0", "Q3")      # candidate order; bytes must increase
TIE_ORDER = (1, 0, 2)                    # Q2_0, ternary, Q3


def costs(err, energy, edge_first=2, edge_last=3):
    """cost[l, e, f] = w_l * err[l, e, f] / energy[l], w_l = 2 on the first
    edge_first and last edge_last layers, else 1."""
    err = np.asarray(err, np.float64)
    L = err.shape[0]
    w = np.array([2.0 if (l < edge_first or l >= L - edge_last) else 1.0 for l in range(L)])
    return w[:, None, None] * err / np.asarray(energy, np.float64)[:, None, None]


def lagrangian_choice(cost, locked, nbytes, lam, cap):
    """Format index per expert for multiplier lam, with the per-layer ternary cap."""
    L, E, _ = cost.shape
    f = np.empty((L, E), np.int64)
    for l in range(L):
        tern = []
        for e in range(E):
            if locked[l, e]:
                f[l, e] = 1
                continue
            vals = {c: cost[l, e, c] + lam * nbytes[c] for c in range(3)}
            best = min(TIE_ORDER, key=lambda c: (vals[c], TIE_ORDER.index(c)))
            f[l, e] = best
            if best == 0:
                alt = min(vals[c] for c in TIE_ORDER if c != 0)
                tern.append((alt - vals[0], -e, e))
        over = len(tern) - cap
        if over > 0:
            tern.sort()
            for _, _, e in tern[:over]:
                vals = {c: cost[l, e, c] + lam * nbytes[c] for c in range(3)}
                f[l, e] = min((c for c in TIE_ORDER if c != 0), key=lambda c: (vals[c], TIE_ORDER.index(c)))
    return f


def allocate(err, tokens, energy, nbytes, max_tern_frac=0.5, min_tokens=8, edge_first=2, edge_last=3):
    """Returns (format names [L, E], total cost, total bytes, budget)."""
    cost = costs(err, energy, edge_first, edge_last)
    L, E, _ = cost.shape
    nbytes = [float(b) for b in nbytes]
    locked = np.asarray(tokens) < min_tokens
    cap = int(np.floor(max_tern_frac * E))
    budget = L * E * nbytes[1]

    def size(f):
        return float(sum(nbytes[c] for c in f.reshape(-1)))

    f = lagrangian_choice(cost, locked, nbytes, 0.0, cap)
    if size(f) > budget:
        lo, hi = 0.0, 1.0
        while True:
            g = lagrangian_choice(cost, locked, nbytes, hi, cap)
            if size(g) <= budget or hi > 1e300:
                break
            lo, hi = hi, hi * 2.0
        for _ in range(200):
            if not hi - lo > 0.0:
                break
            mid = lo + (hi - lo) * 0.5
            if mid <= lo or mid >= hi:
                break
            if size(lagrangian_choice(cost, locked, nbytes, mid, cap)) <= budget:
                hi = mid
            else:
                lo = mid
        f = lagrangian_choice(cost, locked, nbytes, hi, cap)
    left = budget - size(f)
    flat = f.reshape(-1)
    cflat = cost.reshape(-1, 3)
    lflat = locked.reshape(-1)
    ver = np.zeros(flat.size, np.int64)
    heap = []

    def push(i):
        if lflat[i]:
            return
        cur = flat[i]
        for c in range(3):
            extra = nbytes[c] - nbytes[cur]
            gain = cflat[i, cur] - cflat[i, c]
            if extra > 0.0 and gain > 0.0:
                heapq.heappush(heap, (-(gain / extra), i, c, ver[i]))

    for i in range(flat.size):
        push(i)
    while heap:
        _, i, c, v = heapq.heappop(heap)
        if v != ver[i]:
            continue
        extra = nbytes[c] - nbytes[flat[i]]
        if extra > left:
            continue
        left -= extra
        flat[i] = c
        ver[i] += 1
        push(i)
    total_cost = float(sum(cflat[i, flat[i]] for i in range(flat.size)))
    names = np.array([[FORMATS[c] for c in row] for row in flat.reshape(L, E)])
    return names, total_cost, size(flat.reshape(L, E)), budget
