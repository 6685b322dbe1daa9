"""Device-resident MoE layers: packing with the library's packer, placement in
one HBM buffer, the expert table, and thin calls into the C ABI.

Layout of a layer's weight buffer: every expert's gate, up and down matrices
(planar packed, include/moe.h) back to back, each starting on a 256-byte
boundary; the shared expert last.  The expert table (one 32-byte record per
routed expert) lives in device memory beside it.
"""

import numpy as np

from . import _lib as L
from . import synth

ALIGN = 256


def _align(v):
    return (v + ALIGN - 1) // ALIGN * ALIGN


def expert_sizes(fmt, hidden, inter):
    gu = L.packed_bytes(fmt, inter, hidden)
    dn = L.packed_bytes(fmt, hidden, inter)
    return gu, dn


def plan(fmts, shared_fmt, hidden, inter):
    """Byte offsets of each expert's matrices; returns (table, shared_ref, total)."""
    table = np.zeros(len(fmts), L.EXPERT_REF_DTYPE)
    off = 0
    for e, f in enumerate(fmts):
        gu, dn = expert_sizes(f, hidden, inter)
        table[e] = (L.FMT[f], 0, off, _align(off + gu), _align(_align(off + gu) + gu))
        off = _align(table[e]["down"] + dn)
    shared = None
    if shared_fmt is not None:
        gu, dn = expert_sizes(shared_fmt, hidden, inter)
        shared = np.zeros(1, L.EXPERT_REF_DTYPE)
        shared[0] = (L.FMT[shared_fmt], 0, off, _align(off + gu), _align(_align(off + gu) + gu))
        off = _align(shared[0]["down"] + dn)
    return table, shared, off


class DeviceLayer:
    """One MoE layer of a workload, resident on the current HIP device.

    materialize: iterable of routed expert ids whose weights are generated and
    packed; every other slot is zero-filled (an all-zero expert in every
    format), or filled from `pool` when given.
    pool: dict fmt -> list of packed expert triples (gate, up, down) as numpy
    uint8 arrays; slot e takes pool[fmt][e % len(pool[fmt])].
    """

    def __init__(self, wl, layer, materialize=(), pool=None, device="cuda", packed=None, flags=0, fmts=None):
        import torch
        self.wl, self.layer = wl, layer
        self.dims = L.dims(wl.hidden, wl.inter, wl.n_experts, wl.top_k, flags)
        # the routed experts' formats: the workload's seeded draw, or a given map
        self.fmts = list(fmts) if fmts is not None else synth.format_map(wl, layer)
        table, shared, total = plan(self.fmts, wl.shared_fmt, wl.hidden, wl.inter)
        self.table, self.shared_table, self.total = table, shared, total
        st = L.check_experts(self.dims, table, total)
        if st != L.MOE_OK:
            raise L.MoeError("moe_check_experts", st)
        self.weights = torch.zeros(total, dtype=torch.uint8, device=device)
        self.materialized = set()
        # where each routed slot's weights come from: (layer, expert) for
        # synth.expert_weights, or None for an all-zero expert
        self.source = [None] * wl.n_experts
        for e in sorted(set(int(v) for v in materialize)):
            self._put(e, *self.pack_expert(e))
            self.materialized.add(e)
            self.source[e] = (layer, e)
        # experts this layer's own weights were already packed for (e ->
        # (gate, up, down) bytes from moe_pack of synth.expert_weights(wl, layer, e))
        for e, trip in sorted((packed or {}).items()):
            if e == wl.n_experts:
                continue                     # the shared expert is packed below
            self._put(int(e), *trip)
            self.materialized.add(int(e))
            self.source[int(e)] = (layer, int(e))
        if pool is not None:
            for e in range(wl.n_experts):
                if e not in self.materialized:
                    p = pool[self.fmts[e]]
                    self._put_dev(e, p[e % len(p)])
                    self.source[e] = (pool_layer(layer_of_pool(pool), self.fmts[e]), e % len(p))
        if wl.shared_fmt is not None:
            sh = (packed or {}).get(wl.n_experts)
            self._put(-1, *(sh if sh is not None else self.pack_expert(wl.n_experts)))
        self.experts = torch.from_numpy(table.view(np.uint8).copy()).to(device)
        self.shared = (torch.from_numpy(shared.view(np.uint8).copy()).to(device)
                       if shared is not None else None)
        self.router = torch.from_numpy(synth.router(wl, layer)).to(device)
        b = synth.bias(wl, layer)
        self.bias = torch.from_numpy(b).to(device) if b is not None else None

    def fmt_of(self, e):
        return self.wl.shared_fmt if e < 0 or e == self.wl.n_experts else self.fmts[e]

    def pack_expert(self, e):
        """Generate expert e (n_experts = the shared one) and pack it with moe_pack."""
        fmt = self.wl.shared_fmt if e == self.wl.n_experts else self.fmts[e]
        g, u, d = synth.expert_weights(self.wl, self.layer, e)
        return L.pack(fmt, g), L.pack(fmt, u), L.pack(fmt, d)

    def _ref(self, e):
        return self.shared_table[0] if e < 0 else self.table[e]

    def _put(self, e, g, u, d):
        import torch
        ref = self._ref(e)
        for off, buf in ((ref["gate"], g), (ref["up"], u), (ref["down"], d)):
            self.weights[int(off):int(off) + buf.size].copy_(torch.from_numpy(buf))

    def _put_dev(self, e, triple):
        ref = self._ref(e)
        for off, buf in zip((ref["gate"], ref["up"], ref["down"]), triple):
            self.weights[int(off):int(off) + buf.numel()].copy_(buf)


def pool_layer(layer, fmt):
    """The synth layer key a pool's experts of `fmt` are drawn with."""
    return layer + 1000 * (1 + list(L.FMT).index(fmt))


class Pool(dict):
    """fmt -> list of packed expert triples (device tensors); remembers its base layer."""

    def __init__(self, layer):
        super().__init__()
        self.layer = layer


def layer_of_pool(pool):
    return getattr(pool, "layer", 0)


def make_pool(wl, layer, fmts, count, device="cuda"):
    """Distinct packed experts per format (device tensors), for throughput-only slots.
    Item i of format f is synth.expert_weights(wl, pool_layer(layer, f), i), packed."""
    import torch
    pool = Pool(layer)
    for f in sorted(set(fmts)):
        items = []
        for i in range(count):
            g, u, d = synth.expert_weights(wl, pool_layer(layer, f), i)
            items.append(tuple(torch.from_numpy(L.pack(f, m)).to(device) for m in (g, u, d)))
        pool[f] = items
    return pool


def workspace(d, rows, device="cuda"):
    """A zero-filled workspace of moe_workspace_bytes(d, rows)."""
    import torch
    n = L.workspace_bytes(d, rows)
    if n == 0:
        raise L.MoeError("moe_workspace_bytes", L.MOE_ESHAPE)
    return torch.zeros(n, dtype=torch.uint8, device=device)
