"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no routing, no packing, no expert math).  The oracle and
the HIP path are both fed from here.

Every tensor has its own stream: SeedSequence(seed, spawn_key=(workload,
layer, tensor, expert)), so any layer or expert can be regenerated alone.

Distributions (the pages have no real weights to offer; these stand in):
  x            fp32 N(0, 1) rounded to bf16 (round to nearest even)
  router       fp32 N(0, 0.02^2)        [E x H]
  experts      fp32 N(0, 0.02^2)        gate, up [I x H]; down [H x I]
  bias         fp32 U(-0.6, 1.0)        one per expert (selection only)
  format map   exact per-layer counts from the shares 42.8 / 39.2 / 18.0 %
               (ternary / Q2_0 / Q3, [P3 §五.1]) placed by a seeded permutation
"""

from dataclasses import dataclass, field

import numpy as np

# tensor ids in the spawn key
T_X, T_ROUTER, T_BIAS, T_FMAP, T_NOISE, T_ROUTE, T_EXPERT = 0, 1, 2, 3, 4, 5, 16
# matrix ids inside an expert stream
M_GATE, M_UP, M_DOWN = 0, 1, 2

MIX_SHARES = (("TERN160", 0.428), ("Q2_0", 0.392), ("Q3", 0.180))


@dataclass(frozen=True)
class Workload:
    """A named layer shape and how its weights are drawn."""
    name: str
    key: int                      # workload id inside the spawn key
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    routed_fmt: str               # "Q2_0", "MXFP4", ... or "MIX"
    shared_fmt: str | None        # None: no shared expert
    use_bias: bool = False
    layers: int = 1
    rows: tuple = (1,)
    seed: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # tiny layer, CPU-checkable in seconds
    "tiny": Workload("tiny", 1, 512, 256, 16, 2, "Q2_0", "Q2_0", rows=(4,)),
    # one real-shape decode layer: Q2_0 routed experts, int8 shared expert
    "decode_q2": Workload("decode_q2", 2, 5120, 2304, 384, 6, "Q2_0", "Q8", rows=(1,)),
    # mixed-format speculative-verify layer with a selection-only bias
    "mixed_verify": Workload("mixed_verify", 3, 5120, 2304, 384, 6, "MIX", "Q8",
                             use_bias=True, rows=(1, 5, 8)),
    # 40-layer routed stack in the mixed formats
    "stack40_mixed": Workload("stack40_mixed", 4, 5120, 2304, 384, 6, "MIX", "Q8",
                              use_bias=True, layers=40, rows=(1, 7)),
    # tiny stack in the mixed formats, CPU-checkable: chained decode parity
    "tiny_stack": Workload("tiny_stack", 6, 512, 256, 16, 2, "MIX", "Q8", use_bias=True,
                           layers=4, rows=(1, 7)),
    # 20-layer FP4 stack (no shared expert); 2048 rows is the prefill shape
    "fp4_stack20": Workload("fp4_stack20", 5, 5120, 2304, 384, 6, "MXFP4", None,
                            layers=20, rows=(1, 8, 2048)),
}


def rng(wl, layer, tensor, expert=0):
    ss = np.random.SeedSequence(wl.seed, spawn_key=(wl.key, layer, tensor, expert))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(v):
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def x_bf16(wl, layer, rows, stream=0):
    """Activations [rows x H] as bf16 bits; `stream` selects an independent draw."""
    g = rng(wl, layer, T_X, stream)
    return f32_to_bf16_bits(g.standard_normal((rows, wl.hidden), dtype=np.float32))


def router(wl, layer):
    g = rng(wl, layer, T_ROUTER)
    return (g.standard_normal((wl.n_experts, wl.hidden), dtype=np.float32)
            * np.float32(0.02)).astype(np.float32)


def bias(wl, layer):
    if not wl.use_bias:
        return None
    g = rng(wl, layer, T_BIAS)
    return g.uniform(-0.6, 1.0, wl.n_experts).astype(np.float32)


def expert_weights(wl, layer, expert):
    """(gate [I x H], up [I x H], down [H x I]) fp32; expert == n_experts is the shared one."""
    g = rng(wl, layer, T_EXPERT, expert)
    s = np.float32(0.02)
    gate = g.standard_normal((wl.inter, wl.hidden), dtype=np.float32) * s
    up = g.standard_normal((wl.inter, wl.hidden), dtype=np.float32) * s
    down = g.standard_normal((wl.hidden, wl.inter), dtype=np.float32) * s
    return gate, up, down


def mix_counts(n_experts):
    """Exact per-layer counts for MIX_SHARES; the remainder goes to the last format."""
    counts = [int(np.floor(n_experts * s + 0.5)) for _, s in MIX_SHARES[:-1]]
    counts.append(n_experts - sum(counts))
    return counts


def format_map(wl, layer):
    """List of format names, one per routed expert."""
    if wl.routed_fmt != "MIX":
        return [wl.routed_fmt] * wl.n_experts
    names = []
    for (name, _), c in zip(MIX_SHARES, mix_counts(wl.n_experts)):
        names += [name] * c
    perm = rng(wl, layer, T_FMAP).permutation(wl.n_experts)
    return [names[i] for i in perm]


def zipf_routing(wl, layer, rows, s=1.1, stream=0):
    """Prefill routing given to the expert FFN: expert popularity p_i proportional
    to rank_i^-s over a seeded permutation of the ids; each row takes the top_k
    of log p + Gumbel noise (a draw of top_k distinct experts without
    replacement), with weights = softmax of those keys over the selection.
    Returns (idx int32 [rows x k], w fp32 [rows x k]), keys descending."""
    g = rng(wl, layer, T_ROUTE, stream)
    perm = g.permutation(wl.n_experts)
    logp = np.empty(wl.n_experts)
    logp[perm] = -s * np.log(np.arange(1, wl.n_experts + 1, dtype=np.float64))
    keys = logp[None, :] + g.gumbel(size=(rows, wl.n_experts))
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :wl.top_k]
    kv = np.take_along_axis(keys, idx, axis=1)
    w = np.exp(kv - kv[:, :1])
    w /= w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w.astype(np.float32)


def noise(wl, layer, rows):
    """N(0,1) fp32 [rows x H] added to a layer's output before it feeds the next layer."""
    return rng(wl, layer, T_NOISE).standard_normal((rows, wl.hidden), dtype=np.float32)
