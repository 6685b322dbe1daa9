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
  bias         fp32 U(-0.6, 1.0)        one per expert (selection only), or the
               residency policy: +1.0 / 0 / -0.6 by tier, times a scale
  correlated   rows of a verify window x_r = rho x_0 + sqrt(1 - rho^2) z_r
  format map   exact per-layer counts from the shares 42.8 / 39.2 / 18.0 %
               (ternary / Q2_0 / Q3, [P3 §五.1]) placed by a seeded permutation
"""

from dataclasses import dataclass, field

import numpy as np

# tensor ids in the spawn key
T_X, T_ROUTER, T_BIAS, T_FMAP, T_NOISE, T_ROUTE, T_TIER, T_EXPERT = 0, 1, 2, 3, 4, 5, 6, 16
# matrix ids inside an expert stream
M_GATE, M_UP, M_DOWN = 0, 1, 2

MIX_SHARES = (("TERN160", 0.428), ("Q2_0", 0.392), ("Q3", 0.180))
# every routed format in equal shares (tests of a table that mixes all five)
MIX_ALL_SHARES = (("TERN160", 0.2), ("Q2_0", 0.2), ("Q3", 0.2), ("MXFP4", 0.2), ("Q8", 0.2))


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
    # the draft model's MoE layer: 128 routed experts, top-3 ([P1 §1]:
    # dspark_n_routed_experts 128, dspark_num_experts_per_tok 3), a block of 5
    # drafted rows (dspark_block_size 5); Q2_0 experts (the draft sidecar is a
    # 2-bit file, [P3 §三])
    "draft128": Workload("draft128", 7, 5120, 2304, 128, 3, "Q2_0", "Q2_0", rows=(1, 5)),
    # the mixed stack under the residency-style selection bias ([P3 §五.3]),
    # scale 0.5 (the page's default; the bench also runs 0, 0.25 and 1.0)
    "policy_stack40": Workload("policy_stack40", 8, 5120, 2304, 384, 6, "MIX", "Q8",
                               layers=40, rows=(1, 7), extra={"policy_scale": 0.5}),
    # the mixed stack decoded in verify windows of correlated rows, rho chosen
    # so that a 7-row window touches about 25 distinct experts per layer
    # ([P1 §3B]: 38,543 + 5,857 expert evaluations in 44 passes of 40 layers)
    "verify_correlated": Workload("verify_correlated", 9, 5120, 2304, 384, 6, "MIX", "Q8",
                                  use_bias=True, layers=40, rows=(1, 2, 3, 4, 5, 6, 7, 8),
                                  extra={"rho": 0.9}),
}

# Tiers of the residency policy per layer of 384 experts: fast (+1.0), middle
# (0) and slow (-0.6).  [P3 §五.2] keeps ~1,300-1,600 experts in VRAM, ~6,700
# in a pinned RAM arena and the rest (~8,700) on NVMe over 40 layers; per
# layer that is ~36 / ~168 / ~180.  [P3 §五.3]: resident +1.0, NVMe -0.6.
POLICY_TIERS = (36, 168, 180)
POLICY_BIAS = (1.0, 0.0, -0.6)


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
    """The layer's selection bias, or None: the residency policy when the
    workload names a policy scale, else U(-0.6, 1.0) when it uses a bias."""
    if "policy_scale" in wl.extra:
        return policy_bias(wl, layer, wl.extra["policy_scale"])
    if not wl.use_bias:
        return None
    g = rng(wl, layer, T_BIAS)
    return g.uniform(-0.6, 1.0, wl.n_experts).astype(np.float32)


def policy_tiers(wl, layer):
    """Tier (0 fast, 1 middle, 2 slow) of every routed expert: the per-layer
    counts of POLICY_TIERS (scaled to n_experts, remainder to the slow tier)
    placed by a seeded permutation."""
    n = wl.n_experts
    fast = int(np.floor(n * POLICY_TIERS[0] / 384 + 0.5))
    mid = int(np.floor(n * POLICY_TIERS[1] / 384 + 0.5))
    tiers = np.array([0] * fast + [1] * mid + [2] * (n - fast - mid), np.int64)
    return tiers[rng(wl, layer, T_TIER).permutation(n)]


def policy_bias(wl, layer, scale):
    """+1.0 / 0 / -0.6 by tier, times scale, as fp32."""
    b = np.asarray(POLICY_BIAS, np.float64)[policy_tiers(wl, layer)] * scale
    return b.astype(np.float32)


def correlated_x(wl, layer, rows, rho, stream=0):
    """A verify window: rows x_r = rho * x_0 + sqrt(1 - rho^2) * z_r (x_0, z_r
    iid N(0, 1) in fp32, x_0 = z_0), rounded to bf16."""
    g = rng(wl, layer, T_X, 10_000_000 + stream)
    z = g.standard_normal((rows, wl.hidden), dtype=np.float32)
    x = np.float32(rho) * z[:1] + np.float32(np.sqrt(1.0 - rho * rho)) * z
    x[0] = z[0]
    return f32_to_bf16_bits(x)


def correlated_noise(wl, layer, rows, rho):
    """Stack noise for a verify window, correlated across rows like the rows."""
    g = rng(wl, layer, T_NOISE, 1)
    z = g.standard_normal((rows, wl.hidden), dtype=np.float32)
    e = np.float32(rho) * z[:1] + np.float32(np.sqrt(1.0 - rho * rho)) * z
    e[0] = z[0]
    return e


def expert_weights(wl, layer, expert):
    """(gate [I x H], up [I x H], down [H x I]) fp32; expert == n_experts is the shared one."""
    g = rng(wl, layer, T_EXPERT, expert)
    s = np.float32(0.02)
    gate = g.standard_normal((wl.inter, wl.hidden), dtype=np.float32) * s
    up = g.standard_normal((wl.inter, wl.hidden), dtype=np.float32) * s
    down = g.standard_normal((wl.hidden, wl.inter), dtype=np.float32) * s
    return gate, up, down


def mix_counts(n_experts, shares=MIX_SHARES):
    """Exact per-layer counts for the shares; the remainder goes to the last format."""
    counts = [int(np.floor(n_experts * s + 0.5)) for _, s in shares[:-1]]
    counts.append(n_experts - sum(counts))
    return counts


def format_map(wl, layer):
    """List of format names, one per routed expert ("MIX": the ternary / Q2_0 /
    Q3 shares; "MIXALL": all five formats in equal shares)."""
    if wl.routed_fmt not in ("MIX", "MIXALL"):
        return [wl.routed_fmt] * wl.n_experts
    shares = MIX_SHARES if wl.routed_fmt == "MIX" else MIX_ALL_SHARES
    names = []
    for (name, _), c in zip(shares, mix_counts(wl.n_experts, shares)):
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


# Held-out relative output error of an expert per format: ternary, Q2_0, Q3
# ([P1 §1], the GSQ quality proxy: 0.443 / 0.378 / 0.183).
PAGE_ERRORS = (0.443, 0.378, 0.183)
T_ALLOC = 7


def alloc_inputs(wl, n_layers=None, heldout_tokens=61_440, s=1.1):
    """Synthetic inputs of the per-expert format allocation of a stack:
      err [L, E, 3]  PAGE_ERRORS per format x a per-(layer, expert) sensitivity
                     LogNormal(0, 0.35) x a per-(layer, expert, format) factor
                     LogNormal(0, 0.15) x a per-layer factor LogNormal(0, 0.3)
                     (layer 32 of 40 x3: the pages' most sensitive layer);
      tokens [L, E]  held-out tokens per expert: heldout_tokens x top_k pairs
                     per layer over Zipf(s) expert popularity (a seeded
                     permutation per layer);
      energy [L]     the layer's routed output energy, LogNormal(0, 0.5)."""
    L = n_layers or wl.layers
    E = wl.n_experts
    g = rng(wl, 0, T_ALLOC)
    base = np.asarray(PAGE_ERRORS)
    layer_f = g.lognormal(0.0, 0.3, L)
    if L > 32:
        layer_f[32] *= 3.0
    sens = g.lognormal(0.0, 0.35, (L, E))
    per_f = g.lognormal(0.0, 0.15, (L, E, 3))
    err = base[None, None, :] * sens[:, :, None] * per_f * layer_f[:, None, None]
    tokens = np.empty((L, E), np.int32)
    ranks = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    for l in range(L):
        p = np.empty(E)
        p[g.permutation(E)] = np.exp(ranks)
        tokens[l] = g.multinomial(heldout_tokens * wl.top_k, p / p.sum())
    energy = g.lognormal(0.0, 0.5, L)
    return err, tokens, energy


def noise(wl, layer, rows):
    """N(0,1) fp32 [rows x H] added to a layer's output before it feeds the next layer."""
    return rng(wl, layer, T_NOISE).standard_normal((rows, wl.hidden), dtype=np.float32)
