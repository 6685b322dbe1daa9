"""Oracle: the routed-MoE layer in plain fp64 NumPy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The method, as the pages give it:
  * [P1 §1] the layer: hidden 5120, moe_intermediate 2304, 384 routed
    experts, 1 shared expert, 6 experts per token.
  * [P1 §2] each expert is three 5120 x 2304 matrices (gate, up, down); the
    cost of a token is the bytes of the experts it selects.
  * [P3 §五.3] a selection-only bias changes WHICH experts run; the mixing
    weights stay those of the unbiased router and every expert stays reachable.
  * [P3 §四] prefill runs the experts as dense matrix products.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * scoring: softmax over all experts of the unbiased logits, top-k by
    (logit + bias), weights renormalised over the selected set;
  * the bias is added to the logit, before any softmax;
  * ties in the selection key go to the lower expert id;
  * SwiGLU: h = silu(W_gate x) * (W_up x), silu(z) = z / (1 + e^-z);
  * y = sum over selected e (ascending id) of w_e * W_down,e h_e, plus the
    shared expert with weight 1;
  * prefill activations are quantised to MXFP8 (e4m3, per-32 e8m0 scale)
    before the products.
"""

import numpy as np


# ----------------------------------------------------------------------------
# activations
# ----------------------------------------------------------------------------
def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# router and selection
# ----------------------------------------------------------------------------
def router_logits(x, w_router):
    """logits[r, e] = sum_h x[r, h] * Wr[e, h], in fp64.

    x: fp64 [R, H] (exact bf16 values); w_router: fp32 [E, H].  Every product
    of a bf16 and an fp32 value is exact in fp64, so only summation order
    separates this from any other fp64 evaluation."""
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def select_experts(logits, k, bias=None):
    """Top-k selection with an optional selection-only bias.

    key = logit + b (b = 0 when absent).  The k largest keys are selected,
    ties broken toward the lower expert id, and ordered by (key desc, id asc).
    Mixing weights: p = softmax over ALL experts of the UNBIASED logits,
    w_e = p_e / sum_{j in S} p_j  [P3 §五.3: the bias leaves the mixing
    weights exact].

    Returns idx int64 [R, k], w fp64 [R, k], and min_gap fp64 [R]: the
    smallest difference among adjacent keys in the order (key desc, id asc)
    from the first to the (k+1)-th key (inf when k == E)."""
    logits = np.asarray(logits, np.float64)
    r, e = logits.shape
    if not 1 <= k <= e:
        raise ValueError("top_k must be in [1, E]")
    key = logits + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    ids = np.arange(e)
    idx = np.empty((r, k), np.int64)
    gap = np.full(r, np.inf)
    for i in range(r):
        order = np.lexsort((ids, -key[i]))         # primary: key desc, then id asc
        idx[i] = order[:k]
        ks = key[i, order[: min(k + 1, e)]]
        if ks.size > 1:
            gap[i] = np.min(ks[:-1] - ks[1:])
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    ps = np.take_along_axis(p, idx, axis=1)
    w = ps / ps.sum(axis=1, keepdims=True)
    return idx, w, gap


def route(x, w_router, k, bias=None):
    """Router GEMV followed by selection: returns idx, w, logits, min_gap."""
    logits = router_logits(x, w_router)
    idx, w, gap = select_experts(logits, k, bias)
    return idx, w, logits, gap


# ----------------------------------------------------------------------------
# expert FFN and combine
# ----------------------------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_ffn(x, w_gate, w_up, w_down):
    """SwiGLU expert: o = Wd (silu(Wg x) * (Wu x)), all in fp64.

    x [R, H]; w_gate, w_up [I, H]; w_down [H, I] -> o [R, H]."""
    g = x @ w_gate.T
    v = x @ w_up.T
    return (silu(g) * v) @ w_down.T


def expert_ffn_loops(x, w_gate, w_up, w_down):
    """The same expert as expert_ffn with every sum written as an explicit loop.

    Pure Python; for tiny shapes only.  Used to pin expert_ffn."""
    x = np.asarray(x, np.float64)
    r_, h_ = x.shape
    i_ = w_gate.shape[0]
    out = np.zeros((r_, h_))
    for r in range(r_):
        hvec = [0.0] * i_
        for i in range(i_):
            g = 0.0
            v = 0.0
            for c in range(h_):
                g += w_gate[i, c] * x[r, c]
                v += w_up[i, c] * x[r, c]
            hvec[i] = g / (1.0 + np.exp(-g)) * v
        for n in range(h_):
            acc = 0.0
            for i in range(i_):
                acc += w_down[n, i] * hvec[i]
            out[r, n] = acc
    return out


def combine_outputs(shape, idx, w, outputs, shared_out=None):
    """The weighted sum of given expert outputs:
    y_r = sum_{e in S_r, ascending e} w_{r,e} * outputs[e][i]  +  shared_out[r],
    where outputs[e][i] is expert e's output for the i-th row that selects e
    (rows in ascending order, as np.nonzero(idx == e) lists them)."""
    y = np.zeros(shape)
    w = np.asarray(w, np.float64)
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        y[rows] += w[rows, slots][:, None] * outputs[int(e)]
    if shared_out is not None:
        y += shared_out
    return y


def combine(x, idx, w, expert_fn, shared=None):
    """y_r = sum_{e in S_r, ascending e} w_{r,e} * E_e(x_r)  +  shared(x_r).

    expert_fn(e) -> (Wg, Wu, Wd) decoded fp64 matrices; it is called once per
    distinct selected expert.  shared: (Wg, Wu, Wd) or None."""
    x = np.asarray(x, np.float64)
    outs = {}
    for e in np.unique(idx):
        rows, _ = np.nonzero(idx == e)
        outs[int(e)] = expert_ffn(x[rows], *expert_fn(int(e)))
    return combine_outputs(x.shape, idx, w, outs,
                           expert_ffn(x, *shared) if shared is not None else None)


def moe_layer(x, w_router, k, expert_fn, shared=None, bias=None):
    """One MoE layer: route, then the weighted sum of the selected experts.

    Returns dict(idx, w, y, logits, min_gap, unique)."""
    idx, w, logits, gap = route(x, w_router, k, bias)
    y = combine(x, idx, w, expert_fn, shared)
    return dict(idx=idx, w=w, y=y, logits=logits, min_gap=gap, unique=np.unique(idx))


def dense_moe(x, w_router, expert_list, shared=None):
    """All experts computed and mixed by the full softmax (top_k = E, no bias).

    The dense special case of moe_layer, written without any selection."""
    logits = router_logits(x, w_router)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    y = sum(p[:, e:e + 1] * expert_ffn(x, *m) for e, m in enumerate(expert_list))
    if shared is not None:
        y = y + expert_ffn(x, *shared)
    return y


# ----------------------------------------------------------------------------
# MXFP8 activations (prefill path)
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def round_e4m3(v):
    """fp64 values -> nearest OCP e4m3 (FN) value, ties to even, saturating at 448.

    Normal range: quantum 2^(e-3) for |v| in [2^e, 2^(e+1)), e >= -6;
    below 2^-6 the subnormal quantum 2^-9."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, e - 3)
    r = np.rint(a / q) * q
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, v)


def quant_mxfp8(x):
    """Per 32 consecutive elements of a row: E = floor(log2(amax)) - 8 + 127,
    clamped to [0, 254] (amax = 0 gives E = 0); elements e4m3_RNE(x / 2^(E-127)).

    Returns (dequantised fp64 values, E int64 [R, K/32])."""
    x = np.asarray(x, np.float64)
    r, k = x.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    blk = x.reshape(r, k // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, ex - 1 - 8 + 127, 0)
    e = np.clip(e, 0, 254)
    s = np.ldexp(1.0, e - 127)[..., None]
    return (round_e4m3(blk / s) * s).reshape(r, k), e


# ----------------------------------------------------------------------------
# prefill (many rows, MXFP4 experts on scaled matrix cores)
# ----------------------------------------------------------------------------
def prefill_layer(x, idx, w, expert_fn):
    """y[r] = sum over the row's experts in ascending id of w * FFN_e(Q(x_r)),
    Q = MXFP8 of the bf16 activations (the matrix cores take them as fp8),
    FFN_e the SwiGLU expert in fp64 (h is not re-quantised).  x fp64 [R x H]
    (exact bf16 values); expert_fn(e) -> decoded (gate, up, down)."""
    x = np.asarray(x, np.float64)
    xq, _ = quant_mxfp8(x)
    y = np.zeros_like(x)
    idx = np.asarray(idx)
    for e in sorted(set(idx.reshape(-1).tolist())):
        rows, cols = np.nonzero(idx == e)
        o = expert_ffn(xq[rows], *expert_fn(e))
        y[rows] += np.asarray(w, np.float64)[rows, cols][:, None] * o
    return y


def many_row_layer(x, idx, w, expert_fn, fmt_of, act_mxfp8, shared=None):
    """The many-row call for a given routing, with experts of any format.

    y[r] = sum over the row's experts in ascending id of w * FFN_e(x_e[r])
           + FFN_shared(x[r]) (weight 1, when there is a shared expert),
    where x_e = Q_MXFP8(x) for an MXFP4 expert when act_mxfp8 is set (those
    experts run on the fp8 x fp4 matrix cores) and x_e = x otherwise (the
    decode tiles, on unquantised activations; the shared expert always).
    The pages run prefill as matrix products ([P3 §四]); which activations
    each expert sees follows the library's flag and is this reading's choice.
    fmt_of(e) -> format name of routed expert e."""
    x = np.asarray(x, np.float64)
    xq = quant_mxfp8(x)[0] if act_mxfp8 else None
    y = np.zeros_like(x)
    idx = np.asarray(idx)
    wv = np.asarray(w, np.float64)
    for e in sorted(set(idx.reshape(-1).tolist())):
        rows, cols = np.nonzero(idx == e)
        xin = xq if (act_mxfp8 and fmt_of(e) == "MXFP4") else x
        y[rows] += wv[rows, cols][:, None] * expert_ffn(xin[rows], *expert_fn(e))
    if shared is not None:
        y += expert_ffn(x, *shared)
    return y


# ----------------------------------------------------------------------------
# stacked decode
# ----------------------------------------------------------------------------
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(v):
    """fp64 values -> nearest bf16 value, ties to the even significand.

    A bf16 keeps 8 significant bits: quantum 2^(e-7) for |v| in [2^e, 2^(e+1))
    with e >= -126, the subnormal quantum 2^-133 below 2^-126.  A result past
    the largest finite bf16 is infinite (IEEE round to nearest)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -126)
    q = np.ldexp(1.0, e - 7)
    r = np.rint(a / q) * q                  # a / q is exact; rint ties to even
    r = np.where(r > BF16_MAX, np.inf, r)
    return np.copysign(r, v)


def chain_next(y, eps):
    """The next layer's input in a stacked decode (the workload feeds each
    layer's output plus Gaussian noise to the next layer).

    v = y + eps, one IEEE fp32 addition per element (y, eps fp32, [R, H] or
    one row [H]); per row, when the largest |v| is 4 or more, v is divided by
    2^s with s = floor(log2 max|v|) - 1, which brings that largest value into
    [2, 4) (s = 0 for a row holding a NaN or an infinity); then bf16, round to
    nearest even.  Returns fp64 values.

    Reading: a trained stack keeps every layer's input bounded (its layers
    normalise their inputs).  Synthetic N(0, 0.02^2) SwiGLU experts have a
    gain above one and a quadratic response: chained unbounded, x overflows
    bf16 within a few layers and the routing degenerates.  Dividing by a power
    of two chosen from the row's maximum is exact and does not depend on any
    summation order."""
    s = np.asarray(y, np.float32) + np.asarray(eps, np.float32)
    v = s.astype(np.float64)
    rows = np.atleast_2d(v)
    out = np.empty_like(rows)
    for r in range(rows.shape[0]):
        with np.errstate(invalid="ignore"):
            m = np.max(np.abs(rows[r]))
        sh = 0
        if np.isfinite(m) and m >= 4.0:
            _, ex = np.frexp(m)             # m = f * 2^ex, f in [0.5, 1): floor(log2 m) = ex - 1
            sh = int(ex) - 2
        out[r] = round_bf16(np.ldexp(rows[r], -sh))
    return out.reshape(v.shape)
