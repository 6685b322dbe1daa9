"""Oracle: the pages' byte arithmetic.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[P1 §2] reduces decode cost to expert-weight bytes moved per token: one
expert is 3 x hidden x intermediate parameters, a token touches top_k
experts in each of the layers, and a channel of bandwidth B gives a decode
ceiling of B / (bytes per token).  [P3 §五.1] gives the mixed-format average
as the share-weighted mean of the format bit rates; [P3 §三] reconciles the
expert parameter count with the file size at that average.
"""

import numpy as np

from . import formats


def params_per_expert(hidden, inter):
    """gate (inter x hidden) + up (inter x hidden) + down (hidden x inter)."""
    return 3 * hidden * inter


def expert_bytes_at(hidden, inter, bytes_per_param):
    """Bytes of one expert at a flat bytes-per-parameter rate (scales ignored)."""
    return params_per_expert(hidden, inter) * bytes_per_param


def bytes_per_token(hidden, inter, top_k, layers, bytes_per_param):
    return top_k * layers * expert_bytes_at(hidden, inter, bytes_per_param)


def decode_ceiling(bytes_token, bandwidth):
    """(seconds per token, tokens per second) for a channel of `bandwidth` B/s."""
    t = bytes_token / bandwidth
    return t, 1.0 / t


def mixed_average_bpw(shares_and_bpw):
    """Share-weighted mean bit rate: sum share_f * bpw_f."""
    return float(sum(s * b for s, b in shares_and_bpw))


def packed_expert_bytes(fmt, hidden, inter):
    """Exact bytes of one packed expert in `fmt` (gate + up + down)."""
    return (2 * formats.packed_bytes(fmt, inter, hidden)
            + formats.packed_bytes(fmt, hidden, inter))


def layer_pass_bytes(hidden, inter, n_experts, unique_fmts, shared_fmt=None, rows=1):
    """Algorithmic bytes of one layer pass: fp32 router + the distinct
    selected experts + the shared expert + bf16 x in and fp32 y out."""
    b = 4 * n_experts * hidden
    b += sum(packed_expert_bytes(f, hidden, inter) for f in unique_fmts)
    if shared_fmt is not None:
        b += packed_expert_bytes(shared_fmt, hidden, inter)
    return b + rows * hidden * (2 + 4)


def format_counts(n_experts, shares):
    """Per-layer expert counts for shares (rounded; the remainder goes to the last)."""
    counts = [int(np.floor(n_experts * s + 0.5)) for s in shares[:-1]]
    counts.append(n_experts - sum(counts))
    return counts
