"""Pins of oracle.sizes against the byte arithmetic the pages print."""

import pytest

from oracle import formats as F
from oracle import sizes as S


def test_model_shape_params(golden):
    g = golden("pages_arithmetic.json")["model_shape"]
    # 3 matrices of 5120 x 2304 (the page's own statement of the expert)
    assert S.params_per_expert(g["hidden"], g["inter"]) == 3 * 5120 * 2304 == 35_389_440


def test_fp4_expert_and_token_bytes(golden):
    gp = golden("pages_arithmetic.json")
    m = gp["model_shape"]
    e = gp["fp4_expert_MB"]
    b = S.expert_bytes_at(m["hidden"], m["inter"], e["bytes_per_param"])
    assert b == 17_694_720
    assert abs(b / 1e6 - e["value"]) <= e["abs_tol"]
    t = gp["fp4_bytes_per_token_GB"]
    bt = S.bytes_per_token(m["hidden"], m["inter"], m["top_k"], m["layers"], 0.5)
    assert bt == 4_246_732_800
    assert abs(bt / 1e9 - t["value"]) <= t["abs_tol"]
    a = gp["fp4_all_experts_GB"]
    assert a["n_experts_total"] == m["layers"] * m["n_experts"]
    assert abs(a["n_experts_total"] * b / 1e9 - a["value"]) <= a["abs_tol"]


def test_decode_ceilings(golden):
    g = golden("pages_arithmetic.json")["decode_ceilings"]
    for row in g["rows"]:
        t, tok = S.decode_ceiling(g["bytes_per_token_GB"] * 1e9, row["GBps"] * 1e9)
        assert t * 1e3 == pytest.approx(row["ms"], rel=g["rel_tol"])
        assert tok == pytest.approx(row["tok_s"], rel=g["rel_tol"])


def test_mixed_average_and_gsq_size(golden):
    gp = golden("pages_arithmetic.json")
    mix = gp["mixed_average_bpw"]
    avg = S.mixed_average_bpw([(s, b) for _, s, b in mix["shares"]])
    assert abs(avg - mix["value"]) <= mix["abs_tol"]
    gs = gp["gsq_size_GB"]
    assert abs(gs["params"] * gs["bpw"] / 8 / 1e9 - gs["value"]) <= gs["abs_tol"]


def test_format_bit_rates(golden):
    g = golden("pages_arithmetic.json")["format_bpw"]
    assert F.bits_per_weight("Q2_0") == g["Q2_0"]
    assert abs(F.bits_per_weight("Q3") - g["Q3"]) <= g["Q3_abs_tol"]
    # the library's ternary block: 32 bytes for 160 trits (5 per byte) + fp16 scale
    assert F.bits_per_weight("TERN160") == 34 * 8 / 160 == 1.7
    assert F.bits_per_weight("MXFP4") == 17 * 8 / 32 == 4.25
    assert F.bits_per_weight("Q8") == 34 * 8 / 32 == 8.5


def test_real_shape_expert_bytes():
    # gate/up: 2304 rows x 80 blocks; down: 5120 rows x 36 blocks (18 B per Q2_0 block)
    assert S.packed_expert_bytes("Q2_0", 5120, 2304) == 2 * 2304 * 80 * 18 + 5120 * 36 * 18 == 9_953_280
    # ternary down rows pad 2304 -> 2400 (15 blocks of 160)
    assert F.packed_bytes("TERN160", 5120, 2304) == 5120 * 15 * 34 == 2_611_200
    assert S.packed_expert_bytes("TERN160", 5120, 2304) == 7_624_704
    assert S.packed_expert_bytes("Q3", 5120, 2304) == 15_206_400
    assert S.packed_expert_bytes("MXFP4", 5120, 2304) == 18_800_640
    assert S.packed_expert_bytes("Q8", 5120, 2304) == 37_601_280
    # one decode row of the Q2_0 layer with an int8 shared expert
    assert S.layer_pass_bytes(5120, 2304, 384, ["Q2_0"] * 6, "Q8", rows=1) == \
        384 * 5120 * 4 + 6 * 9_953_280 + 37_601_280 + 5120 * 6


def test_mix_counts():
    assert S.format_counts(384, [0.428, 0.392, 0.180]) == [164, 151, 69]
