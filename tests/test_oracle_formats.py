"""Pins of oracle.formats: hand-derived blocks, spec tables, brute force, on-grid round trips.

Expected bytes here are built by hand-written loops over the layout
definitions, independent of the oracle's vectorised bit helpers."""

import numpy as np
import pytest

from oracle import formats as F


def _fp16_bytes(v):
    return np.array([v], np.float16).view(np.uint8).tolist()


# ---------------------------------------------------------------- worked blocks
def test_q2_0_worked_block(golden):
    g = golden("worked_blocks.json")["q2_0_block"]
    c = np.arange(64) % 4
    w = (g["d"] * (c - 2.0)).astype(np.float32)[None, :]
    b = F.pack("Q2_0", w)
    assert b[:16].tobytes().hex() == g["code_bytes_hex"]
    assert b[16:].tobytes().hex() == g["scale_bytes_hex"]
    assert np.array_equal(F.decode("Q2_0", b, 1, 64), w.astype(np.float64))


def test_tern160_bytes_worked(golden):
    for trits, byte in golden("worked_blocks.json")["tern160_byte"]["examples"]:
        assert F.tern_byte_trits(byte).tolist() == trits


def test_q8_worked_block(golden):
    g = golden("worked_blocks.json")["q8_block"]
    q = np.array([127] + [i - 16 for i in range(1, 32)])
    w = (g["d"] * q).astype(np.float32)[None, :]
    b = F.pack("Q8", w)
    assert b[:32].tobytes().hex() == g["code_bytes_hex"]
    assert b[32:].tobytes().hex() == g["scale_bytes_hex"]


def test_mxfp4_worked_block(golden):
    g = golden("worked_blocks.json")["mxfp4_block"]
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1] = 6.0, -0.5
    b = F.pack("MXFP4", w)
    assert b[:16].tobytes().hex() == g["code_bytes_hex"]
    assert b[16:].tobytes().hex() == g["scale_bytes_hex"]


# ---------------------------------------------------------------- spec tables
def test_e2m1_table_all_bytes(golden):
    t = golden("ocp_mx_tables.json")["e2m1"]
    table = t["codes_0_to_7"] + t["codes_8_to_15"]
    for e, scale in golden("ocp_mx_tables.json")["e8m0"]["examples"]:
        codes = np.arange(256, dtype=np.uint8)                 # every byte once
        for start in range(0, 256, 16):
            buf = np.concatenate([codes[start:start + 16], np.array([e], np.uint8)])
            got = F.decode("MXFP4", buf, 1, 32)[0]
            for i in range(32):
                byte = int(codes[start + i // 2])
                nib = byte & 15 if i % 2 == 0 else byte >> 4
                assert got[i] == table[nib] * scale


def test_e8m0_nan_rejected():
    buf = np.zeros(17, np.uint8)
    buf[16] = 255
    with pytest.raises(ValueError):
        F.decode("MXFP4", buf, 1, 32)


def test_ternary_bytes_brute_force():
    seen = {}
    for b in range(243):
        t = tuple(F.tern_byte_trits(b).tolist())
        assert all(v in (-1, 0, 1) for v in t)
        assert sum((v + 1) * 3 ** m for m, v in enumerate(t)) == b
        seen[t] = b
    assert len(seen) == 243
    for bad in (243, 250, 255):
        with pytest.raises(ValueError):
            F.tern_byte_trits(bad)


def test_q8_int8_twos_complement():
    buf = np.concatenate([np.arange(224, 256, dtype=np.uint8), np.array(_fp16_bytes(1.0), np.uint8)])
    assert F.decode("Q8", buf, 1, 32)[0].tolist() == list(range(-32, 0))


# ---------------------------------------------------------------- layouts by hand
def _q2_bytes_by_hand(codes):
    out = bytearray(16)
    for i, c in enumerate(codes):
        out[(2 * i) // 8] |= int(c) << ((2 * i) % 8)
    return bytes(out)


def test_q2_0_on_grid_random():
    rng = np.random.default_rng(1)
    n, k = 3, 192
    ds = [-0.25, 0.0078125, -3.0, 0.5, 2.0 ** -14, -0.125, 1.5, -0.75, 0.375]
    w = np.zeros((n, k), np.float32)
    exp_codes, exp_scales = bytearray(), bytearray()
    for r in range(n):
        for b in range(k // 64):
            d = ds[(r * 3 + b) % len(ds)]
            c = rng.integers(1, 4, 64)
            c[rng.integers(0, 64)] = 0                       # the signed absmax element
            # with d < 0 the largest magnitude is d*(0-2) = -2d > 0; with d > 0 it is negative
            w[r, 64 * b:64 * b + 64] = d * (c - 2)
            d_eff = float(np.float16((-2 * d) / -2.0))        # packer: fp16(m / -2)
            assert d_eff == d
            exp_codes += _q2_bytes_by_hand(c)
            exp_scales += bytes(_fp16_bytes(d))
    got = F.pack("Q2_0", w)
    assert got.tobytes() == bytes(exp_codes) + bytes(exp_scales)
    assert np.array_equal(F.decode("Q2_0", got, n, k), w.astype(np.float64))


def test_tern160_on_grid_padded():
    rng = np.random.default_rng(2)
    n, k = 2, 300                                            # pads to 320 = 2 blocks
    d = 0.0625
    t = rng.integers(-1, 2, (n, k))
    t[:, 0] = 1
    t[:, 160] = -1
    w = (d * t).astype(np.float32)
    buf = F.pack("TERN160", w)
    assert buf.size == n * 2 * 34
    tp = np.concatenate([t, np.zeros((n, 20), int)], axis=1)
    exp = bytearray()
    for r in range(n):
        for j in range(64):                                  # 2 blocks x 32 bytes
            exp.append(sum((tp[r, 5 * j + m] + 1) * 3 ** m for m in range(5)))
    assert buf[: n * 64].tobytes() == bytes(exp)
    assert np.array_equal(F.decode("TERN160", buf, n, k), w.astype(np.float64))


def test_q3_on_grid_layout():
    rng = np.random.default_rng(3)
    n, k = 2, 512
    d = 2.0 ** -9
    w = np.zeros((n, k), np.float32)
    exp_lo, exp_hi, exp_d, exp_u = [], [], [], []
    for r in range(n):
        for b in range(k // 256):
            s = rng.integers(-31, 32, 16)
            pick = rng.permutation(16)
            s[pick[0]] = 31 if rng.random() < 0.5 else -31   # max |sigma_j| = 31 d
            s[pick[1]] = 0                                     # one all-zero sub-block
            q = rng.integers(1, 8, (16, 16))
            q[:, 3] = 0                                      # signed absmax at q = 0 in every sub-block
            for j in range(16):
                if s[j] == 0:
                    q[j, :] = 4
            w[r, 256 * b:256 * b + 256] = (d * s[:, None] * (q - 4)).reshape(256)
            qf = q.reshape(256)
            # the layout rule, word by word: quarter u holds six 32-bit words;
            # field f of a word is the 3 bits at 16h + 1 + 3f; pairs 0-2 of
            # every sub-block fill fields 0 then 3 of the words in turn, pairs
            # 3-5 fields 1 then 4, pairs 6-7 field 2, the last two spread
            # their bits over bit 16h of three words
            words = [[0] * 6 for _ in range(4)]
            for i in range(256):
                u, rem = divmod(i, 64)
                j, t = divmod(rem, 16)
                h, pp = divmod(t, 8)
                if pp < 3 or 3 <= pp < 6:
                    cls = 0 if pp < 3 else 1
                    q2 = 3 * j + pp - 3 * cls
                    word, fld = (q2, cls) if q2 < 6 else (q2 - 6, cls + 3)
                    words[u][word] |= int(qf[i]) << (16 * h + 1 + 3 * fld)
                else:
                    q2 = 2 * j + pp - 6
                    if q2 < 6:
                        words[u][q2] |= int(qf[i]) << (16 * h + 1 + 3 * 2)
                    else:
                        for bb in range(3):
                            words[u][3 * (q2 - 6) + bb] |= ((int(qf[i]) >> bb) & 1) << (16 * h)
            code = b"".join(wv.to_bytes(4, "little") for wq in words for wv in wq)
            u = bytearray(12)
            for j in range(16):
                for bb in range(6):
                    pos = 6 * j + bb
                    u[pos // 8] |= (((int(s[j]) + 32) >> bb) & 1) << (pos % 8)
            exp_lo.append(code)
            exp_d.append(bytes(_fp16_bytes(d)))
            exp_u.append(bytes(u))
    buf = F.pack("Q3", w)
    assert buf.tobytes() == b"".join(exp_lo) + b"".join(exp_d) + b"".join(exp_u)
    assert np.array_equal(F.decode("Q3", buf, n, k), w.astype(np.float64))


def test_mxfp4_on_grid_random():
    rng = np.random.default_rng(4)
    n, k = 3, 96
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    w = np.zeros((n, k), np.float32)
    exp_c, exp_s = bytearray(), bytearray()
    for r in range(n):
        for b in range(k // 32):
            e = int(rng.integers(100, 140))
            c = rng.integers(0, 16, 32)
            c[rng.integers(0, 32)] = 7 if rng.random() < 0.5 else 15   # amax in [4, 8) x scale
            c[c == 8] = 0                                     # -0 packs as +0 from a +0.0 weight
            val = np.where(c >= 8, -table[c & 7], table[c & 7]) * 2.0 ** (e - 127)
            w[r, 32 * b:32 * b + 32] = val
            for i in range(0, 32, 2):
                exp_c.append(int(c[i]) | (int(c[i + 1]) << 4))
            exp_s.append(e)
    buf = F.pack("MXFP4", w)
    assert buf.tobytes() == bytes(exp_c) + bytes(exp_s)
    assert np.array_equal(F.decode("MXFP4", buf, n, k), w.astype(np.float64))


def test_mxfp4_rounding_ties_and_saturation():
    # scale 1 (amax 6 -> E 127); probe each midpoint of the e2m1 grid
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 6.0
    w[0, 1:1 + len(mids)] = mids
    w[0, 10] = -0.75
    got = F.decode("MXFP4", F.pack("MXFP4", w), 1, 32)[0]
    assert got[1:1 + len(mids)].tolist() == want
    assert got[10] == -1.0
    # amax 7.9 -> E 127 too (floor(log2 7.9) = 2); 7.9 saturates to 6
    w[0, 0] = 7.9
    assert F.decode("MXFP4", F.pack("MXFP4", w), 1, 32)[0][0] == 6.0


def test_q8_on_grid_random():
    rng = np.random.default_rng(5)
    n, k = 2, 64
    w = np.zeros((n, k), np.float32)
    for r in range(n):
        for b in range(2):
            d = float(np.float16(rng.uniform(0.001, 0.01)))
            q = rng.integers(-127, 128, 32)
            q[rng.integers(0, 32)] = 127 if rng.random() < 0.5 else -127
            w[r, 32 * b:32 * b + 32] = np.float32(d) * q.astype(np.float32)
    buf = F.pack("Q8", w)
    got = F.decode("Q8", buf, n, k)
    # d = fp16(127 d / 127) reproduces d only when 127*d/127 rounds back; check exactness directly
    assert np.array_equal(got, w.astype(np.float64))


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("fmt", F.FORMATS)
def test_idempotence_and_sizes(fmt):
    rng = np.random.default_rng(6)
    n, k = 5, (2304 if fmt == "TERN160" else 1024)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    b1 = F.pack(fmt, w)
    assert b1.size == F.packed_bytes(fmt, n, k)
    d1 = F.decode(fmt, b1, n, k)
    b2 = F.pack(fmt, d1.astype(np.float32))
    assert np.array_equal(F.decode(fmt, b2, n, k), d1)
    # RTN error of each format stays in the range expected from its grid
    err = np.linalg.norm(d1 - w) / np.linalg.norm(w)
    assert err < {"TERN160": 0.9, "Q2_0": 0.5, "Q3": 0.25, "MXFP4": 0.15, "Q8": 0.01}[fmt]


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_zero_matrix(fmt):
    k = 320 if fmt != "Q3" else 512
    w = np.zeros((2, k), np.float32)
    assert not np.any(F.decode(fmt, F.pack(fmt, w), 2, k))


def test_block_multiple_required():
    with pytest.raises(ValueError):
        F.packed_bytes("Q2_0", 1, 100)
    assert F.packed_bytes("TERN160", 1, 100) == 34


def test_q3_layout_hand_worked_bits():
    """One block whose sub-blocks all have the signed absmax -4 (so s * d is
    1 to fp16 rounding and q = w + 4): every code is 4 (value 0) except weight
    0 -> q = 7 (sub-block 0, pair 0, low half: field 0 of word 0, bits 1..3),
    weight 8 -> q = 1 (the same pair's high half: bits 17..19), weight 54 ->
    q = 3 (sub-block 3, pair 6: q' = 6, so bit 0 of words 0, 1, 2) and the
    absmax weights (16 j + 3, and 16 instead of 19) -> q = 0."""
    q = np.full(256, 4)
    q[0], q[8], q[54] = 7, 1, 3
    q[16 * np.arange(16) + 3] = 0      # every sub-block's signed absmax is -4 ...
    q[19], q[16] = 4, 0                # ... sub-block 1 has it at weight 16
    w = (q - 4.0).astype(np.float32).reshape(1, 256)
    buf = F.pack("Q3", w)
    code = buf[:96]
    word = [int.from_bytes(code[4 * i:4 * i + 4].tobytes(), "little") for i in range(24)]
    # sub-block 0, pair 0: weights 0 (low) and 8 (high) at bits 1..3 / 17..19
    assert (word[0] >> 1) & 7 == 7 and (word[0] >> 17) & 7 == 1
    # sub-block 3, pair 6 (t = 6 and 14): weight 54 = 3 = 0b011 -> bit 0 of
    # words 0, 1, 2 = 1, 1, 0; weight 62 = 4 = 0b100 -> bit 16 of words 0, 1,
    # 2 = 0, 0, 1
    assert [(word[b] >> 0) & 1 for b in range(3)] == [1, 1, 0]
    assert [(word[b] >> 16) & 1 for b in range(3)] == [0, 0, 1]
    # weight 3 (q = 0; sub-block 0, pair 3: q' = 0 -> field 1 of word 0, bits
    # 4..6) and weight 35 (q = 0; sub-block 2, pair 3: q' = 6 -> field 4 of
    # word 0, bits 13..15)
    assert (word[0] >> 4) & 7 == 0 and (word[0] >> 13) & 7 == 0
    # weight 19 (q = 4; sub-block 1, pair 3: q' = 3 -> field 1 of word 3)
    assert (word[3] >> 4) & 7 == 4
    # weight 1 (q = 4; sub-block 0, pair 1: q' = 1 -> field 0 of word 1)
    assert (word[1] >> 1) & 7 == 4
    # d = fp16(1 / 31), every s = 31: the decoded values are d * 31 * (q - 4)
    ds = float(np.float16(np.float32(1.0) / np.float32(31.0))) * 31.0
    assert np.array_equal(F.decode("Q3", buf, 1, 256)[0], ds * (q - 4.0))

