"""Oracle: packed low-bit weight formats -- RTN packers and exact fp64 decoders.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Independent of the HIP
library: the byte layouts below are implemented here from their definition,
not from the library's packer.

What the pages fix, and what this module adds
---------------------------------------------
[P3 §五.1] lists the per-expert formats and their bit rates: ternary {-1,0,+1}
at 1.75 bpw (5 trits per byte, [P3 §一]), Q2_0 at 2.25 bpw, Q3_K at 3.44 bpw,
mixed to a 2.250 average.  [P1 §1] says the routed experts of the FP8
checkpoint are FP4 with a per-32 distribution; [P3 §二] keeps the dense half
as Q8_0.  The pages give names and bit rates only; the block structure and the
bit order below are this library's own definitions:

  Q2_0    64 weights / block: 16 code bytes + fp16 d.  Weight i of the block
          is the 2-bit field at bits [2i, 2i+2) of the block's 128-bit
          little-endian code word; value = d * (c - 2).            2.25 bpw
  TERN160 160 weights / block: 32 code bytes + fp16 d.  Byte j holds weights
          5j..5j+4 as sum_m (t_{5j+m} + 1) * 3^m (bytes 243..255 invalid);
          value = d * t.  A row whose length is not a multiple of 160 is
          padded with zero trits to the next block.               1.7 bpw
  Q3      256 weights / block = 16 sub-blocks of 16: 96 code bytes, fp16 d,
          and 12 bytes of sixteen 6-bit sub-scales u_j at bits [6j, 6j+6).
          The 3-bit codes q are laid out by quarter block (64 weights, four
          sub-blocks, 24 bytes = six little-endian 32-bit words W0..W5 at
          byte 24u).  Weight t of the quarter's sub-block j lies in half
          h = t div 8 of pair i = t mod 8.  Field f of a word is the 3 bits
          at 16h + 1 + 3f.  Pairs i < 3: q' = 3j + i, field 0 (q' < 6) or 3
          of word q' mod 6; pairs 3 <= i < 6: q' = 3j + i - 3, field 1 or 4
          likewise; pairs i >= 6: q' = 2j + i - 6, field 2 of word q' for
          q' < 6, else code bit b is bit 16h of word 3(q' - 6) + b.
          value = d * (u_j - 32) * (q - 4).                    3.4375 bpw
  MXFP4   32 weights / block: 16 code bytes (element i in byte i/2, low nibble
          for even i) + one e8m0 byte E.  value = 2^(E-127) * e2m1(c), with
          e2m1 = sign * {0, .5, 1, 1.5, 2, 3, 4, 6}[c & 7] (OCP MX v1.0);
          E = 255 is NaN (invalid here).                          4.25 bpw
  Q8      32 weights / block: 32 int8 codes + fp16 d; value = d * q.  8.5 bpw

Every matrix W[N x K] is stored planar: first a codes plane with blocks in
(row, block) order, then a scales plane in the same order.  The Q3 scales
plane is itself two sub-planes: all fp16 d values, then all 12-byte sub-scale
records.  Total bytes = N * nb * (code bytes + scale bytes), nb = ceil(K / B).

Packers: round-to-nearest from fp32 weights, all arithmetic in IEEE fp32 with
ties to even (np.rint) and fp16 conversion by round-to-nearest-even,
saturating at +-65504.  They only decide which bytes are produced; parity
never depends on them because both sides decode the same bytes.
Decoders: exact in fp64 (a few-bit integer times an fp16 or power-of-two scale).
"""

import numpy as np

FORMATS = ("TERN160", "Q2_0", "Q3", "MXFP4", "Q8")

# weights per block, code bytes per block, scale bytes per block
BLOCK = {"Q2_0": 64, "TERN160": 160, "Q3": 256, "MXFP4": 32, "Q8": 32}
CODE_BYTES = {"Q2_0": 16, "TERN160": 32, "Q3": 96, "MXFP4": 16, "Q8": 32}
SCALE_BYTES = {"Q2_0": 2, "TERN160": 2, "Q3": 14, "MXFP4": 1, "Q8": 2}

# OCP Microscaling Formats v1.0, e2m1 element magnitudes for codes 0..7
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
FP16_MAX = np.float32(65504.0)


# ----------------------------------------------------------------------------
# sizes
# ----------------------------------------------------------------------------
def blocks_per_row(fmt, k):
    """nb = ceil(K / B); only TERN160 ever pads (K is a block multiple otherwise)."""
    b = BLOCK[fmt]
    if fmt != "TERN160" and k % b:
        raise ValueError(f"{fmt}: K={k} is not a multiple of {b}")
    return -(-k // b)


def packed_bytes(fmt, n, k):
    """Bytes of one packed N x K matrix: N * nb * (code + scale bytes)."""
    return n * blocks_per_row(fmt, k) * (CODE_BYTES[fmt] + SCALE_BYTES[fmt])


def bits_per_weight(fmt):
    return 8.0 * (CODE_BYTES[fmt] + SCALE_BYTES[fmt]) / BLOCK[fmt]


# ----------------------------------------------------------------------------
# small helpers (fp32 arithmetic, as the packers define it)
# ----------------------------------------------------------------------------
def _fp16_sat(v32):
    """fp32 -> fp16, round to nearest even, saturating at +-65504."""
    return np.clip(np.asarray(v32, np.float32), -FP16_MAX, FP16_MAX).astype(np.float16)


def _signed_absmax(blocks):
    """Per block (last axis), the element of largest magnitude, sign kept.

    On equal magnitudes the first such element (lowest index) is taken."""
    j = np.argmax(np.abs(blocks), axis=-1)
    return np.take_along_axis(blocks, j[..., None], axis=-1)[..., 0]


def _div_or(w, d, fallback):
    """w / d in fp32, elementwise; where d == 0 the result is `fallback`."""
    d = np.asarray(d, np.float32)
    safe = np.where(d == 0, np.float32(1), d).astype(np.float32)
    q = (np.asarray(w, np.float32) / safe).astype(np.float32)
    return np.where(d == 0, np.float32(fallback), q)


def _blocks(w, fmt):
    """[N, K] fp32 -> [N, nb, B] fp32 (TERN160 rows zero-padded)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    nb, b = blocks_per_row(fmt, k), BLOCK[fmt]
    if nb * b != k:
        w = np.concatenate([w, np.zeros((n, nb * b - k), np.float32)], axis=1)
    return w.reshape(n, nb, b)


def _bits_to_bytes(bits):
    """[..., nbits] of 0/1 -> [..., nbits/8] uint8, little-endian bit order."""
    return np.packbits(bits.astype(np.uint8), axis=-1, bitorder="little")


def _bytes_to_bits(by):
    return np.unpackbits(by, axis=-1, bitorder="little")


def _fields_to_bytes(vals, width):
    """[..., m] unsigned fields of `width` bits, field j at bits [j*width, ...)."""
    sh = np.arange(width, dtype=np.uint32)
    bits = (vals.astype(np.uint32)[..., None] >> sh) & 1
    return _bits_to_bytes(bits.reshape(*vals.shape[:-1], vals.shape[-1] * width))


def _bytes_to_fields(by, width, m):
    bits = _bytes_to_bits(by)[..., : m * width].reshape(*by.shape[:-1], m, width)
    return (bits.astype(np.int64) << np.arange(width)).sum(axis=-1)


def _planar(codes, scales):
    """codes [N, nb, CB] uint8, scales [N, nb, SB] uint8 -> flat planar bytes."""
    return np.concatenate([codes.reshape(-1), scales.reshape(-1)])


def _split(buf, fmt, n, k):
    buf = np.frombuffer(np.asarray(buf, np.uint8).tobytes(), np.uint8)
    nb = blocks_per_row(fmt, k)
    if buf.size != packed_bytes(fmt, n, k):
        raise ValueError(f"{fmt}: got {buf.size} bytes, expected {packed_bytes(fmt, n, k)}")
    cb = CODE_BYTES[fmt]
    codes = buf[: n * nb * cb].reshape(n, nb, cb)
    return codes, buf[n * nb * cb:], nb


# ----------------------------------------------------------------------------
# Q2_0
# ----------------------------------------------------------------------------
def pack_q2_0(w):
    """RTN: m = signed absmax, d = fp16(m / -2), c = clamp(rint(w/d) + 2, 0, 3)."""
    blk = _blocks(w, "Q2_0")
    m = _signed_absmax(blk)
    d = _fp16_sat(m / np.float32(-2.0))
    q = _div_or(blk, d.astype(np.float32)[..., None], 0.0)
    c = np.clip(np.rint(q) + 2, 0, 3).astype(np.uint32)
    codes = _fields_to_bytes(c, 2)                        # [N, nb, 16]
    scales = d.view(np.uint8).reshape(*d.shape, 2)
    return _planar(codes, scales)


def decode_q2_0(buf, n, k):
    codes, rest, nb = _split(buf, "Q2_0", n, k)
    d = rest.view("<f2").reshape(n, nb).astype(np.float64)
    c = _bytes_to_fields(codes, 2, 64).astype(np.float64)
    return (d[..., None] * (c - 2.0)).reshape(n, nb * 64)


# ----------------------------------------------------------------------------
# TERN160
# ----------------------------------------------------------------------------
_POW3 = np.array([1, 3, 9, 27, 81], np.int64)


def pack_tern160(w):
    """RTN: d = fp16(max|w|), t = clamp(rint(w/d), -1, 1); padding trits are 0."""
    blk = _blocks(w, "TERN160")
    d = _fp16_sat(np.max(np.abs(blk), axis=-1))
    q = _div_or(blk, d.astype(np.float32)[..., None], 0.0)
    t = np.clip(np.rint(q), -1, 1).astype(np.int64)
    codes = ((t.reshape(*t.shape[:-1], 32, 5) + 1) * _POW3).sum(axis=-1).astype(np.uint8)
    scales = d.view(np.uint8).reshape(*d.shape, 2)
    return _planar(codes, scales)


def tern_byte_trits(byte_values):
    """Byte value(s) -> the five trits t_0..t_4 in {-1, 0, 1} (last axis)."""
    b = np.asarray(byte_values, np.int64)
    if np.any(b > 242) or np.any(b < 0):
        raise ValueError("TERN160: byte value above 242 is not a valid code")
    return (b[..., None] // _POW3) % 3 - 1


def decode_tern160(buf, n, k):
    codes, rest, nb = _split(buf, "TERN160", n, k)
    d = rest.view("<f2").reshape(n, nb).astype(np.float64)
    t = tern_byte_trits(codes).reshape(n, nb, 160).astype(np.float64)
    return (d[..., None] * t).reshape(n, nb * 160)[:, :k]


# ----------------------------------------------------------------------------
# Q3
# ----------------------------------------------------------------------------
def _q3_code_bits(i):
    """The three bit indices (code bit 0, 1, 2) of weight i of a block inside
    its 768-bit code string."""
    u, w = divmod(i, 64)
    j, t = divmod(w, 16)
    h, pr = divmod(t, 8)
    base = 192 * u
    if pr < 6:
        q = 3 * j + pr % 3
        m, f = q % 6, (pr // 3) + (0 if q < 6 else 3)
    else:
        q = 2 * j + pr - 6
        if q >= 6:
            return [base + 32 * (3 * (q - 6) + b) + 16 * h for b in range(3)]
        m, f = q, 2
    return [base + 32 * m + 16 * h + 1 + 3 * f + b for b in range(3)]


_Q3_BITS = np.array([_q3_code_bits(i) for i in range(256)])            # [256, 3]


def pack_q3(w):
    """RTN with a two-level scale.

    sigma_j = m_j / -4 (m_j the signed absmax of sub-block j); d = fp16(max_j
    |sigma_j| / 31); u_j = clamp(rint(sigma_j / d), -31, 31) + 32; s_j = u_j - 32;
    q = clamp(rint(w / (d * s_j)) + 4, 0, 7); zero divisors give u = 32, q = 4.
    """
    blk = _blocks(w, "Q3")                               # [N, nb, 256]
    sub = blk.reshape(*blk.shape[:-1], 16, 16)
    sigma = (_signed_absmax(sub) / np.float32(-4.0)).astype(np.float32)   # [N, nb, 16]
    d = _fp16_sat(np.max(np.abs(sigma), axis=-1) / np.float32(31.0))
    s = np.clip(np.rint(_div_or(sigma, d.astype(np.float32)[..., None], 0.0)), -31, 31)
    u = (s + 32).astype(np.uint32)
    ds = (d.astype(np.float32)[..., None] * s.astype(np.float32)).astype(np.float32)
    q = np.clip(np.rint(_div_or(sub, ds[..., None], 0.0)) + 4, 0, 7).astype(np.uint32)
    q = q.reshape(*blk.shape)
    bits = np.zeros((*q.shape[:-1], 768), np.uint8)
    for b in range(3):
        bits[..., _Q3_BITS[:, b]] = (q >> b) & 1
    codes = _bits_to_bytes(bits)                          # [N, nb, 96]
    d_plane = d.view(np.uint8).reshape(-1)
    u_plane = _fields_to_bytes(u, 6).reshape(-1)          # 12 bytes per block
    return np.concatenate([codes.reshape(-1), d_plane, u_plane])


def decode_q3(buf, n, k):
    codes, rest, nb = _split(buf, "Q3", n, k)
    d = rest[: n * nb * 2].view("<f2").reshape(n, nb).astype(np.float64)
    u = _bytes_to_fields(rest[n * nb * 2:].reshape(n, nb, 12), 6, 16)    # [N, nb, 16]
    bits = _bytes_to_bits(codes).astype(np.int64)                         # [N, nb, 768]
    q = sum(bits[..., _Q3_BITS[:, b]] << b for b in range(3))             # [N, nb, 256]
    s = (u - 32).astype(np.float64)
    val = d[..., None, None] * s[..., None] * (q.reshape(n, nb, 16, 16) - 4.0)
    return val.reshape(n, nb * 256)


# ----------------------------------------------------------------------------
# MXFP4 (OCP MX v1.0: e2m1 elements, e8m0 shared scale per 32)
# ----------------------------------------------------------------------------
def _floor_log2(a32):
    """floor(log2(a)) of positive finite fp32 values, exactly (frexp exponent - 1)."""
    _, e = np.frexp(np.asarray(a32, np.float64))
    return e.astype(np.int64) - 1


def _round_e2m1(v):
    """fp32 values already divided by the block scale -> e2m1 codes (RNE, saturating).

    Nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}; on a tie the code with even mantissa
    bit (even code) wins; magnitudes above 6 saturate to 6.  Sign = sign bit."""
    a = np.abs(v).astype(np.float64)
    dist = np.abs(a[..., None] - E2M1)                    # [..., 8]
    best = np.argmin(dist, axis=-1)
    # tie: both neighbours equally near -> prefer the even code
    dmin = np.take_along_axis(dist, best[..., None], axis=-1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    tie = (np.take_along_axis(dist, nxt[..., None], axis=-1)[..., 0] == dmin) & (nxt != best)
    best = np.where(tie & (best % 2 == 1), nxt, best)
    best = np.where(a > 6.0, 7, best)
    sign = np.signbit(v).astype(np.int64)
    return (best + 8 * sign).astype(np.uint8)


def pack_mxfp4(w):
    """E = clamp(floor(log2(amax)) - 2 + 127, 0, 254) (amax = 0 gives E = 0);
    element = e2m1_RNE(w / 2^(E-127)), saturating at +-6."""
    blk = _blocks(w, "MXFP4")
    amax = np.max(np.abs(blk), axis=-1)
    e = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1)) - 2 + 127, 0)
    e = np.clip(e, 0, 254)
    scale = np.ldexp(np.float64(1.0), e - 127)
    v = (blk.astype(np.float64) / scale[..., None]).astype(np.float32)   # exact (power of 2)
    c = _round_e2m1(v).astype(np.uint32)                                 # [N, nb, 32]
    codes = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)        # [N, nb, 16]
    return _planar(codes, e.astype(np.uint8)[..., None])


def decode_mxfp4(buf, n, k):
    codes, rest, nb = _split(buf, "MXFP4", n, k)
    e = rest.reshape(n, nb).astype(np.int64)
    if np.any(e == 255):
        raise ValueError("MXFP4: e8m0 scale 0xFF (NaN) is not a valid code")
    c = np.empty((n, nb, 32), np.int64)
    c[..., 0::2] = codes & 15
    c[..., 1::2] = codes >> 4
    mag = E2M1[c & 7]
    val = np.where(c >= 8, -mag, mag) * np.ldexp(1.0, e - 127)[..., None]
    return val.reshape(n, nb * 32)


# ----------------------------------------------------------------------------
# Q8
# ----------------------------------------------------------------------------
def pack_q8(w):
    """RTN: d = fp16(max|w| / 127), q = clamp(rint(w/d), -127, 127)."""
    blk = _blocks(w, "Q8")
    d = _fp16_sat(np.max(np.abs(blk), axis=-1) / np.float32(127.0))
    q = np.clip(np.rint(_div_or(blk, d.astype(np.float32)[..., None], 0.0)), -127, 127)
    codes = q.astype(np.int8).view(np.uint8)
    scales = d.view(np.uint8).reshape(*d.shape, 2)
    return _planar(codes, scales)


def decode_q8(buf, n, k):
    codes, rest, nb = _split(buf, "Q8", n, k)
    d = rest.view("<f2").reshape(n, nb).astype(np.float64)
    q = codes.view(np.int8).astype(np.float64)
    return (d[..., None] * q).reshape(n, nb * 32)


_PACK = {"Q2_0": pack_q2_0, "TERN160": pack_tern160, "Q3": pack_q3,
         "MXFP4": pack_mxfp4, "Q8": pack_q8}
_DECODE = {"Q2_0": decode_q2_0, "TERN160": decode_tern160, "Q3": decode_q3,
           "MXFP4": decode_mxfp4, "Q8": decode_q8}


def pack(fmt, w):
    """fp32 [N, K] -> planar packed bytes (uint8 array)."""
    out = _PACK[fmt](np.asarray(w, np.float32))
    assert out.size == packed_bytes(fmt, *np.shape(w))
    return out


def decode(fmt, buf, n, k):
    """Planar packed bytes -> exact fp64 [N, K]."""
    return _DECODE[fmt](buf, n, k)
