"""Independent packers and field-level references for the oracle's pins.

Written from the public GGUF block layout, separately from the oracle's C
unpackers: they go the other way (fields -> bytes), so a misread offset or
bit position in either one shows up as a round-trip mismatch.  Test use only.
"""
import numpy as np


def f16_bits(v):
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


def f16_val(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def pack_q8_0(d_bits, q):
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (32,) and q.min() >= -128 and q.max() <= 127
    out = bytearray(34)
    out[0] = d_bits & 0xFF
    out[1] = d_bits >> 8
    for i in range(32):
        out[2 + i] = int(q[i]) & 0xFF
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def pack_q4_0(d_bits, nib):
    """nib: 32 values in [0, 15] (weight = d * (nib - 8))."""
    nib = [int(v) for v in nib]
    assert len(nib) == 32 and min(nib) >= 0 and max(nib) <= 15
    out = bytearray(18)
    out[0], out[1] = d_bits & 0xFF, d_bits >> 8
    for b in range(16):
        out[2 + b] = nib[b] | (nib[16 + b] << 4)      # weight b low, weight 16 + b high
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def _pack_scales_k(sc, mn):
    """The 12 packed bytes of 8 six-bit scales and mins (Q4_K, Q5_K)."""
    s = bytearray(12)
    for j in range(4):
        # bytes 0..3: scale j in the low 6 bits, top 2 bits of scale j+4 on top
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        # bytes 4..7: min j in the low 6 bits, top 2 bits of min j+4 on top
        s[4 + j] = (mn[j] & 63) | ((mn[j + 4] >> 4) << 6)
        # bytes 8..11: low 4 bits of scale j+4 and of min j+4
        s[8 + j] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    return s


def pack_q5_K(d_bits, dmin_bits, sc, mn, q5):
    """sc, mn: 8 values in [0, 63]; q5: 256 values in [0, 31]."""
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    q5 = [int(v) for v in q5]
    assert len(sc) == 8 and len(mn) == 8 and len(q5) == 256 and min(q5) >= 0 and max(q5) <= 31
    out = bytearray(176)
    out[0], out[1] = d_bits & 0xFF, d_bits >> 8
    out[2], out[3] = dmin_bits & 0xFF, dmin_bits >> 8
    out[4:16] = _pack_scales_k(sc, mn)
    for i in range(256):
        j, l = divmod(i, 32)              # group j, position l in it
        c = j // 2                        # 64-weight chunk: groups 2c (low nibbles) and 2c + 1 (high)
        out[48 + 32 * c + l] |= (q5[i] & 15) << (4 if j & 1 else 0)
        out[16 + l] |= (q5[i] >> 4) << j  # the fifth bits: bit j of byte l
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def pack_q4_K(d_bits, dmin_bits, sc, mn, nib):
    """sc, mn: 8 values in [0, 63]; nib: 256 values in [0, 15]."""
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    nib = [int(v) for v in nib]
    assert len(sc) == 8 and len(mn) == 8 and len(nib) == 256
    out = bytearray(144)
    out[0], out[1] = d_bits & 0xFF, d_bits >> 8
    out[2], out[3] = dmin_bits & 0xFF, dmin_bits >> 8
    out[4:16] = _pack_scales_k(sc, mn)
    for c in range(4):            # 64-weight chunks
        for r in range(32):
            out[16 + 32 * c + r] = nib[64 * c + r] | (nib[64 * c + 32 + r] << 4)
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def pack_q6_K(d_bits, sc, q6):
    """sc: 16 int8 scales; q6: 256 values in [0, 63] (before the -32 offset)."""
    q6 = [int(v) for v in q6]
    assert len(q6) == 256 and len(sc) == 16
    out = bytearray(210)
    for i in range(256):
        h, r = divmod(i, 128)
        g, l = divmod(r, 32)
        lo, hi = q6[i] & 15, q6[i] >> 4
        out[64 * h + 32 * (g & 1) + l] |= lo << (4 if g >= 2 else 0)
        out[128 + 32 * h + l] |= hi << (2 * g)
    for j in range(16):
        out[192 + j] = int(sc[j]) & 0xFF
    out[208], out[209] = d_bits & 0xFF, d_bits >> 8
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def random_fields(t, r):
    """Random field values for one block of type t (2 / 8 / 12 / 13 / 14)."""
    if t == 2:
        return dict(d=f16_bits(r.uniform(1e-3, 2e-2)), nib=r.integers(0, 16, 32))
    if t == 13:
        return dict(d=f16_bits(r.uniform(1e-3, 2e-2)), dmin=f16_bits(r.uniform(1e-3, 2e-2)),
                    sc=r.integers(0, 64, 8), mn=r.integers(0, 64, 8), q5=r.integers(0, 32, 256))
    if t == 8:
        return dict(d=f16_bits(r.uniform(1e-3, 2e-2)), q=r.integers(-128, 128, 32))
    if t == 12:
        return dict(d=f16_bits(r.uniform(1e-3, 2e-2)), dmin=f16_bits(r.uniform(1e-3, 2e-2)),
                    sc=r.integers(0, 64, 8), mn=r.integers(0, 64, 8), nib=r.integers(0, 16, 256))
    if t == 14:
        return dict(d=f16_bits(r.uniform(1e-4, 5e-3)), sc=r.integers(-128, 128, 16), q6=r.integers(0, 64, 256))
    raise ValueError(t)


def pack(t, f):
    if t == 2:
        return pack_q4_0(f["d"], f["nib"])
    if t == 13:
        return pack_q5_K(f["d"], f["dmin"], f["sc"], f["mn"], f["q5"])
    if t == 8:
        return pack_q8_0(f["d"], f["q"])
    if t == 12:
        return pack_q4_K(f["d"], f["dmin"], f["sc"], f["mn"], f["nib"])
    return pack_q6_K(f["d"], f["sc"], f["q6"])


def weights_f64(t, f):
    """Dequantized weights of one block in float64, from the fields."""
    if t == 2:
        return f16_val(f["d"]) * (np.asarray(f["nib"], dtype=np.float64) - 8)
    if t == 13:
        d, dmin = f16_val(f["d"]), f16_val(f["dmin"])
        j = np.arange(256) // 32
        return d * np.asarray(f["sc"], np.float64)[j] * np.asarray(f["q5"], np.float64) \
            - dmin * np.asarray(f["mn"], np.float64)[j]
    if t == 8:
        return f16_val(f["d"]) * np.asarray(f["q"], dtype=np.float64)
    if t == 12:
        d, dmin = f16_val(f["d"]), f16_val(f["dmin"])
        j = np.arange(256) // 32
        return d * np.asarray(f["sc"], np.float64)[j] * np.asarray(f["nib"], np.float64) \
            - dmin * np.asarray(f["mn"], np.float64)[j]
    d = f16_val(f["d"])
    j = np.arange(256) // 16
    return d * np.asarray(f["sc"], np.float64)[j] * (np.asarray(f["q6"], np.float64) - 32)


def dot_quants(t, f):
    """Signed integer weight quants entering the per-group int dot."""
    if t == 2:
        return np.asarray(f["nib"], dtype=np.int64) - 8
    if t == 13:
        return np.asarray(f["q5"], dtype=np.int64)
    if t == 8:
        return np.asarray(f["q"], dtype=np.int64)
    if t == 12:
        return np.asarray(f["nib"], dtype=np.int64)
    return np.asarray(f["q6"], dtype=np.int64) - 32


def parse_q8_1(row):
    """uint8 q8_1 row -> (d fp32 [nb], s fp32 [nb], qs int8 [nb*32])."""
    b = np.asarray(row, dtype=np.uint8).reshape(-1, 40)
    d = b[:, 0:4].copy().view(np.float32).ravel()
    s = b[:, 4:8].copy().view(np.float32).ravel()
    qs = b[:, 8:40].copy().view(np.int8).ravel()
    return d, s, qs
