"""Brute-force statement of the codec, independent of the oracle's code.

Used only to pin the oracle on small inputs.  Every rounding decision is an
argmin over all candidate codes with exact rational arithmetic
(``fractions.Fraction``); binary32 / binary16 arithmetic goes through numpy
scalars (IEEE), the E4M3 value table through torch's ``float8_e4m3fn``.  Tile
layouts are written at the 32-bit-word level, the INT3 planes as bit-plane
splits of per-group nibble words, which is a different description from the
oracle's per-element bit positions.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

TILE, BLOCK = 2048, 32


def _e4m3_table():
    import torch
    vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return [Fraction(float(v)) for v in vals]


E4M3 = _e4m3_table()
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def nearest_code(q: Fraction, table) -> int:
    """argmin_c |q - table[c]|, ties to the even code (table increasing)."""
    best, bestd = 0, abs(q - table[0])
    for c in range(1, len(table)):
        d = abs(q - table[c])
        if d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best


def int_mag(v: float, s: float, qmax: int) -> int:
    """The nearest of 0..qmax to the exact rational |v| / s, ties to the even
    integer (an argmin over every candidate)."""
    q = Fraction(abs(float(np.float32(v)))) / Fraction(float(s))
    return nearest_code(q, [Fraction(k) for k in range(qmax + 1)])


def int_scale(a: np.float32, qmax: int) -> np.float16:
    s32 = np.float32(a) / np.float32(qmax)
    if s32 > np.float32(65504.0):
        s32 = np.float32(65504.0)
    return np.float16(s32)


def fp8_scale(a: np.float32) -> np.float32:
    s = np.float32(a) / np.float32(448.0)
    return np.float32(0.0) if s < np.finfo(np.float32).tiny else s


def mx_exponent(a: float) -> int:
    if a == 0:
        return -127
    fa = Fraction(float(a))
    e = -160
    while Fraction(2) ** (e + 1) <= fa:
        e += 1
    return max(-127, min(127, e - 2))


def _sign(v) -> int:
    return 1 if np.signbit(np.float32(v)) else 0


def _words_to_bytes(words) -> bytes:
    return b"".join(int(w & 0xFFFFFFFF).to_bytes(4, "little") for w in words)


def fp8_planes(codes) -> bytes:
    """2048 FP8 codes in element order -> the code region: a plane of the
    first 16 codes of every 32-element group, then a plane of the last 16."""
    codes = bytes(codes)
    assert len(codes) == TILE
    lo = b"".join(codes[32 * g:32 * g + 16] for g in range(TILE // 32))
    hi = b"".join(codes[32 * g + 16:32 * g + 32] for g in range(TILE // 32))
    return lo + hi


def fp8_byte(tile: bytes, i: int) -> int:
    """The FP8 code byte of tile element i."""
    g, e = divmod(i, 32)
    return tile[16 * g + e] if e < 16 else tile[1024 + 16 * g + (e - 16)]


def encode_tile(fmt: str, v: np.ndarray) -> bytes:
    """v: 2048 float32 values (tail already zero)."""
    v = np.asarray(v, dtype=np.float32)
    assert v.size == TILE
    codes = bytearray()
    scales = bytearray()
    int3_q2w, int3_q1w = [], []
    for b in range(64):
        vb = v[32 * b:32 * b + 32]
        a = np.max(np.abs(vb))
        if fmt in ("int4", "int3"):
            qmax = 7 if fmt == "int4" else 3
            h = int_scale(a, qmax)
            s = float(h)
            if s == 0.0:
                nib = [0] * 32
                hbits = 0
            else:
                nib = [(_sign(x) << 3) | int_mag(x, s, qmax) for x in vb]
                hbits = int(h.view(np.uint16))
            scales += hbits.to_bytes(2, "little")
            if fmt == "int4":
                words = [sum(nib[8 * d + j] << (4 * j) for j in range(8)) for d in range(4)]
                codes += _words_to_bytes(words)
            else:
                # group g = elements 4j+g, nibble j of word N_g
                N = [sum(nib[4 * j + g] << (4 * j) for j in range(8)) for g in range(4)]
                m = 0x33333333
                w0 = (N[0] & m) | ((N[1] & m) << 2)
                w1 = (N[2] & m) | ((N[3] & m) << 2)
                hw = ((N[0] >> 3) & 0x11111111) | ((N[1] >> 2) & 0x22222222) | \
                     ((N[2] >> 1) & 0x44444444) | (N[3] & 0x88888888)
                int3_q2w += [w0, w1]
                int3_q1w += [hw]
        elif fmt == "fp8":
            s = fp8_scale(a)
            if s == 0:
                codes += bytes(32)
            else:
                for x in vb:
                    q = Fraction(abs(float(x))) / Fraction(float(s))
                    codes.append((_sign(x) << 7) | nearest_code(q, E4M3))
            scales += np.float32(s).tobytes()
        elif fmt == "mxfp4":
            e = mx_exponent(float(a))
            nib = []
            for x in vb:
                y = Fraction(abs(float(x))) * Fraction(2) ** (-e)
                nib.append((_sign(x) << 3) | nearest_code(y, E2M1))
            words = [sum(nib[8 * d + j] << (4 * j) for j in range(8)) for d in range(4)]
            codes += _words_to_bytes(words)
            scales.append(e + 127)
        else:
            raise ValueError(fmt)
    if fmt == "int3":
        return _words_to_bytes(int3_q2w) + _words_to_bytes(int3_q1w) + bytes(scales)
    if fmt == "fp8":
        return fp8_planes(codes) + bytes(scales)
    return bytes(codes) + bytes(scales)


def encode(fmt: str, x_f32: np.ndarray) -> bytes:
    x = np.asarray(x_f32, dtype=np.float32)
    tiles = (x.size + TILE - 1) // TILE
    out = b""
    for t in range(tiles):
        v = np.zeros(TILE, dtype=np.float32)
        chunk = x[t * TILE:(t + 1) * TILE]
        v[:chunk.size] = chunk
        out += encode_tile(fmt, v)
    return out


def decode_tile(fmt: str, tile: bytes) -> np.ndarray:
    """Exact decode of one tile to float32 values."""
    out = np.zeros(TILE, dtype=np.float32)
    words = lambda off, cnt: [int.from_bytes(tile[off + 4 * i: off + 4 * i + 4], "little")
                              for i in range(cnt)]
    for b in range(64):
        if fmt in ("int4", "int3"):
            soff = 1024 if fmt == "int4" else 768
            s = float(np.frombuffer(tile[soff + 2 * b: soff + 2 * b + 2], dtype=np.float16)[0])
            if fmt == "int4":
                ws = words(16 * b, 4)
                nib = [(ws[e // 8] >> (4 * (e % 8))) & 15 for e in range(32)]
            else:
                w0, w1 = words(8 * b, 2)
                (hw,) = words(512 + 4 * b, 1)
                nib = [0] * 32
                for g in range(4):
                    W = w0 if g < 2 else w1
                    Ng = ((W >> (2 * (g & 1))) & 0x33333333) | ((hw << (3 - g)) & 0x88888888)
                    for j in range(8):
                        nib[4 * j + g] = (Ng >> (4 * j)) & 15
            for e in range(32):
                mag = nib[e] & 7
                val = np.float32(float(Fraction(mag) * Fraction(s)))
                out[32 * b + e] = -val if nib[e] & 8 else val
        elif fmt == "fp8":
            s = np.frombuffer(tile[2048 + 4 * b: 2052 + 4 * b], dtype=np.float32)[0]
            for e in range(32):
                c = fp8_byte(tile, 32 * b + e)
                dec = np.float32(float(E4M3[c & 127])) if (c & 127) != 127 else np.float32(np.nan)
                val = dec * s                      # one binary32 product (IEEE)
                out[32 * b + e] = -val if c & 128 else val
        else:
            ws = words(16 * b, 4)
            e8 = tile[1024 + b]
            for e in range(32):
                nb = (ws[e // 8] >> (4 * (e % 8))) & 15
                val = np.float32(float(E2M1[nb & 7] * Fraction(2) ** (e8 - 127)))
                out[32 * b + e] = -val if nb & 8 else val
    return out


def tile_bytes(fmt: str) -> int:
    return {"int4": 1152, "int3": 896, "fp8": 2304, "mxfp4": 1088}[fmt]


def reduce(fmt: str, streams, n: int):
    """Decode every stream, add in stream order in binary32, requantize."""
    tb = tile_bytes(fmt)
    tiles = (n + TILE - 1) // TILE
    out = b""
    sums = np.zeros(n, dtype=np.float32)
    for t in range(tiles):
        acc = None
        for s in streams:
            d = decode_tile(fmt, bytes(s[t * tb:(t + 1) * tb]))
            acc = d.copy() if acc is None else (acc + d).astype(np.float32)
        lim = min(TILE, n - t * TILE)
        acc[lim:] = 0.0
        sums[t * TILE:t * TILE + lim] = acc[:lim]
        out += encode_tile(fmt, acc)
    return out, sums


# ---- every codec: (element format, scale type, block size) ------------------
#
# Element formats 1 INT4, 2 INT3, 3 E4M3, 4 E2M1, 5 E5M2; scale types 1 fp16,
# 2 fp32, 3 E8M0.  The tile is 2048 elements: the code region (layout as
# above, INT3 planes by 32-element groups) then 2048/block scales.

def _e5m2_table():
    import torch
    vals = torch.arange(124, dtype=torch.uint8).view(torch.float8_e5m2).float().numpy()
    return [Fraction(float(v)) for v in vals]


E5M2 = _e5m2_table()
CODE_BYTES = {1: 1024, 2: 768, 3: 2048, 4: 1024, 5: 2048}
SCALE_SIZE = {1: 2, 2: 4, 3: 1}
FMAX = {3: Fraction(448), 5: Fraction(57344)}
EMAX = {1: 2, 2: 1, 3: 8, 4: 2, 5: 15}       # largest element exponent (INT: floor log2 qmax)


def codec_tile_bytes(c) -> int:
    fmt, sc, bl = c
    return CODE_BYTES[fmt] + (TILE // bl) * SCALE_SIZE[sc]


def _floor_log2(a: Fraction) -> int:
    e = 0
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    while Fraction(2) ** e > a:
        e -= 1
    return e


def _e8m0_exp(a: float, emax: int) -> int:
    if a == 0:
        return -127
    return max(-127, min(127, _floor_log2(Fraction(float(a))) - emax))


def _nibbles_to_bytes(nib) -> bytes:
    """nib[i] at nibble i of a little-endian bitstream."""
    out = bytearray(len(nib) // 2)
    for i, v in enumerate(nib):
        out[i // 2] |= (v & 15) << (4 * (i % 2))
    return bytes(out)


def encode_codec(c, x_f32: np.ndarray) -> bytes:
    """Packed bytes of x under codec c = (format, scale, block): tiles of 2048
    with a zero-padded tail; per block the scale rule, then per element the
    nearest code (ties to the even code, saturating)."""
    fmt, sc, bl = c
    x = np.asarray(x_f32, dtype=np.float32)
    out = b""
    for t in range((x.size + TILE - 1) // TILE):
        v = np.zeros(TILE, dtype=np.float32)
        chunk = x[t * TILE:(t + 1) * TILE]
        v[:chunk.size] = chunk
        codes = [0] * TILE           # sign-magnitude code per element (format width)
        scales = bytearray()
        for b in range(TILE // bl):
            vb = v[b * bl:(b + 1) * bl]
            a = np.float32(np.max(np.abs(vb)))
            zero = False
            if sc == 3:
                ex = _e8m0_exp(float(a), EMAX[fmt])
                scales.append(ex + 127)
                den = Fraction(2) ** ex
            elif fmt in (1, 2):                   # INT with fp16 scale
                h = int_scale(a, 7 if fmt == 1 else 3)
                zero = float(h) == 0.0
                scales += (0 if zero else int(h.view(np.uint16))).to_bytes(2, "little")
                den = None if zero else float(h)
            elif sc == 1:                         # FP8 with fp16 scale
                s32 = np.float32(a) / np.float32(float(FMAX[fmt]))
                h = np.float16(min(s32, np.float32(65504.0)))
                zero = float(h) == 0.0
                scales += (0 if zero else int(h.view(np.uint16))).to_bytes(2, "little")
                den = None if zero else Fraction(float(h))
            else:                                 # FP8 with fp32 scale
                s = np.float32(a) / np.float32(float(FMAX[fmt]))
                zero = s < np.finfo(np.float32).tiny
                scales += np.float32(0.0 if zero else s).tobytes()
                den = None if zero else Fraction(float(s))
            for e in range(bl):
                i = b * bl + e
                if zero:
                    codes[i] = 0
                    continue
                sign = _sign(vb[e])
                if fmt in (1, 2):
                    qmax = 7 if fmt == 1 else 3
                    if sc == 1:
                        mag = int_mag(vb[e], den, qmax)
                    else:
                        mag = nearest_code(Fraction(abs(float(vb[e]))) / den, [Fraction(k) for k in range(qmax + 1)])
                    codes[i] = (sign << 3) | mag
                elif fmt == 4:
                    codes[i] = (sign << 3) | nearest_code(Fraction(abs(float(vb[e]))) / den, E2M1)
                else:
                    table = E4M3 if fmt == 3 else E5M2
                    codes[i] = (sign << 7) | nearest_code(Fraction(abs(float(vb[e]))) / den, table)
        out += code_region(fmt, codes) + bytes(scales)
    return out


def code_region(fmt: int, codes) -> bytes:
    """The code bytes of one tile from its 2048 sign-magnitude codes in
    element order (INT3: sign << 3 | magnitude)."""
    if fmt in (1, 4):
        return _nibbles_to_bytes(codes)
    if fmt == 2:
        q2w, q1w = [], []
        for g in range(64):
            nib = codes[32 * g:32 * g + 32]
            N = [sum(nib[4 * j + k] << (4 * j) for j in range(8)) for k in range(4)]
            m = 0x33333333
            q2w += [(N[0] & m) | ((N[1] & m) << 2), (N[2] & m) | ((N[3] & m) << 2)]
            q1w.append(((N[0] >> 3) & 0x11111111) | ((N[1] >> 2) & 0x22222222) |
                       ((N[2] >> 1) & 0x44444444) | (N[3] & 0x88888888))
        return _words_to_bytes(q2w) + _words_to_bytes(q1w)
    return fp8_planes(codes)


def decode_codec(c, tile: bytes) -> np.ndarray:
    """Exact decode of one tile to float32 (FP8 with an fp32 scale: one IEEE
    binary32 product)."""
    fmt, sc, bl = c
    cb = CODE_BYTES[fmt]
    out = np.zeros(TILE, dtype=np.float32)
    for i in range(TILE):
        b = i // bl
        if fmt in (1, 4):
            nb = (tile[i // 2] >> (4 * (i % 2))) & 15
            mag = nb & 7
            val = Fraction(mag) if fmt == 1 else E2M1[mag]
            neg = bool(nb & 8)
        elif fmt == 2:
            g, e = divmod(i, 32)
            w0, w1 = [int.from_bytes(tile[8 * g + 4 * k:8 * g + 4 * k + 4], "little") for k in range(2)]
            hw = int.from_bytes(tile[512 + 4 * g:516 + 4 * g], "little")
            k, j = e % 4, e // 4
            W = w0 if k < 2 else w1
            nib = (((W >> (2 * (k & 1))) & 0x33333333) | ((hw << (3 - k)) & 0x88888888)) >> (4 * j) & 15
            val, neg = Fraction(nib & 7), bool(nib & 8)
        else:
            code = fp8_byte(tile, i)
            table = E4M3 if fmt == 3 else E5M2
            if (fmt == 3 and (code & 127) == 127) or (fmt == 5 and (code & 127) >= 124):
                spec = np.float32(np.nan)
                if fmt == 5 and (code & 127) == 124:
                    spec = np.float32(np.inf)
                val, neg = None, bool(code & 128)
            else:
                val, neg = table[code & 127], bool(code & 128)
        so = cb + b * SCALE_SIZE[sc]
        if val is None:                                  # NaN / infinite code: IEEE product with the scale
            if sc == 2:
                s = np.frombuffer(tile[so:so + 4], dtype=np.float32)[0]
            elif sc == 1:
                s = np.float32(np.frombuffer(tile[so:so + 2], dtype=np.float16)[0])
            else:
                s = np.float32(np.nan) if tile[so] == 255 else np.float32(2.0 ** (tile[so] - 127))
            with np.errstate(invalid="ignore"):
                r = (-spec if neg else spec) * s
            out[i] = r
            continue
        if sc == 2:
            s = np.frombuffer(tile[so:so + 4], dtype=np.float32)[0]
            with np.errstate(all="ignore"):              # non-finite scales: IEEE product
                r = np.float32(float(val)) * s
        elif sc == 1:
            s = np.frombuffer(tile[so:so + 2], dtype=np.float16)[0]
            if np.isfinite(s):
                r = np.float32(float(val * Fraction(float(s))))
                if r == 0 and np.signbit(s):                 # a zero product takes the scale's sign too
                    r = np.float32(-0.0)
            else:                                        # +-inf or NaN scale: IEEE product
                with np.errstate(invalid="ignore"):
                    r = np.float32(float(val)) * np.float32(s)
        else:
            if tile[so] == 255:
                r = np.float32(np.nan)
            else:                                        # rounded once: +-inf beyond binary32
                with np.errstate(over="ignore"):
                    r = np.float32(float(val * Fraction(2) ** (tile[so] - 127)))
        out[i] = -r if neg else r
    return out


def reduce_codec(c, streams, n: int):
    """Decode every stream, add in stream order in binary32, requantize."""
    tb = codec_tile_bytes(c)
    tiles = (n + TILE - 1) // TILE
    out = b""
    sums = np.zeros(n, dtype=np.float32)
    for t in range(tiles):
        acc = None
        for s in streams:
            d = decode_codec(c, bytes(s[t * tb:(t + 1) * tb]))
            acc = d.copy() if acc is None else (acc + d).astype(np.float32)
        lim = min(TILE, n - t * TILE)
        acc[lim:] = 0.0
        sums[t * TILE:t * TILE + lim] = acc[:lim]
        out += encode_codec(c, acc)
    return out, sums


# ---- MXFP4 GEMV in exact rationals -----------------------------------------

def rn32(q: Fraction) -> Fraction:
    """Round a rational to the nearest binary32 value, ties to even
    (subnormals included); returns the rounded value as a Fraction."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = _floor_log2(a)
    e = max(e, -126)                                 # subnormal quantum 2^-149
    scale = Fraction(2) ** (23 - e)
    m = a * scale
    k = m.numerator // m.denominator
    rem = m - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    if k >= 2 ** 24 and e + 1 > 127:
        raise OverflowError
    return sign * Fraction(k) / scale


def gemv_mxfp4_exact(w_packed: bytes, rows: int, cols: int, x: np.ndarray):
    """y = W x in exact rationals: every weight decoded from its nibble and
    E8M0 byte (decode_codec), every x value as a Fraction, the row sum exact.
    Returns a list of Fractions."""
    tb = codec_tile_bytes((4, 3, 32))
    T = cols // TILE
    xs = [Fraction(float(v)) for v in np.asarray(x, dtype=np.float32)]
    out = []
    for r in range(rows):
        acc = Fraction(0)
        for j in range(T):
            d = decode_codec((4, 3, 32), w_packed[(r * T + j) * tb:(r * T + j + 1) * tb])
            for i in range(TILE):
                acc += Fraction(float(d[i])) * xs[j * TILE + i]
        out.append(acc)
    return out
