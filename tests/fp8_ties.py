"""Seeded messages whose blocks hold exact FP8 rounding ties.

An E4M3 / E5M2 code is the round-to-nearest-even code of the exact quotient
x / s ("FP8 Formats for Deep Learning", abstract, for the encodings; "RCCLX:
Innovating GPU communications on AMD platforms", Low-Precision Collectives,
for FP8 payloads with scales computed in FP32).  With block values of a few
significant bits (bf16, fp16) the quotient often lands exactly on a midpoint
m between two neighbouring codes:

* FP32 scale s = RN32(a / fmax), a the block's largest magnitude: when
  fmax x = m a exactly, the quotient x / s lies above m if s was rounded down
  (a - s fmax > 0), below m if rounded up, and on m if a / fmax is exact;
* FP16 scale s: when x = m s exactly, the quotient is m.

`tie_message` builds such blocks (the block maximum, planted ties and filler
values, random signs) and returns the per-block facts a test needs to state
the code each tie must get.  Nothing here encodes anything: the expected code
follows from the rule above, not from an implementation.
"""
from fractions import Fraction

import numpy as np

FMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def magnitudes(elem: str) -> np.ndarray:
    """The finite non-negative code values in increasing order."""
    if elem == "e4m3":
        v = [c * 2.0 ** -9 for c in range(8)] + [(8 + m) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8)]
        return np.array(v[:127])                       # 0x7F is NaN
    v = [c * 2.0 ** -16 for c in range(4)] + [(4 + m) * 2.0 ** (e - 17) for e in range(1, 31) for m in range(4)]
    return np.array(v)                                 # 124 finite values, largest 57344


def _narrow_ok(x: Fraction, dt: str) -> bool:
    """x is exactly a finite bf16 / fp16 value (x > 0)."""
    f = float(x)
    if Fraction(f) != x:
        return False
    if dt == "fp16":
        h = np.float16(f)
        return bool(np.isfinite(h)) and float(h) == f
    b = np.float32(f)
    return float(b) == f and (int(np.array([b]).view(np.uint32)[0]) & 0xFFFF) == 0


def _random_narrow(r, dt: str, seven: bool) -> float:
    """A random positive bf16 / fp16 value; with `seven`, its integer
    significand is a multiple of 7 (so that a / fmax is exact)."""
    bits = 8 if dt == "bf16" else 11
    lo, hi = 1 << (bits - 1), 1 << bits
    while True:
        m = int(r.integers(lo, hi))
        if not seven or m % 7 == 0:
            break
    e = int(r.integers(-4, 8)) if dt == "fp16" else int(r.integers(-20, 20))
    return float(m) * 2.0 ** (e - bits + 1)


def _narrow_down(x: float, dt: str) -> float:
    """A bf16 / fp16 value at most x (x >= 0), near it."""
    if dt == "fp16":
        h = float(np.float16(x))
        return h if h <= x else float(np.nextafter(np.float16(x), np.float16(0)))
    b = int(np.array([np.float32(x)]).view(np.uint32)[0]) & 0xFFFF0000
    v = float(np.array([b], dtype=np.uint32).view(np.float32)[0])
    return v if v <= x else float(np.array([b - 0x10000], dtype=np.uint32).view(np.float32)[0])


def scale_of(a: float, elem: str, scale: str) -> float:
    """The block scale by the FP32 rule RN32(a / fmax) or the FP16 rule
    RN16(min(RN32(a / fmax), 65504))."""
    s32 = np.float32(a) / np.float32(FMAX[elem])
    if scale == "f32":
        return float(s32)
    return float(np.float16(min(float(s32), 65504.0)))


def tie_block(r, elem: str, scale: str, dt: str, block: int):
    """One block: (values as float64, {position: (lower, upper)} for the
    planted ties, side) with side = sign of a - s fmax for FP32 scales (0 for
    FP16 scales: the quotient is the midpoint itself)."""
    vals = magnitudes(elem)
    mids = [(Fraction(vals[i]) + Fraction(vals[i + 1])) / 2 for i in range(len(vals) - 1)]
    fmax = Fraction(FMAX[elem])
    for _ in range(400):
        a = _random_narrow(r, dt, seven=bool(r.random() < 0.3))
        s = scale_of(a, elem, scale)
        if not 0.0 < s or (scale == "f32" and s < 2.0 ** -64):
            continue
        fa, fs = Fraction(a), Fraction(s)
        ties = []
        for i, m in enumerate(mids):
            x = m * fa / fmax if scale == "f32" else m * fs
            if 0 < x < fa and _narrow_ok(x, dt):
                ties.append((float(x), i))
        if not ties:
            continue
        side = (fa - fs * fmax) if scale == "f32" else Fraction(0)
        side = (side > 0) - (side < 0)
        out = np.empty(block)
        tie_at = {}
        pos = r.permutation(block)
        out[pos[0]] = a
        for j in pos[1:]:
            if r.random() < 0.6:
                x, i = ties[int(r.integers(0, len(ties)))]
                out[j] = x
                tie_at[int(j)] = (i, i + 1)
            else:
                out[j] = _narrow_down(a * r.random(), dt)
        signs = np.where(r.random(block) < 0.5, -1.0, 1.0)
        return out * signs, tie_at, side
    raise RuntimeError("no block with ties found")


def tie_message(elem: str, scale: str, dt: str, block: int, n: int, seed: int):
    """n values (float32, exactly representable in dt) built block by block;
    returns (values, blocks) with blocks[b] = (tie positions, side)."""
    r = np.random.default_rng(seed)
    nb = -(-n // block)
    v = np.empty(nb * block)
    info = []
    for b in range(nb):
        vals, tie_at, side = tie_block(r, elem, scale, dt, block)
        v[b * block:(b + 1) * block] = vals
        info.append((tie_at, side))
    x = v[:n].astype(np.float32)
    assert np.array_equal(x.astype(np.float64), v[:n]), "values must be exact in binary32"
    return x, info


def expected_code_index(lower: int, upper: int, side: int) -> int:
    """The code a tie gets: upper when the quotient lies above the midpoint,
    lower when below, the even one of the two when on it."""
    if side > 0:
        return upper
    if side < 0:
        return lower
    return lower if lower % 2 == 0 else upper
