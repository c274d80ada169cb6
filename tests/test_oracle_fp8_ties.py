"""The oracle's FP8 codes at exact rounding ties.

Blocks of bf16 / fp16 values with planted exact ties (tests/fp8_ties.py):
the code of a tie follows from where the exact quotient lies against the
midpoint -- above it when the FP32 scale RN32(a / fmax) was rounded down,
below when rounded up, on it when a / fmax is exact or the scale is FP16
(then the even code) ("FP8 Formats for Deep Learning", abstract;
"RCCLX: Innovating GPU communications on AMD platforms", Low-Precision
Collectives).  The oracle computes codes by exact comparisons of x with
midpoint times scale; this derives them from the scale's rounding direction
instead, so a sign slip or a wrong tie rule in either shows up.
"""
import numpy as np
import pytest

import datagen
import oracle
from tests.fp8_ties import expected_code_index, magnitudes, scale_of, tie_message

DT = {"bf16": oracle.DT_BF16, "fp16": oracle.DT_FP16}


CASES = [(e, sc, dt, b, 0) for e in ("e4m3", "e5m2") for sc in ("f32", "f16") for dt in ("bf16", "fp16")
         for b in (16, 32, 64)]
# bf16 blocks 2^-80 smaller (exact; every tie and its side is kept): FP32
# scales down to about 2^-108, many below 2^-64
CASES += [(e, "f32", "bf16", b, -80) for e in ("e4m3", "e5m2") for b in (16, 32, 64)]


@pytest.mark.parametrize("elem,scale,dt,block,shift", CASES)
def test_oracle_codes_at_exact_fp8_ties(elem, scale, dt, block, shift):
    n = 2048 + 320
    x, info = tie_message(elem, scale, dt, block, n, seed=hash((elem, scale, dt, block)) % 2**32)
    exact = np.ldexp(x.astype(np.float64), shift)
    xn = datagen.narrow(exact.astype(np.float32), dt)
    x = oracle.widen_to_f32(xn, DT[dt])
    kept = x.astype(np.float64) == exact          # shifted below the normal range: rounded, no tie
    c = oracle.ALL_CODECS[f"{elem}_{scale}_b{block}"]
    packed = oracle.quantize_pack(c, xn, dtype=DT[dt])
    dec = oracle.unpack_dequant(c, packed, n, oracle.DT_FP32)
    vals = magnitudes(elem)
    ties, sides = 0, set()
    for b, (tie_at, side) in enumerate(info):
        base = b * block
        blk = x[base:min(n, base + block)].astype(np.float64)
        if blk.size == 0:
            continue
        a = float(np.abs(blk).max())
        assert kept[base:base + blk.size][np.abs(blk) == a].all()
        s = scale_of(a, elem, scale)
        for j, (lo, hi) in tie_at.items():
            if base + j >= n or not kept[base + j]:
                continue
            want = float(np.float32(vals[expected_code_index(lo, hi, side)] * s))
            got = float(dec[base + j])
            assert got == np.copysign(want, x[base + j]), (b, j, got, want, side)
            ties += 1
        sides.add(side)
    assert ties >= 200
    if scale == "f32" and not (elem == "e5m2" and dt == "fp16"):
        # E5M2 midpoints have odd parts 9..15 (and 7 only at 7 * 2^-17), so
        # with fp16 values fmax x = m a needs a / fmax exact: side 0 only
        assert sides == {-1, 0, 1}, sides
