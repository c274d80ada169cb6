"""Pins of the oracle's MXFP4 GEMV (y = W x on packed MXFP4 tiles).  The
pages fix no summation order, so the oracle is the definition: the exact dot
product of the decoded weights and x, rounded once to binary64 (math.fsum of
exact binary64 products).  It is pinned to an exact-rational statement of
the same sum (tests/brute.py), to one-hot inputs (the decoded weight column)
and to dyadic inputs whose sums are exact in any order."""
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle
from tests import brute

RNG = np.random.default_rng(77)


def packed_weight(rows, cols, seed):
    r = np.random.default_rng(seed)
    w = (r.standard_normal(rows * cols) * np.exp(r.uniform(-3, 3, rows * cols))).astype(np.float32)
    w[:32] = 0.0                                     # a zero block
    return w, oracle.quantize_pack(oracle.MXFP4, w)


def round_f64(q: Fraction) -> float:
    """Fraction -> nearest binary64 (ties to even), by Python's correctly
    rounded int/int division."""
    return q.numerator / q.denominator


@pytest.mark.parametrize("cols", [2048, 4096])
def test_gemv_equals_exact_rational_sum(cols):
    rows = 2
    _, p = packed_weight(rows, cols, 1)
    x = (RNG.standard_normal(cols) * np.exp(RNG.uniform(-4, 4, cols))).astype(np.float32)
    x[5] = 0.0
    x[7] = -0.0
    y, mag = oracle.mxfp4_gemv(p, rows, cols, x)
    ref = brute.gemv_mxfp4_exact(p.tobytes(), rows, cols, x)
    assert [float(v) for v in y] == [round_f64(q) for q in ref]
    assert (mag >= np.abs(y)).all()


def test_gemv_bf16_x_on_the_weight_recipe_vs_exact_rationals():
    """Three rows of the 4096 x 4096 weight recipe with a bf16 x."""
    rows, cols = 3, 4096
    wbits = datagen.bf16_weight_4096x4096()[:rows * cols]
    p = oracle.quantize_pack(oracle.MXFP4, wbits, dtype=oracle.DT_BF16)
    x = datagen.narrow(RNG.standard_normal(cols).astype(np.float32), "bf16")
    y, _ = oracle.mxfp4_gemv(p, rows, cols, x, x_dtype=oracle.DT_BF16)
    ref = brute.gemv_mxfp4_exact(p.tobytes(), rows, cols, oracle.bf16_bits_to_f32(x))
    assert [float(v) for v in y] == [round_f64(q) for q in ref]


def test_gemv_one_hot_returns_the_decoded_weight_column():
    rows, cols = 5, 2048
    _, p = packed_weight(rows, cols, 3)
    wd = oracle.unpack_dequant(oracle.MXFP4, p, rows * cols).reshape(rows, cols)
    for j in (0, 31, 32, 1000, 2047):
        x = np.zeros(cols, dtype=np.float32)
        x[j] = 1.0
        y, _ = oracle.mxfp4_gemv(p, rows, cols, x)
        assert np.array_equal(y, wd[:, j].astype(np.float64))


def test_gemv_dyadic_sums_are_exact():
    """Weights k * 2^-3 and x integers: every partial sum is a multiple of
    2^-3 far below 2^20, so the sum is exact; it equals an integer formula."""
    rows, cols = 4, 4096
    r = np.random.default_rng(9)
    idx = r.integers(0, 8, rows * cols)
    w = (np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[idx] * r.choice([-1, 1], rows * cols)).astype(np.float32)
    w[::32] = 6.0                                    # every block max 6: E8M0 exponent 0
    p = oracle.quantize_pack(oracle.MXFP4, w)
    x = r.integers(-50, 51, cols).astype(np.float32)
    y, _ = oracle.mxfp4_gemv(p, rows, cols, x)
    ref = (w.reshape(rows, cols).astype(np.float64) * x.astype(np.float64)).sum(axis=1)
    assert np.array_equal(y, ref)


def test_gemv_rejects_ragged_columns():
    with pytest.raises(ValueError):
        oracle.mxfp4_gemv(np.zeros(4096, np.uint8), 1, 1000, np.zeros(1000, np.float32))
