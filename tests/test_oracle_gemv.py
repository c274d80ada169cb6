"""Pins of the oracle's MXFP4 GEMV (y = W x on packed MXFP4 tiles): the
summation order is the definition in rco_mxfp4_gemv; it is checked against
an independent exact-rational statement of that order (tests/brute.py),
against the exact dot product within the rounding bound of that order, and
on one-hot inputs where every rounding is exact."""
import math

import numpy as np
import pytest

import datagen
import oracle
from tests import brute

RNG = np.random.default_rng(77)


def packed_weight(rows, cols, seed):
    w = (RNG.standard_normal(rows * cols) * np.exp(RNG.uniform(-3, 3, rows * cols))).astype(np.float32)
    w[:32] = 0.0                                     # a zero block
    return w, oracle.quantize_pack(oracle.MXFP4, w)


@pytest.mark.parametrize("cols", [2048, 4096])
def test_gemv_equals_exact_rational_statement_of_the_order(cols):
    rows = 2
    _, p = packed_weight(rows, cols, 1)
    x = (RNG.standard_normal(cols) * np.exp(RNG.uniform(-4, 4, cols))).astype(np.float32)
    x[5] = 0.0
    x[7] = -0.0
    ours = oracle.mxfp4_gemv(p, rows, cols, x)
    ref = brute.gemv_mxfp4(p.tobytes(), rows, cols, x)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_gemv_within_rounding_bound_of_exact_dot_product():
    """|y - exact| <= (32 + T + 6) 2^-24 sum |W_ij x_j| (each term passes
    through at most that many roundings), on the 4096 x 4096 weight recipe."""
    rows, cols = 48, 4096
    wbits = datagen.bf16_weight_4096x4096()[:rows * cols]
    p = oracle.quantize_pack(oracle.MXFP4, wbits, dtype=oracle.DT_BF16)
    x = datagen.narrow((RNG.standard_normal(cols)).astype(np.float32), "bf16")
    y = oracle.mxfp4_gemv(p, rows, cols, x, x_dtype=oracle.DT_BF16)
    wd = oracle.unpack_dequant(oracle.MXFP4, p, rows * cols).reshape(rows, cols).astype(np.float64)
    xd = oracle.bf16_bits_to_f32(x).astype(np.float64)
    T = cols // 2048
    for r in range(rows):
        terms = wd[r] * xd                           # exact in binary64
        exact = math.fsum(terms)
        bound = (32 + T + 6) * 2.0 ** -24 * math.fsum(np.abs(terms))
        assert abs(float(y[r]) - exact) <= bound + 1e-300


def test_gemv_one_hot_returns_the_decoded_weight_column():
    rows, cols = 5, 2048
    w, p = packed_weight(rows, cols, 3)
    wd = oracle.unpack_dequant(oracle.MXFP4, p, rows * cols).reshape(rows, cols)
    for j in (0, 31, 32, 1000, 2047):
        x = np.zeros(cols, dtype=np.float32)
        x[j] = 1.0
        y = oracle.mxfp4_gemv(p, rows, cols, x)
        assert np.array_equal(y, wd[:, j])


def test_gemv_output_dtypes_round_the_fp32_result():
    rows, cols = 4, 4096
    _, p = packed_weight(rows, cols, 4)
    x = RNG.standard_normal(cols).astype(np.float32)
    y32 = oracle.mxfp4_gemv(p, rows, cols, x)
    assert np.array_equal(oracle.mxfp4_gemv(p, rows, cols, x, y_dtype=oracle.DT_BF16), oracle.f32_to_bf16_bits(y32))
    assert np.array_equal(oracle.mxfp4_gemv(p, rows, cols, x, y_dtype=oracle.DT_FP16).view(np.uint16),
                          oracle.f32_to_f16_bits(y32))


def test_gemv_rejects_ragged_columns():
    with pytest.raises(RuntimeError):
        oracle.mxfp4_gemv(np.zeros(4096, np.uint8), 1, 1000, np.zeros(1000, np.float32))
