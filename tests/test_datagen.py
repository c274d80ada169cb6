"""Pins of the seeded input generators: the SplitMix64 reference outputs,
counter-based determinism (slices and thread counts do not change values) and
the moments of each workload's distribution."""
import json
import os

import numpy as np

import datagen

G = 0x9E3779B97F4A7C15


def test_splitmix64_reference_outputs():
    with open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed0.json")) as f:
        ref = json.load(f)["outputs_hex"]
    lib = datagen._load()
    got = [format(lib.rcg_mix64((k * G) % 2**64), "016x") for k in range(len(ref))]
    assert got == ref


def test_slices_regenerate_identically():
    a = datagen.student_t4(500, 300000)
    b = datagen.student_t4(500, 1000, start=123456)
    assert np.array_equal(a[123456:124456], b)
    c = datagen.fill(datagen.STUDENT4, 500, 300000, 0.0, 1.0)
    assert np.array_equal(a, c)


def test_moments():
    z = datagen.normal(0, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    h = datagen.normal(300, 1 << 20, 0.0, 0.5).astype(np.float64)
    assert abs(h.std() - 0.5) < 3e-3
    t = datagen.student_t4(500, 1 << 21).astype(np.float64)
    assert abs(t.mean()) < 1e-2
    assert abs(np.median(np.abs(t)) - 0.7407) < 1e-2          # t_4 median |x|
    assert abs((np.abs(t) > 4.604).mean() - 0.01) < 1.5e-3     # two-sided 1% point of t_4
    o = datagen.normal_outliers(2, 1 << 21, 20.0, 0.001).astype(np.float64)
    assert 0.00060 < (np.abs(o) > 8).mean() < 0.00078      # 0.001 * P(|z| > 0.4)
    w = datagen.rowdrift(41, 40, 512, 4096).reshape(512, 4096).astype(np.float64)
    rs = w.std(axis=1) / 0.02
    assert rs.min() > 0.45 and rs.max() < 2.05
    assert abs(rs.mean() - 1.25) < 0.06


def test_workload_shapes_and_dtypes():
    assert datagen.fp16_normal_64x2048(0).dtype == np.float16
    assert datagen.fp16_normal_64x2048(1).size == 131072
    x = datagen.bf16_act_256x8192_outl()
    assert x.dtype == np.uint16 and x.size == 256 * 8192
    assert datagen.bf16_student4(1 << 20).size == 1 << 19
