"""Pins of the oracle's number-format rules against things other than itself:
library casts (numpy float16, torch bfloat16 / float8_e4m3fn), exhaustive
enumeration, the facts the pages print, and a generic minifloat decoder that is
first checked on formats a library knows."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")
RNG = np.random.default_rng(1234)


def facts():
    with open(GOLDEN) as f:
        return json.load(f)


# ---- tile sizes: printed on the QuickReduce INT3 page -------------------

def test_tile_sizes_match_page():
    f = facts()
    assert oracle.tile_bytes(oracle.INT4) == f["int4_tile_bytes"]["value"]
    assert oracle.tile_bytes(oracle.INT3) == f["int3_tile_bytes"]["value"]
    red = 100 * (1 - f["int3_tile_bytes"]["value"] / f["int4_tile_bytes"]["value"])
    assert round(red) == f["int3_vs_int4_reduction_percent"]["value"]


def test_tile_geometry_derived_from_page():
    """(1152 - 896) bytes * 8 bits / (4 - 3) bits = 2048 elements per tile,
    leaving 1152 - 2048*4/8 = 128 bytes = 64 fp16 scales = one per 32 values."""
    f = facts()
    i4, i3 = f["int4_tile_bytes"]["value"], f["int3_tile_bytes"]["value"]
    elems = (i4 - i3) * 8 // (4 - f["int3_bits_per_value"]["value"])
    assert elems == oracle.TILE == 2048
    scale_bytes = i4 - elems * 4 // 8
    assert scale_bytes == 128 and elems // (scale_bytes // 2) == oracle.BLOCK
    assert i3 == elems * 2 // 8 + elems // 8 + scale_bytes       # q2w + q1w + scales


def test_fp8_payload_ratio_4_to_1():
    """FP8 code bytes are one quarter of the fp32 input bytes (the 4:1 of the
    RCCLX low-precision section); with the per-block fp32 scales the tile
    ratio is 8192/2304."""
    f = facts()
    x = np.zeros(4096, dtype=np.float32)
    p = oracle.quantize_pack(oracle.FP8, x)
    tiles = 2
    code_bytes = tiles * 2048
    assert (x.nbytes) / code_bytes == f["fp8_max_compression"]["value"]
    assert p.size == tiles * 2304


@pytest.mark.parametrize("c,tb", [(oracle.INT4, 1152), (oracle.INT3, 896), (oracle.FP8, 2304),
                                  (oracle.MXFP4, 1088)])
def test_packed_bytes(c, tb):
    for n in [0, 1, 2047, 2048, 2049, 131072, 10**6 + 3]:
        assert oracle.packed_bytes(c, n) == -(-n // 2048) * tb


def test_unsupported_codecs():
    for c in [(1, 2, 32), (2, 2, 32), (4, 1, 32), (4, 2, 32), (1, 1, 8), (3, 2, 128), (5, 2, 48), (9, 1, 32), (0, 3, 32)]:
        assert oracle.tile_bytes(c) == 0


# ---- binary16 / bfloat16 -------------------------------------------------

def test_f16_decode_all_patterns_vs_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f32_probe_values():
    """Every half, every midpoint between neighbouring halves (the ties), one
    float32 ulp either side of each midpoint, random float32s over the whole
    range, and the overflow / subnormal borders."""
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    hv = h.view(np.float16).astype(np.float64)
    mids = (hv[:-1] + hv[1:]) / 2
    mids32 = mids.astype(np.float32)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    rnd = RNG.integers(0, 2**31, 400000, dtype=np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    edge = np.array([65504, 65519.99, 65520, 65536, 1e9, 2**-24, 2**-25, 2**-26, 3 * 2**-26,
                     2**-14, 2**-14 * (1 - 2**-11), 0.0, 1e-45], dtype=np.float32)
    v = np.concatenate([hv.astype(np.float32), mids32, up, dn, rnd, edge])
    return np.concatenate([v, -v]).astype(np.float32)


def test_f32_to_f16_vs_numpy():
    x = _f32_probe_values()
    ours = oracle.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):             # values beyond fp16 range become +-inf on purpose
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_all_patterns_vs_torch():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_vs_torch():
    rnd = RNG.integers(0, 2**32, 1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    # ties: bf16 value + half a bf16 ulp, exactly representable in float32
    b = RNG.integers(0, 0x7F80, 100000, dtype=np.uint32)
    ties = ((b << 16) | 0x8000).view(np.float32)
    edge = np.array([3.3895314e38, 3.4028235e38, 1e-40, 1e-45, 0.0], dtype=np.float32)
    x = np.concatenate([rnd, ties, -ties, edge, -edge]).astype(np.float32)
    ours = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---- E4M3 -----------------------------------------------------------------

def test_e4m3_decode_all_codes_vs_torch_and_page():
    f = facts()
    ours = np.array([oracle.e4m3_decode(c) for c in range(256)], dtype=np.float32)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # page: no infinities, one NaN mantissa pattern (S.1111.111 -> two codes)
    assert not np.isinf(ours).any() and f["e4m3_no_infinities"]["value"]
    nan_codes = [c for c in range(256) if np.isnan(ours[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert len({c & 0x07 for c in nan_codes}) == f["e4m3_nan_mantissa_patterns"]["value"]
    assert np.nanmax(ours) == 448.0


def test_e4m3_encode_vs_torch_cast():
    """For quotients y/1 with |y| <= 448 the exact-quotient RNE equals torch's
    RNE cast; above 448 the oracle saturates (torch returns NaN past 464)."""
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = (e4[:-1] + e4[1:]) / 2
    rnd = np.abs(RNG.standard_normal(200000) * 30).astype(np.float32)
    rnd = np.concatenate([rnd, RNG.uniform(0, 2**-6, 50000).astype(np.float32)])
    y = np.concatenate([e4, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)), rnd]).astype(np.float32)
    y = y[y <= 448]
    ours = oracle.e4m3_mag_of_quotient(y.astype(np.float64), 1.0)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int32)
    assert np.array_equal(ours, ref)
    big = np.array([448.5, 460, 464, 470, 1e6], dtype=np.float64)
    assert (oracle.e4m3_mag_of_quotient(big, 1.0) == 126).all()


def test_e4m3_quotient_brute_force():
    """num/den with den a random binary32: argmin over all 127 magnitudes in
    exact rationals, ties to even code."""
    from tests.brute import E4M3, nearest_code
    den = np.abs(RNG.standard_normal(3000)).astype(np.float32) + np.float32(1e-3)
    q = RNG.uniform(0, 470, 3000)
    num = (q * den).astype(np.float32)
    # exact ties: num = midpoint * den when representable
    mids = [(E4M3[c] + E4M3[c + 1]) / 2 for c in range(126)]
    tnum, tden = [], []
    for i in range(300):
        m = mids[RNG.integers(0, 126)]
        d = np.float32(2.0 ** RNG.integers(-10, 10))
        tnum.append(np.float32(float(m) * float(d)))
        tden.append(d)
    num = np.concatenate([num, np.array(tnum, np.float32)])
    den = np.concatenate([den, np.array(tden, np.float32)])
    ours = oracle.e4m3_mag_of_quotient(num.astype(np.float64), den.astype(np.float64))
    ref = [nearest_code(Fraction(float(a)) / Fraction(float(b)), E4M3) for a, b in zip(num, den)]
    assert ours.tolist() == ref


# ---- generic minifloat: pinned on fp16 and E4M3, then read off for E2M1 ----

def minifloat_values(ebits, mbits, bias, finite_all=False):
    """Value of every non-negative code of a binary format from its field
    widths: subnormals at exponent field 0, no special values if finite_all."""
    vals = []
    for code in range(1 << (ebits + mbits)):
        e, m = code >> mbits, code & ((1 << mbits) - 1)
        if not finite_all and e == (1 << ebits) - 1:
            vals.append(None)
            continue
        if e == 0:
            vals.append(Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias))
        else:
            vals.append((1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias))
    return vals


def test_minifloat_decoder_matches_libraries():
    h = minifloat_values(5, 10, 15)
    ref = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    assert [float(v) for v in h[:0x7C00]] == ref.tolist()
    e4 = minifloat_values(4, 3, 7, finite_all=True)[:127]
    ref8 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert [float(v) for v in e4] == ref8.astype(np.float64).tolist()


def test_e2m1_decode_and_encode():
    """E2M1 = 2 exponent bits (bias 1), 1 mantissa bit, all codes finite (the
    MX element; the pages name the format but do not print its table)."""
    table = minifloat_values(2, 1, 1, finite_all=True)
    ours = [oracle.e2m1_decode(c) for c in range(16)]
    assert ours[:8] == [float(v) for v in table]
    assert [abs(v) for v in ours[8:]] == [float(v) for v in table]
    assert all(np.signbit(v) for v in ours[8:])
    from tests.brute import nearest_code
    y = np.concatenate([RNG.uniform(0, 8, 5000), [float(v) for v in table],
                        [float((table[i] + table[i + 1]) / 2) for i in range(7)], [6.5, 7, 100]])
    ours = oracle.e2m1_mag_of(y)
    ref = [nearest_code(Fraction(float(v)), table) for v in y]
    assert ours.tolist() == ref


def test_e8m0_decode():
    assert oracle.e8m0_decode(127) == 1.0
    assert oracle.e8m0_decode(0) == 2.0 ** -127
    assert oracle.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_decode(255))
    for b in range(255):
        assert oracle.e8m0_decode(b) == float(Fraction(2) ** (b - 127))
