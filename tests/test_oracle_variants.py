"""Pins of the oracle's format and scale-type variants: E5M2 elements, E8M0
(MX-style) scales on INT and FP8 elements, FP16 scales on FP8 elements, and
16- and 64-element blocks, for every supported (format, scale, block).

Pinned against: the brute-force statement in exact rationals
(tests/brute.py: argmin over every code, values from torch's float8 tables
and the field widths), torch's float8_e5m2 casts, the page facts, and
invariants that tie each variant to the already pinned default codecs."""
from fractions import Fraction
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests import brute
from tests.arbitrary import CODE_BITS, E8M0_CODECS, arbitrary_tile, e8m0_every_pair_stream
from tests.test_oracle_quant import special_tile

RNG = np.random.default_rng(2024)
ALL = sorted(oracle.ALL_CODECS)
X = np.concatenate([special_tile(1), special_tile(2)[:300]])          # 1 tile + ragged tail


def facts():
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")) as f:
        return json.load(f)


# ---- sizes ------------------------------------------------------------------

@pytest.mark.parametrize("name", ALL)
def test_tile_bytes_are_code_region_plus_scales(name):
    c = oracle.ALL_CODECS[name]
    assert oracle.tile_bytes(c) == brute.codec_tile_bytes(c)
    assert oracle.tile_bytes(c) % 16 == 0
    assert oracle.packed_bytes(c, 2048 * 3 + 1) == 4 * oracle.tile_bytes(c)


def test_default_codecs_keep_their_sizes():
    for name, tb in [("int4_f16_b32", 1152), ("int3_f16_b32", 896), ("e4m3_f32_b32", 2304),
                     ("e2m1_e8m0_b32", 1088)]:
        assert oracle.tile_bytes(oracle.ALL_CODECS[name]) == tb


# ---- E5M2 -------------------------------------------------------------------

def test_e5m2_decode_all_codes_vs_torch_and_page():
    f = facts()
    ours = np.array([oracle.e5m2_decode(c) for c in range(256)], dtype=np.float32)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # page: 5 exponent / 2 mantissa bits, IEEE specials (infinity, NaNs)
    assert f["e5m2_field_widths"]["value"] == {"exponent": 5, "mantissa": 2}
    assert f["e5m2_ieee_special_values"]["value"]
    assert ours[0x7C] == np.inf and ours[0xFC] == -np.inf
    assert [c for c in range(128) if np.isnan(ours[c])] == [0x7D, 0x7E, 0x7F]
    assert np.nanmax(ours[np.isfinite(ours)]) == 57344.0


def test_e5m2_encode_vs_torch_cast():
    """|y| <= 57344: the oracle's nearest-even code equals torch's RNE cast;
    above it the oracle saturates at 57344 (finite data never encodes to inf)."""
    e5 = np.array([float(v) for v in brute.E5M2])
    mids = (e5[:-1] + e5[1:]) / 2
    rnd = np.abs(RNG.standard_normal(200000) * 3000).astype(np.float32)
    rnd = np.concatenate([rnd, RNG.uniform(0, 2**-13, 50000).astype(np.float32)])
    y = np.concatenate([e5, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)), rnd]).astype(np.float32)
    y = y[y <= 57344]
    ours = oracle.e5m2_mag_of_quotient(y.astype(np.float64), 1.0)
    ref = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy().astype(np.int32)
    assert np.array_equal(ours, ref)
    big = np.array([57345.0, 61440.0, 65536.0, 1e9], dtype=np.float64)
    assert (oracle.e5m2_mag_of_quotient(big, 1.0) == 0x7B).all()


def test_e5m2_quotient_brute_force():
    den = np.abs(RNG.standard_normal(2000)).astype(np.float32) + np.float32(1e-3)
    num = (RNG.uniform(0, 60000, 2000) * den).astype(np.float32)
    ours = oracle.e5m2_mag_of_quotient(num.astype(np.float64), den.astype(np.float64))
    ref = [brute.nearest_code(Fraction(float(a)) / Fraction(float(b)), brute.E5M2) for a, b in zip(num, den)]
    assert ours.tolist() == ref


# ---- scale rules ------------------------------------------------------------

def test_element_emax_and_e8m0_exponent():
    """The MX shared exponent is floor(log2 a) minus the element format's
    largest exponent: 6 = 1.5*2^2, 448 = 1.75*2^8, 57344 = 1.75*2^15, and for
    the integers floor(log2 qmax)."""
    assert [oracle.elem_emax(f) for f in (1, 2, 3, 4, 5)] == [2, 1, 8, 2, 15]
    a = np.concatenate([np.abs(RNG.standard_normal(5000) * 10.0 ** RNG.integers(-30, 30, 5000)),
                        [0.0, 1e-45, 3e38, 1.0, 2.0, 0.75]]).astype(np.float32)
    for emax in (1, 2, 8, 15):
        ours = oracle.e8m0_exponent(a, emax)
        ref = [-127 if v == 0 else max(-127, min(127, brute._floor_log2(Fraction(float(v))) - emax)) for v in a]
        assert ours.tolist() == ref


def test_fp8_fp16_scale_rule_vs_numpy():
    a = np.abs(RNG.standard_normal(20000) * 10.0 ** RNG.integers(-8, 10, 20000)).astype(np.float32)
    for fmt, fmax in ((oracle.FMT_FP8_E4M3, 448.0), (oracle.FMT_FP8_E5M2, 57344.0)):
        ours = oracle.fp8_scale_f16_bits(a, fmt)
        s32 = np.minimum(a / np.float32(fmax), np.float32(65504.0)).astype(np.float32)
        assert np.array_equal(ours, s32.astype(np.float16).view(np.uint16))
        assert oracle.fp8_scale_f32(448.0 * 3, oracle.FMT_FP8_E4M3) == 3.0
        assert oracle.fp8_scale_f32(57344.0 * 3, oracle.FMT_FP8_E5M2) == 3.0


# ---- whole tiles against brute force -----------------------------------------

@pytest.mark.parametrize("name", ALL)
def test_variant_tiles_equal_brute_force(name):
    c = oracle.ALL_CODECS[name]
    assert oracle.quantize_pack(c, X).tobytes() == brute.encode_codec(c, X)


@pytest.mark.parametrize("name", ALL)
def test_variant_unpack_equals_brute_decode(name):
    c = oracle.ALL_CODECS[name]
    p = oracle.quantize_pack(c, X[:2048])
    ours = oracle.unpack_dequant(c, p, 2048, oracle.DT_FP32)
    ref = brute.decode_codec(c, p.tobytes())
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name", ALL)
def test_variant_reduce_equals_brute_force(name):
    c = oracle.ALL_CODECS[name]
    n = 2048 + 100
    # scaled so that no sum overflows (non-finite inputs are outside the spec)
    xs = [X[:n] * np.float32(0.25), (RNG.standard_normal(n) * 3).astype(np.float32),
          np.concatenate([special_tile(7), special_tile(8)])[:n] * np.float32(0.25)]
    streams = [oracle.quantize_pack(c, x) for x in xs]
    ours, sums = oracle.dequant_reduce_requant(c, streams, n, want_sum=True)
    ref, ref_sums = brute.reduce_codec(c, streams, n)
    assert ours.tobytes() == ref
    ok = (sums.view(np.uint32) == ref_sums.view(np.uint32)) | (np.isnan(sums) & np.isnan(ref_sums))
    assert ok.all()


# ---- variants tied to the pinned default codecs -----------------------------

def _equalize(v: np.ndarray, group: int, sub: int) -> np.ndarray:
    """Copy each group's largest-|v| element into every sub-block of the group,
    so all sub-blocks of a group share the group's absmax."""
    v = v.copy()
    for g in range(v.size // group):
        seg = v[g * group:(g + 1) * group]
        i = int(np.argmax(np.abs(seg)))
        for s in range(group // sub):
            if not (s * sub <= i < (s + 1) * sub):
                seg[s * sub] = seg[i]
    return v


def _codes_and_scales(c, p: np.ndarray):
    cb = brute.CODE_BYTES[c[0]]
    tb = oracle.tile_bytes(c)
    t = p.reshape(-1, tb)
    return t[:, :cb], t[:, cb:]


@pytest.mark.parametrize("el,sc", [(1, 1), (2, 1), (1, 3), (2, 3), (3, 2), (3, 1), (3, 3), (5, 2), (5, 1),
                                   (5, 3), (4, 3)])
def test_block_sizes_agree_when_sub_blocks_share_absmax(el, sc):
    """16-element blocks give the 32-element codes when both halves of every
    32 block have the same absmax (each scale then appears twice); 64-element
    blocks give them when both 32 blocks of every 64 do."""
    base = (RNG.standard_normal(4096) * np.exp(RNG.uniform(-3, 3, 4096))).astype(np.float32)
    v16 = _equalize(base, 32, 16)
    c32, c16 = (el, sc, 32), (el, sc, 16)
    k32, s32 = _codes_and_scales(c32, oracle.quantize_pack(c32, v16))
    k16, s16 = _codes_and_scales(c16, oracle.quantize_pack(c16, v16))
    sz = brute.SCALE_SIZE[sc]
    assert np.array_equal(k16, k32)
    assert np.array_equal(s16.reshape(-1, 64, 2, sz)[:, :, 0], s32.reshape(-1, 64, sz))
    assert np.array_equal(s16.reshape(-1, 64, 2, sz)[:, :, 1], s32.reshape(-1, 64, sz))
    v64 = _equalize(base, 64, 32)
    c64 = (el, sc, 64)
    k32, s32 = _codes_and_scales(c32, oracle.quantize_pack(c32, v64))
    k64, s64 = _codes_and_scales(c64, oracle.quantize_pack(c64, v64))
    assert np.array_equal(k64, k32)
    assert np.array_equal(s64.reshape(-1, 32, sz), s32.reshape(-1, 32, 2, sz)[:, :, 0])


@pytest.mark.parametrize("el,qmax", [(1, 7), (2, 3)])
def test_e8m0_int_half_step_bound_and_clipping(el, qmax):
    """INT elements with a power-of-two scale S = 2^e: |v - q S| <= S/2 unless
    |v|/S >= qmax + 1/2, where the code clips to qmax; the block max lands in
    [2^k, 2^(k+1)) with k = floor(log2 qmax)."""
    c = (el, oracle.SCALE_E8M0, 32)
    v = (RNG.standard_normal(2048 * 4) * np.exp(RNG.uniform(-5, 5, 2048 * 4))).astype(np.float32)
    p = oracle.quantize_pack(c, v)
    d = oracle.unpack_dequant(c, p, v.size, oracle.DT_FP32)
    tb = oracle.tile_bytes(c)
    sbytes = p.reshape(-1, tb)[:, brute.CODE_BYTES[el]:].reshape(-1).astype(np.int64)
    S = np.ldexp(1.0, sbytes - 127).repeat(32)
    y = np.abs(v.astype(np.float64)) / S
    unclipped = y < qmax + 0.5
    assert (np.abs(v - d)[unclipped] <= S[unclipped] / 2).all()
    assert (np.abs(d[~unclipped]) == qmax * S[~unclipped]).all()
    amax = np.abs(v.reshape(-1, 32)).max(axis=1)
    k = int(np.floor(np.log2(qmax)))
    r = amax / np.ldexp(1.0, sbytes - 127)
    assert ((r >= 2 ** k) & (r < 2 ** (k + 1))).all()


@pytest.mark.parametrize("name", [n for n in ALL if "_e8m0_" in n])
def test_e8m0_k1_reduce_is_identity(name):
    """A power-of-two scale is recomputed exactly from the decoded block, so a
    one-stream reduce returns the packed tiles unchanged."""
    c = oracle.ALL_CODECS[name]
    v = (RNG.standard_normal(2048 * 2) * np.exp(RNG.uniform(-4, 4, 4096))).astype(np.float32)
    p = oracle.quantize_pack(c, v)
    out, _ = oracle.dequant_reduce_requant(c, [p], v.size)
    assert np.array_equal(out, p)


@pytest.mark.parametrize("name", [n for n in ALL if "_e8m0_" in n])
def test_e8m0_k_copies_shift_exponent(name):
    """K copies of one stream (K a power of two) keep every code and add
    log2 K to every scale byte."""
    c = oracle.ALL_CODECS[name]
    v = (RNG.standard_normal(2048) * np.exp(RNG.uniform(-4, 4, 2048))).astype(np.float32)
    p = oracle.quantize_pack(c, v)
    for K in (2, 4):
        out, _ = oracle.dequant_reduce_requant(c, [p] * K, v.size)
        k0, s0 = _codes_and_scales(c, p)
        k1, s1 = _codes_and_scales(c, out)
        assert np.array_equal(k1, k0)
        assert np.array_equal(s1.astype(np.int64), s0.astype(np.int64) + int(np.log2(K)))


def test_fp16_scaled_fp8_zero_and_subnormal_scales():
    """FP8 with an FP16 scale: a block whose scale rounds to 0 is all-zero
    bytes; a subnormal fp16 scale still gives the nearest code of the exact
    quotient (brute force)."""
    c = (oracle.FMT_FP8_E4M3, oracle.SCALE_FP16, 32)
    v = np.zeros(2048, dtype=np.float32)
    v[:32] = RNG.standard_normal(32).astype(np.float32) * np.float32(1e-9)    # scale -> 0
    v[32:64] = RNG.standard_normal(32).astype(np.float32) * np.float32(3e-3)   # subnormal fp16 scale
    v[64:96] = -0.0
    p = oracle.quantize_pack(c, v)
    assert not p[:16].any() and not p[1024:1040].any() and not p[2048:2050].any()
    assert p.tobytes() == brute.encode_codec(c, v)


# ---- decode of arbitrary bytes ------------------------------------------------

def same_values(got, ref):
    g, r = np.asarray(got, dtype=np.float32), np.asarray(ref, dtype=np.float32)
    ok = (g.view(np.uint32) == r.view(np.uint32)) | (np.isnan(g) & np.isnan(r))
    assert ok.all(), [(int(i), float(g[i]), float(r[i])) for i in np.nonzero(~ok)[0][:6]]


@pytest.mark.parametrize("name", ALL)
def test_decode_of_arbitrary_bytes_equals_brute_decode(name):
    """Every bit pattern decodes to fp32(code * scale), rounded once (the
    brute-force decode in exact rationals; IEEE products for non-finite
    scales): NaN and infinite codes and scales, subnormal scales, and E8M0
    exponents whose products overflow binary32.  Two such streams reduce to
    the binary32 sums of those values."""
    c = oracle.ALL_CODECS[name]
    t0, t1 = arbitrary_tile(c, 11), arbitrary_tile(c, 12)
    d0, d1 = brute.decode_codec(c, t0.tobytes()), brute.decode_codec(c, t1.tobytes())
    same_values(oracle.unpack_dequant(c, t0, 2048, oracle.DT_FP32), d0)
    _, sums = oracle.dequant_reduce_requant(c, [t0, t1], 2048, want_sum=True)
    with np.errstate(all="ignore"):
        want = (d0 + d1).astype(np.float32)
    same_values(sums, want)
    if c[1] == 3:                                   # the planted E8M0 bytes reach binary32's end
        assert np.isinf(d0).any() and np.isnan(d0).any()


@pytest.mark.parametrize("name", E8M0_CODECS)
def test_e8m0_every_pair_stream_covers_every_pair(name):
    """The stream really pairs every code with every scale byte (read back
    with the brute-force layout), and the oracle decodes it as brute force
    does, overflowing products included."""
    c = oracle.ALL_CODECS[name]
    fmt, _, bl = c
    p, n = e8m0_every_pair_stream(c)
    tb = brute.codec_tile_bytes(c)
    seen = set()
    for t in range(n // brute.TILE):
        tile = p[t * tb:(t + 1) * tb].tobytes()
        for i in range(brute.TILE):
            sb = tile[brute.CODE_BYTES[fmt] + i // bl]
            if fmt in (1, 4):
                code = (tile[i // 2] >> (4 * (i % 2))) & 15
            elif fmt == 2:
                code = None                          # checked through the decode below
            else:
                code = brute.fp8_byte(tile, i)
            seen.add((code, sb))
        if t < 2:
            same_values(oracle.unpack_dequant(c, p[t * tb:(t + 1) * tb], brute.TILE, oracle.DT_FP32),
                        brute.decode_codec(c, tile))
    if fmt != 2:
        assert len(seen) == (1 << CODE_BITS[fmt]) * 256
    else:
        d = oracle.unpack_dequant(c, p, n, oracle.DT_FP32).reshape(-1, bl)
        sbytes = np.concatenate([p[t * tb + brute.CODE_BYTES[fmt]:(t + 1) * tb] for t in range(n // brute.TILE)])
        for s in (1, 127, 200):                      # exponents where every product is finite
            vals = set(np.unique(d[sbytes == s]).tolist())
            assert vals == {float(np.float32(q * 2.0 ** (s - 127))) for q in range(-3, 4)}
