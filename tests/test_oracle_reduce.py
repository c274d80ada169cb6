"""Pins of the oracle's dequant -> FP32 accumulate -> requant against brute
force, library float32 arithmetic, the exact sum and closed-form invariants
(K = 1 idempotence, K copies of one stream)."""
import math

import numpy as np
import pytest

import oracle
from tests import brute
from tests.test_oracle_quant import special_tile

RNG = np.random.default_rng(7)
FMTS = ["int4", "int3", "fp8", "mxfp4"]


def codec(fmt):
    return oracle.CODECS[fmt]


def streams_for(fmt, n, k, seed=0):
    r = np.random.default_rng(seed)
    out = []
    for j in range(k):
        x = (r.standard_normal(n) * r.uniform(0.1, 3)).astype(np.float32)
        if j == 1 and n >= 2048:
            x[:2048] = special_tile(seed + j)
        out.append(oracle.quantize_pack(codec(fmt), x))
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_reduce_equals_brute_force(fmt):
    n = 2048 + 777
    s = streams_for(fmt, n, 3, seed=1)
    out, sums = oracle.dequant_reduce_requant(codec(fmt), s, n, want_sum=True)
    ref, rsums = brute.reduce(fmt, [x.tobytes() for x in s], n)
    assert out.tobytes() == ref
    assert np.array_equal(sums.view(np.uint32), rsums.view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [1, 2, 5, 16])
def test_sums_are_sequential_float32_adds(fmt, k):
    n = 4096 + 100
    s = streams_for(fmt, n, k, seed=k)
    _, sums = oracle.dequant_reduce_requant(codec(fmt), s, n, want_sum=True)
    d = [oracle.unpack_dequant(codec(fmt), x, n) for x in s]
    acc = d[0].copy()
    for j in range(1, k):
        acc = (acc + d[j]).astype(np.float32)
    assert np.array_equal(sums.view(np.uint32), acc.view(np.uint32))


@pytest.mark.parametrize("fmt", ["int4", "int3", "mxfp4"])
def test_sum_within_rounding_bound_of_exact_sum(fmt):
    """For INT and MX every decoded term is exact, so the exact sum is known;
    K-1 binary32 additions stay within (K-1) 2^-24 sum|d| of it."""
    n, k = 2048, 8
    s = streams_for(fmt, n, k, seed=3)
    _, sums = oracle.dequant_reduce_requant(codec(fmt), s, n, want_sum=True)
    d = np.stack([oracle.unpack_dequant(codec(fmt), x, n).astype(np.float64) for x in s])
    for i in range(0, n, 7):
        exact = math.fsum(d[:, i])
        bound = (k - 1) * 2.0 ** -24 * math.fsum(np.abs(d[:, i]))
        assert abs(sums[i] - exact) <= bound


@pytest.mark.parametrize("fmt", ["int4", "int3", "mxfp4"])
def test_k1_is_identity_on_packed_tiles(fmt):
    """Re-encoding decoded values reproduces the tile when every block's scale
    is a normal, unsaturated fp16 (INT) -- always for MX."""
    x = (RNG.standard_normal(2048 * 3) * 2).astype(np.float32)
    p = oracle.quantize_pack(codec(fmt), x)
    out, _ = oracle.dequant_reduce_requant(codec(fmt), [p], x.size)
    assert np.array_equal(out, p)


def test_k1_fp8_codes_kept_when_scale_kept():
    x = (RNG.standard_normal(2048 * 3) * 0.5).astype(np.float32)
    p = oracle.quantize_pack(oracle.FP8, x)
    out, _ = oracle.dequant_reduce_requant(oracle.FP8, [p], x.size)
    for t in range(3):
        sp = np.frombuffer(p[t * 2304 + 2048:(t + 1) * 2304].tobytes(), np.float32)
        so = np.frombuffer(out[t * 2304 + 2048:(t + 1) * 2304].tobytes(), np.float32)
        ulps = np.abs(sp.view(np.int32).astype(np.int64) - so.view(np.int32).astype(np.int64))
        assert (ulps <= 1).all()
        for b in range(64):
            if sp[b] == so[b]:
                assert np.array_equal(p[t * 2304 + 32 * b: t * 2304 + 32 * b + 32],
                                      out[t * 2304 + 32 * b: t * 2304 + 32 * b + 32])


@pytest.mark.parametrize("fmt,k", [("int4", 2), ("int3", 4), ("int4", 8), ("mxfp4", 2),
                                   ("mxfp4", 8), ("int3", 16)])
def test_k_copies_scale_by_k(fmt, k):
    """K identical streams: same codes, scale times K (fp16 scale x K for INT,
    exponent + log2 K for MX) while scales stay normal and unsaturated."""
    x = (RNG.standard_normal(2048 * 2) * 0.3).astype(np.float32)
    p = oracle.quantize_pack(codec(fmt), x)
    out, _ = oracle.dequant_reduce_requant(codec(fmt), [p] * k, x.size)
    tb = oracle.tile_bytes(codec(fmt))
    for t in range(2):
        a, b = p[t * tb:(t + 1) * tb], out[t * tb:(t + 1) * tb]
        if fmt == "mxfp4":
            assert np.array_equal(a[:1024], b[:1024])
            assert np.array_equal(a[1024:].astype(int) + int(math.log2(k)), b[1024:].astype(int))
        else:
            off = 1024 if fmt == "int4" else 768
            assert np.array_equal(a[:off], b[:off])
            sa = np.frombuffer(a[off:].tobytes(), np.float16).astype(np.float64)
            sb = np.frombuffer(b[off:].tobytes(), np.float16).astype(np.float64)
            assert np.array_equal(sa * k, sb)


@pytest.mark.parametrize("fmt", FMTS)
def test_tail_codes_are_ignored(fmt):
    """Positions beyond n count as +0 whatever bytes the inputs hold there."""
    n = 2048 + 40
    s = streams_for(fmt, n, 2, seed=5)
    junk = [x.copy() for x in s]
    tb = oracle.tile_bytes(codec(fmt))
    # scramble the second tile's code bytes of blocks 2.. (elements 64.., all past n)
    if fmt == "int3":
        junk[0][tb + 16:tb + 512] = RNG.integers(0, 256, 496, dtype=np.uint8)
        junk[0][tb + 512 + 8:tb + 768] = RNG.integers(0, 256, 248, dtype=np.uint8)
    elif fmt == "fp8":
        # groups 2.. of both code planes (elements 64.., all past n)
        junk[0][tb + 32:tb + 1024] = RNG.integers(0, 127, 992, dtype=np.uint8)
        junk[0][tb + 1056:tb + 2048] = RNG.integers(0, 127, 992, dtype=np.uint8)
    else:
        junk[0][tb + 32:tb + 1024] = RNG.integers(0, 256, 992, dtype=np.uint8)
    a, _ = oracle.dequant_reduce_requant(codec(fmt), s, n)
    b, _ = oracle.dequant_reduce_requant(codec(fmt), junk, n)
    ref, _ = brute.reduce(fmt, [x.tobytes() for x in junk], n)
    assert b.tobytes() == ref
    assert np.array_equal(a, b)


def test_status_codes():
    p = oracle.quantize_pack(oracle.INT4, np.ones(10, np.float32))
    arr = (oracle.ctypes.c_void_p * 17)(*([p.ctypes.data] * 17))
    o = np.zeros_like(p)
    lib = oracle.lib()
    assert lib.rco_dequant_reduce_requant(oracle.Codec(*oracle.INT4), arr, 17, 10,
                                          o.ctypes.data, None) == oracle.ERR_RANGE
    assert lib.rco_dequant_reduce_requant(oracle.Codec(*oracle.INT4), arr, 0, 10,
                                          o.ctypes.data, None) == oracle.ERR_RANGE
    assert lib.rco_quantize_pack(oracle.Codec(1, 2, 32), 1, None, 10, None) == oracle.ERR_UNSUPPORTED
    assert lib.rco_quantize_pack(oracle.Codec(*oracle.INT4), 1, None, 10, None) == oracle.ERR_NULL
    assert lib.rco_quantize_pack(oracle.Codec(*oracle.INT4), 1, None, 0, None) == oracle.OK


@pytest.mark.parametrize("fmt", FMTS)
def test_allreduce_emulation_is_the_composed_pipeline(fmt):
    """The emulated all-reduce: two-shot = unpack of the requantized sum,
    one-shot = the FP32 sums rounded to the messages' dtype; with K copies of
    one INT/MX message (K a power of two) the two-shot result is K times the
    one-message round trip, exactly."""
    c = oracle.CODECS[fmt]
    n = 2048 + 500
    msgs = [(np.random.default_rng(j).standard_normal(n) * (j + 1)).astype(np.float32) for j in range(3)]
    out2, packed = oracle.allreduce_emulate(c, msgs, oracle.DT_FP32, two_shot=True)
    streams = [oracle.quantize_pack(c, m) for m in msgs]
    red, sums = oracle.dequant_reduce_requant(c, streams, n, want_sum=True)
    assert np.array_equal(packed, red)
    assert np.array_equal(out2.view(np.uint32), oracle.unpack_dequant(c, red, n).view(np.uint32))
    out1, _ = oracle.allreduce_emulate(c, msgs, oracle.DT_FP32, two_shot=False)
    assert np.array_equal(out1.view(np.uint32), sums.view(np.uint32))
    if fmt != "fp8":
        x = msgs[0]
        one = oracle.unpack_dequant(c, oracle.quantize_pack(c, x), n)
        four, _ = oracle.allreduce_emulate(c, [x] * 4, oracle.DT_FP32, two_shot=True)
        assert np.array_equal(four, one * np.float32(4))
