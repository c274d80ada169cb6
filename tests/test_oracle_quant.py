"""Pins of the oracle's quantize / pack / unpack against brute force in exact
rationals (tests/brute.py), library arithmetic (numpy float32 / float16) and
invariants the method fixes (half-step error bound, zero blocks, symmetry,
grid round trip)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import brute

RNG = np.random.default_rng(99)
FMTS = ["int4", "int3", "fp8", "mxfp4"]


def codec(fmt):
    return oracle.CODECS[fmt]


def special_tile(seed: int) -> np.ndarray:
    """One 2048-value tile mixing the cases a mistake would hide in: normal
    blocks, an outlier block, a zero block, a block with one negative zero,
    tiny (fp16-subnormal-scale) blocks, huge (saturating) blocks, exact grid
    values, ties and denormal floats."""
    r = np.random.default_rng(seed)
    v = r.standard_normal(2048).astype(np.float32)
    v[32:64] *= 50
    v[64:96] = 0
    v[96:128] = 0
    v[100] = -0.0
    v[128:160] = (r.standard_normal(32) * 1e-5).astype(np.float32)       # subnormal fp16 scale
    v[160:192] = (r.standard_normal(32) * 1e-7).astype(np.float32)       # scale may flush to 0
    v[192:224] = (r.standard_normal(32) * 3e5).astype(np.float32)        # saturating fp16 scale
    v[224:256] = (r.integers(-7, 8, 32) * 0.25).astype(np.float32)       # grid
    v[224] = 1.75
    # ties for INT3 with s = 0.25 (absmax 0.75): k + 1/2 steps
    v[256:288] = (r.integers(-3, 4, 32) * 0.25).astype(np.float32)
    v[256] = 0.75
    v[257:263] = [0.125, 0.375, 0.625, -0.125, -0.375, -0.625]
    v[288:320] = r.uniform(-1, 1, 32).astype(np.float32) * np.float32(1e-38)  # denormals
    v[320:352] = np.float32(3.0e38) * r.uniform(-1, 1, 32).astype(np.float32)
    return v


@pytest.mark.parametrize("fmt", FMTS)
def test_tiles_equal_brute_force(fmt):
    x = np.concatenate([special_tile(1), special_tile(2)[:1500]])     # 2 tiles, ragged tail
    ours = oracle.quantize_pack(codec(fmt), x)
    ref = brute.encode(fmt, x)
    assert ours.tobytes() == ref


@pytest.mark.parametrize("fmt", FMTS)
def test_unpack_equals_brute_decode(fmt):
    x = special_tile(3)
    p = oracle.quantize_pack(codec(fmt), x)
    ours = oracle.unpack_dequant(codec(fmt), p, x.size, oracle.DT_FP32)
    ref = brute.decode_tile(fmt, p.tobytes())
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_int_magnitude_brute_force():
    """Round-half-even of the exact quotient |v| / s, clamped to qmax, against
    an exact-rational argmin over every candidate, on fp16 scales (normal and
    subnormal), random values and values at exact half steps."""
    hbits = RNG.integers(1, 0x7BFF, 4000).astype(np.uint16)
    den = hbits.view(np.float16).astype(np.float32)
    q = RNG.uniform(0, 8.5, 4000)
    num = (q * den).astype(np.float32)
    k = RNG.integers(0, 8, 1000)
    tnum = ((k + 0.5) * den[:1000].astype(np.float64)).astype(np.float32)     # exact ties
    num = np.concatenate([num, tnum])
    den = np.concatenate([den, den[:1000]])
    for qmax in (3, 7):
        ours = oracle.int_mag(num, den, qmax)
        ref = [brute.int_mag(a, b, qmax) for a, b in zip(num, den)]
        assert ours.tolist() == ref


@pytest.mark.parametrize("qmax", [3, 7])
def test_int_half_steps_by_construction(qmax):
    """v = (k + 1/2) s exactly (a binary32 value: at most 4 + 11 significant
    bits) rounds to the even one of k, k + 1; the binary32 neighbours of that
    v round away from the half step, to k + 1 above it and k below.  The
    expected codes follow from the definition alone."""
    hb = np.concatenate([RNG.integers(0x0001, 0x0400, 300),          # subnormal fp16 scales
                         RNG.integers(0x0400, 0x7BFF, 1500)]).astype(np.uint16)
    s = hb.view(np.float16).astype(np.float32)
    for k in range(qmax):
        v = ((k + 0.5) * s.astype(np.float64)).astype(np.float32)
        assert np.array_equal(v.astype(np.float64), (k + 0.5) * s.astype(np.float64))
        even = k if k % 2 == 0 else k + 1
        assert (oracle.int_mag(v, s, qmax) == even).all()
        up = np.nextafter(v, np.float32(np.inf))
        dn = np.nextafter(v, np.float32(0))
        assert (oracle.int_mag(up, s, qmax) == k + 1).all()
        assert (oracle.int_mag(dn, s, qmax) == k).all()
    # beyond qmax + 1/2 the code saturates; just below it stays qmax
    v = ((qmax + 0.5) * s.astype(np.float64)).astype(np.float32)
    assert (oracle.int_mag(v, s, qmax) == qmax).all()
    assert (oracle.int_mag(v * np.float32(40), s, qmax) == qmax).all()
    assert (oracle.int_mag(np.nextafter(v, np.float32(0)), s, qmax) == qmax).all()


@pytest.mark.parametrize("el,qmax", [(oracle.FMT_INT4, 7), (oracle.FMT_INT3, 3)])
def test_e8m0_int_half_steps_go_to_even(el, qmax):
    """INT codes with a power-of-two (E8M0) scale S: a block whose maximum is
    (qmax - 1/2) S has scale S (the maximum lies in [2^k, 2^(k+1)) S with
    k = floor(log2 qmax)), and its exact half steps (j + 1/2) S decode to the
    even one of j, j + 1 times S, with the sign kept ("Microscaling Data
    Formats for Deep Learning", abstract: narrow integer elements under a
    shared power-of-two scale; ties to even as for every rounding here)."""
    c = (el, oracle.SCALE_E8M0, 32)
    blocks = []
    want = []
    for e in (-30, -3, 0, 5, 40):
        S = 2.0 ** e
        halves = [(j + 0.5) * S for j in range(qmax)]
        vals = [(qmax - 0.5) * S] + [h * sgn for h in halves for sgn in (1, -1)]
        vals += [0.0] * (32 - len(vals))
        blocks.append(vals)
        want.append([(qmax - 1 if (qmax - 1) % 2 == 0 else qmax) * S] +
                    [sgn * (j if j % 2 == 0 else j + 1) * S for j in range(qmax) for sgn in (1, -1)] +
                    [0.0] * (32 - 1 - 2 * qmax))
    v = np.array(blocks, dtype=np.float32).reshape(-1)
    d = oracle.unpack_dequant(c, oracle.quantize_pack(c, v), v.size, oracle.DT_FP32)
    assert np.array_equal(d, np.array(want, dtype=np.float32).reshape(-1))


def test_scale_rules_vs_numpy():
    a = np.concatenate([np.abs(RNG.standard_normal(20000)) * 10.0 ** RNG.integers(-12, 7, 20000),
                        [0.0, 1e-45, 3 * 2**-25, 3 * 65504, 7 * 65504, 3e38, 6.1e-5]]).astype(np.float32)
    for qmax in (3, 7):
        ours = oracle.int_scale_bits(a, qmax)
        ref = np.array([brute.int_scale(x, qmax).view(np.uint16) for x in a], dtype=np.uint16)
        assert np.array_equal(ours, ref)
    ours = oracle.fp8_scale(a)
    ref = np.array([brute.fp8_scale(x) for x in a], dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    ours = oracle.mx_exponent(a[:3000])
    ref = [brute.mx_exponent(float(x)) for x in a[:3000]]
    assert ours.tolist() == ref


@pytest.mark.parametrize("fmt,qmax", [("int4", 7), ("int3", 3)])
def test_int_half_step_bound_and_max_code(fmt, qmax):
    """|v - d| <= s/2 for every element of a block whose fp16 scale is normal
    and unsaturated, on full-mantissa binary32 inputs and on bf16 inputs with
    planted exact half steps; where |v| / s is exactly k + 1/2 the code is the
    even neighbour; the element attaining the block max gets code +-qmax."""
    from fractions import Fraction
    x32 = RNG.standard_normal(2048 * 8).astype(np.float32) * np.float32(3.0)
    xb = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(RNG.standard_normal(2048 * 8).astype(np.float32)))
    # the first two tiles: blocks whose maximum is qmax * 2^j (so s = 2^j
    # exactly) and whose other elements are half steps +-(k + 1/2) 2^j
    pw = 2.0 ** RNG.integers(-4, 4, 128)
    xb[:4096] = (RNG.integers(0, qmax, 4096) + 0.5) * np.repeat(pw, 32) * RNG.choice([-1.0, 1.0], 4096)
    xb[:4096:32] = qmax * pw
    ties = 0
    for x in (x32, xb.astype(np.float32)):
        p = oracle.quantize_pack(codec(fmt), x)
        d = oracle.unpack_dequant(codec(fmt), p, x.size)
        tb = oracle.tile_bytes(codec(fmt))
        soff = 1024 if fmt == "int4" else 768
        for t in range(8):
            s = np.frombuffer(p[t * tb + soff: t * tb + soff + 128].tobytes(), dtype=np.float16).astype(np.float64)
            for b in range(64):
                sl = slice(t * 2048 + 32 * b, t * 2048 + 32 * b + 32)
                xv = x[sl].astype(np.float64)
                err = np.abs(xv - d[sl].astype(np.float64))
                assert (err <= s[b] / 2).all()
                j = np.argmax(np.abs(x[sl]))
                assert abs(d[sl][j]) == qmax * s[b]
                for e in np.nonzero(err == s[b] / 2)[0]:
                    q = Fraction(float(d[sl][e])) / Fraction(float(s[b]))
                    assert q.denominator == 1 and q.numerator % 2 == 0
                    ties += 1
    assert ties > 100          # the planted half steps are there


def test_fp8_error_bound():
    """Every element lands on the E4M3 value nearest to v/s: the error is at
    most half the E4M3 spacing at that magnitude times s."""
    x = (RNG.standard_normal(2048 * 4) * 0.5).astype(np.float32)
    p = oracle.quantize_pack(oracle.FP8, x)
    d = oracle.unpack_dequant(oracle.FP8, p, x.size).astype(np.float64)
    for t in range(4):
        s = np.frombuffer(p[t * 2304 + 2048: t * 2304 + 2304].tobytes(), dtype=np.float32).astype(np.float64)
        for b in range(64):
            sl = slice(t * 2048 + 32 * b, t * 2048 + 32 * b + 32)
            y = np.abs(x[sl]) / s[b]
            spacing = np.where(y < 2**-6, 2**-9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2**-6))) - 3))
            err = np.abs(x[sl] - d[sl]) / s[b]
            assert (err <= spacing / 2 * (1 + 1e-6) + 1e-12).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_blocks_are_zero_bytes(fmt):
    x = np.zeros(5000, dtype=np.float32)
    p = oracle.quantize_pack(codec(fmt), x)
    if fmt == "mxfp4":
        # the E8M0 scale of an all-zero block is the smallest scale, 2^-127 (byte 0)
        assert not p.any()
    else:
        assert not p.any()
    assert not oracle.unpack_dequant(codec(fmt), p, 5000).any()


@pytest.mark.parametrize("fmt", FMTS)
def test_sign_symmetry(fmt):
    """pack(-x): same scales and magnitudes, every sign bit flipped."""
    x = special_tile(7)[:1024]
    x = x[np.abs(x) < 1e30]
    p = oracle.quantize_pack(codec(fmt), x)
    q = oracle.quantize_pack(codec(fmt), -x)
    dp = oracle.unpack_dequant(codec(fmt), p, x.size)
    dq = oracle.unpack_dequant(codec(fmt), q, x.size)
    # zero-scale blocks are all-zero bytes by definition (+0 both ways)
    live = np.repeat(block_scale_nonzero(fmt, p), 32)[:x.size]
    assert np.array_equal((-dp[live]).view(np.uint32), dq[live].view(np.uint32))
    assert not dp[~live].view(np.uint32).any() and not dq[~live].view(np.uint32).any()


def block_scale_nonzero(fmt, p):
    tb = oracle.tile_bytes(codec(fmt))
    off, w = {"int4": (1024, 2), "int3": (768, 2), "fp8": (2048, 4), "mxfp4": (1024, 1)}[fmt]
    out = []
    for t in range(p.size // tb):
        sc = p[t * tb + off: t * tb + off + 64 * w].reshape(64, w)
        nz = sc.any(axis=1)
        if fmt == "mxfp4":
            nz = np.ones(64, dtype=bool)     # every MX block keeps its signs
        out.append(nz)
    return np.concatenate(out)


@pytest.mark.parametrize("fmt,qmax", [("int4", 7), ("int3", 3)])
def test_int_grid_round_trip(fmt, qmax):
    """Blocks of q*s with s an fp16 value and one element at qmax*s decode to
    exactly the input."""
    s = np.float16(RNG.uniform(0.01, 10, 64)).astype(np.float32)
    q = RNG.integers(-qmax, qmax + 1, (64, 32))
    q[:, 5] = qmax
    x = (q * s[:, None]).astype(np.float32).ravel()
    p = oracle.quantize_pack(codec(fmt), x)
    d = oracle.unpack_dequant(codec(fmt), p, x.size)
    assert np.array_equal(d, x)


def test_mxfp4_grid_round_trip():
    e = RNG.integers(-20, 20, 64)
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    idx = RNG.integers(0, 8, (64, 32))
    idx[:, 0] = 7
    sign = RNG.choice([-1.0, 1.0], (64, 32))
    x = (sign * table[idx] * 2.0 ** e[:, None]).astype(np.float32).ravel()
    p = oracle.quantize_pack(oracle.MXFP4, x)
    d = oracle.unpack_dequant(oracle.MXFP4, p, x.size)
    assert np.array_equal(np.abs(d), np.abs(x))


def test_int3_planes_are_split_nibbles():
    """The INT3 tile is the INT4-style sign/magnitude nibble of each element
    with its sign bit moved to q1w (bit i for element i) and its two magnitude
    bits to q2w: check the plane bit counts against the decoded codes."""
    x = special_tile(11)
    p = oracle.quantize_pack(oracle.INT3, x)
    d = oracle.unpack_dequant(oracle.INT3, p, 2048)
    s = np.frombuffer(p[768:896].tobytes(), dtype=np.float16).astype(np.float64)
    mags = np.rint(np.abs(d.astype(np.float64)) / np.repeat(np.where(s > 0, s, 1), 32)).astype(np.int64)
    q1w = np.unpackbits(p[512:768], bitorder="little")
    assert np.array_equal(q1w.astype(bool), np.signbit(d) & np.repeat(s > 0, 32))
    q2w = np.unpackbits(p[:512], bitorder="little")
    assert q2w.sum() == sum(bin(int(m)).count("1") for m in mags)


@pytest.mark.parametrize("fmt", FMTS)
def test_bf16_and_fp16_inputs_widen_exactly(fmt):
    x = special_tile(5)
    x = x[np.abs(x) < 60000]
    h = x.astype(np.float16)
    b = oracle.f32_to_bf16_bits(x)
    assert np.array_equal(oracle.quantize_pack(codec(fmt), h),
                          oracle.quantize_pack(codec(fmt), h.astype(np.float32)))
    assert np.array_equal(oracle.quantize_pack(codec(fmt), b, dtype=oracle.DT_BF16),
                          oracle.quantize_pack(codec(fmt), oracle.bf16_bits_to_f32(b)))


@pytest.mark.parametrize("fmt", FMTS)
def test_unpack_to_narrow_dtypes(fmt):
    x = special_tile(9)
    p = oracle.quantize_pack(codec(fmt), x)
    d32 = oracle.unpack_dequant(codec(fmt), p, x.size, oracle.DT_FP32)
    d16 = oracle.unpack_dequant(codec(fmt), p, x.size, oracle.DT_FP16)
    db = oracle.unpack_dequant(codec(fmt), p, x.size, oracle.DT_BF16)
    with np.errstate(over="ignore"):
        assert np.array_equal(d16.view(np.uint16), d32.astype(np.float16).view(np.uint16))
    import torch
    ref = torch.from_numpy(d32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(db, ref)
