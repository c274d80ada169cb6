"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Packed codes and scales must be bit-exact; the FP32 sums of the reduce are
compared bit for bit as well (the stated tolerance, 1e-6 relative, is also
asserted so a failure reports how far off it is).  Oracle inputs always come
from the seeded generators or from the oracle itself, never from the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
import reduction_codec_amd as rca
from tests import brute, fp8_ties
from tests.arbitrary import CODE_BITS, E8M0_CODECS, SPECIAL_SCALES, e8m0_every_pair_stream

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FMTS = ["int4", "int3", "fp8", "mxfp4"]
DTYPES = ["bf16", "fp16", "fp32"]
TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
ORACLE_DT = {"bf16": oracle.DT_BF16, "fp16": oracle.DT_FP16, "fp32": oracle.DT_FP32}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dt: str) -> torch.Tensor:
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8)


def mixed(n: int, seed: int, dt: str) -> np.ndarray:
    """float32 values covering the cases that take the exact path: zero and
    negative-zero blocks, ties at half steps, grid values, tiny blocks with
    subnormal fp16 scales, saturating blocks, denormals -- then narrowed to
    dt (kept inside dt's finite range)."""
    r = np.random.default_rng(seed)
    v = r.standard_normal(n).astype(np.float32)
    blocks = max(1, n // 32)
    kinds = r.integers(0, 10, blocks)
    for b in range(blocks):
        sl = slice(32 * b, min(n, 32 * b + 32))
        m = sl.stop - sl.start
        k = kinds[b]
        if k == 0:
            v[sl] = 0.0
            v[sl.start] = -0.0
        elif k == 1:
            step = np.float32(2.0 ** r.integers(-6, 6))
            v[sl] = (r.integers(-7, 8, m) * step / 2).astype(np.float32)        # half-step ties
            v[sl.start] = 7 * step
            if m > 2:
                v[sl.start + 2] = -0.0                                           # -0 inside a live block
        elif k == 2:
            v[sl] *= np.float32(1e-5)
        elif k == 3:
            v[sl] *= np.float32(3e-8)
        elif k == 4:
            v[sl] *= np.float32(2e5)
        elif k == 5:
            v[sl] = (r.integers(-3, 4, m) * 0.25).astype(np.float32)
            v[sl.start] = 0.75
        elif k == 6:
            v[sl] *= np.float32(50)
    if dt == "fp16":
        v = np.clip(v, -60000, 60000).astype(np.float32)
    return datagen.narrow(v, dt)


def assert_same(got: np.ndarray, ref: np.ndarray, what: str):
    """Bitwise equality of two arrays of the same dtype; on failure report the
    first differing positions with both values."""
    g = np.ascontiguousarray(got)
    r = np.ascontiguousarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    bad = np.nonzero(g.view(np.uint8).reshape(g.size, -1).any(axis=1) if False else
                     (g.view(np.uint8).reshape(g.size, -1) != r.view(np.uint8).reshape(r.size, -1)).any(axis=1))[0]
    if bad.size:
        show = [(int(i), g[i], r[i]) for i in bad[:8]]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first (index, got, ref): {show}")


def oracle_pack(fmt, x, dt):
    return oracle.quantize_pack(oracle.CODECS[fmt], x, dtype=ORACLE_DT[dt])


# ------------------------------------------------------------ quantize ----

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("n", [1, 31, 32, 33, 2047, 2048, 2049, 5 * 2048 + 777])
def test_quantize_pack_bit_exact(fmt, dt, n):
    say(f"case quantize fmt={fmt} dt={dt} n={n}")
    x = mixed(n, seed=n * 7 + len(fmt), dt=dt)
    ref = oracle_pack(fmt, x, dt)
    pb = rca.packed_bytes(rca.CODECS[fmt], n)
    buf = torch.full((pb + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    rca.quantize_pack(to_dev(x, dt), rca.CODECS[fmt], out=buf[:pb])
    got = host_u8(buf)
    assert np.array_equal(got[:pb], ref)
    assert (got[pb:] == 0xA5).all(), "wrote past the packed size"


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_is_deterministic(fmt):
    x = mixed(40 * 2048 + 5, 3, "bf16")
    xt = to_dev(x, "bf16")
    a = rca.quantize_pack(xt, rca.CODECS[fmt]).clone()
    b = rca.quantize_pack(xt, rca.CODECS[fmt])
    assert torch.equal(a, b)


# -------------------------------------------------------------- unpack ----

# E4M3 magnitudes of codes 0..126 from the format's definition (bias 7,
# subnormals m * 2^-9), in increasing order
E4M3_VALUES = [float(np.ldexp(8 + (c & 7), (c >> 3) - 10)) if c >> 3 else float(np.ldexp(c & 7, -9))
               for c in range(127)]


def fp8_near_midpoints(blocks: int, seed: int, emin: int, emax: int) -> np.ndarray:
    """fp32 blocks whose FP8 scale RN32(a / 448) lies near [2^emin, 2^emax)
    and whose other elements sit within 2 ulp of the scale times an E4M3
    rounding midpoint, where the exact quotient decides the code."""
    r = np.random.default_rng(seed)
    v = np.zeros(32 * blocks, dtype=np.float32)
    for b in range(blocks):
        a = np.float32(np.ldexp(1.0 + r.random(), int(r.integers(emin, emax)))) * np.float32(448.0)
        s = np.float32(a) / np.float32(448.0)
        v[32 * b] = a if r.random() < 0.5 else -a
        for i in range(1, 32):
            c = int(r.integers(0, 126))
            x = np.float32((E4M3_VALUES[c] + E4M3_VALUES[c + 1]) / 2 * float(s))
            x = np.frombuffer((np.array([x]).view(np.int32) + np.int32(r.integers(-2, 3))).tobytes(),
                              dtype=np.float32)[0]
            v[32 * b + i] = -x if r.random() < 0.5 else x
    return v


@pytest.mark.parametrize("emin,emax", [(-126, -100), (-100, -64), (-64, -8), (-8, 40)])
def test_fp8_quotients_next_to_midpoints(emin, emax):
    """FP8 codes round the exact quotient x / s: inputs next to rounding
    midpoints, over block scales from the smallest normal up (tiny scales are
    where a residual of the quotient could underflow)."""
    say(f"case fp8 midpoints scales 2^{emin}..2^{emax}")
    x = fp8_near_midpoints(200, seed=emin + 1000, emin=emin, emax=emax)
    ref = oracle_pack("fp8", x, "fp32")
    got = host_u8(rca.quantize_pack(to_dev(x, "fp32"), rca.FP8))
    assert_same(got, ref, "fp8 codes")
    # the same blocks as two reduce streams (requantization of their sums)
    y = fp8_near_midpoints(200, seed=emin + 2000, emin=emin, emax=emax)
    streams = [ref, oracle_pack("fp8", y, "fp32")]
    n = x.size
    want, _ = oracle.dequant_reduce_requant(oracle.CODECS["fp8"], streams, n)
    out, _ = rca.dequant_reduce_requant([torch.from_numpy(t).to(DEV) for t in streams], rca.FP8, n)
    assert_same(host_u8(out), want, "fp8 reduce")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("odt", DTYPES)
def test_unpack_dequant_bit_exact(fmt, odt):
    n = 6 * 2048 + 99
    say(f"case unpack fmt={fmt} odt={odt} n={n}")
    x = mixed(n, 11, "fp32")
    packed = oracle_pack(fmt, x, "fp32")
    ref = oracle.unpack_dequant(oracle.CODECS[fmt], packed, n, ORACLE_DT[odt])
    esz = 4 if odt == "fp32" else 2
    buf = torch.full((n * esz + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    out = buf[:n * esz].view(TORCH_DT[odt])
    rca.unpack_dequant(torch.from_numpy(packed).to(DEV), rca.CODECS[fmt], n, TORCH_DT[odt], out=out)
    got = host_u8(buf)
    assert_same(got[:n * esz].view(np.asarray(ref).dtype), ref, f"unpack {fmt}->{odt}")
    assert (got[n * esz:] == 0x5A).all()


# -------------------------------------------------------------- reduce ----

def oracle_streams(fmt, n, k, seed):
    out = []
    for j in range(k):
        x = mixed(n, seed + 13 * j, "fp32") if j % 2 == 0 else \
            (np.random.default_rng(seed + j).standard_normal(n) * (j + 1)).astype(np.float32)
        out.append(oracle_pack(fmt, x, "fp32"))
    return out


def assert_sums(got: np.ndarray, ref: np.ndarray):
    same = got.view(np.uint32) == ref.view(np.uint32)
    both_nan = np.isnan(got) & np.isnan(ref)
    ok = same | both_nan
    if not ok.all():
        rel = np.abs(got.astype(np.float64) - ref) / np.maximum(np.abs(ref.astype(np.float64)), 1e-300)
        raise AssertionError(f"{(~ok).sum()} sums differ; max rel {np.nanmax(rel):.3g} (bound 1e-6)")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [1, 2, 3, 4, 8, 16])
def test_reduce_bit_exact(fmt, k):
    n = 3 * 2048 + 500
    say(f"case reduce fmt={fmt} k={k} n={n}")
    streams = oracle_streams(fmt, n, k, seed=100 * k)
    ref, ref_sum = oracle.dequant_reduce_requant(oracle.CODECS[fmt], streams, n, want_sum=True)
    dev_streams = [torch.from_numpy(s).to(DEV) for s in streams]
    pb = rca.packed_bytes(rca.CODECS[fmt], n)
    buf = torch.full((pb + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    out, sums = rca.dequant_reduce_requant(dev_streams, rca.CODECS[fmt], n, out=buf[:pb], sum_out=True)
    got = host_u8(buf)
    assert np.array_equal(got[:pb], ref)
    assert (got[pb:] == 0xA5).all()
    assert_sums(sums.cpu().numpy(), ref_sum)


@pytest.mark.parametrize("fmt", FMTS)
def test_reduce_ignores_tail_codes(fmt):
    n = 2048 + 40
    streams = oracle_streams(fmt, n, 2, seed=5)
    tb = oracle.tile_bytes(oracle.CODECS[fmt])
    rng = np.random.default_rng(0)
    junk = streams[0].copy()
    if fmt == "int3":
        junk[tb + 16:tb + 512] = rng.integers(0, 256, 496, dtype=np.uint8)
        junk[tb + 520:tb + 768] = rng.integers(0, 256, 248, dtype=np.uint8)
    elif fmt == "fp8":
        # groups 2.. of both code planes (elements 64.., all past n)
        junk[tb + 32:tb + 1024] = rng.integers(0, 127, 992, dtype=np.uint8)
        junk[tb + 1056:tb + 2048] = rng.integers(0, 127, 992, dtype=np.uint8)
    else:
        junk[tb + 32:tb + 1024] = rng.integers(0, 256, 992, dtype=np.uint8)
    ref, _ = oracle.dequant_reduce_requant(oracle.CODECS[fmt], [junk, streams[1]], n)
    out, _ = rca.dequant_reduce_requant([torch.from_numpy(junk).to(DEV), torch.from_numpy(streams[1]).to(DEV)],
                                        rca.CODECS[fmt], n)
    assert np.array_equal(host_u8(out), ref)


def test_zero_length_and_errors_on_gpu():
    x = torch.zeros(0, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(16, dtype=torch.uint8, device=DEV)
    assert rca.lib().rc_quantize_pack(rca.INT3, rca.DT_BF16, x.data_ptr(), 0, out.data_ptr(), None) == rca.OK
    with pytest.raises(rca.CodecError):
        rca.dequant_reduce_requant([out], rca.Codec(2, 2, 32), 0)


def test_binding_rejects_short_buffers_before_launching():
    """Buffers smaller than the call needs are refused by the binding with
    ValueError, before anything runs; the buffers keep their contents."""
    n = 2 * 2048 + 5
    x = torch.ones(n, dtype=torch.bfloat16, device=DEV)
    pb = rca.packed_bytes(rca.INT3, n)
    p = rca.quantize_pack(x, rca.INT3)
    short = torch.full((pb - 1,), 0x5A, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        rca.quantize_pack(x, rca.INT3, out=short)
    with pytest.raises(ValueError):
        rca.dequant_reduce_requant([p, p], rca.INT3, n, out=short)
    with pytest.raises(ValueError):
        rca.dequant_reduce_requant([p, short], rca.INT3, n)
    with pytest.raises(ValueError):
        rca.dequant_reduce_requant([p], rca.INT3, n, sum_out=torch.empty(n - 1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        rca.unpack_dequant(short, rca.INT3, n)
    with pytest.raises(ValueError):
        rca.unpack_dequant(p, rca.INT3, n, out=torch.empty(n - 1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        rca.allreduce_emulate([x, x[:-1]], rca.INT3)
    with pytest.raises(ValueError):
        rca.copy(short[:16], p[:32])
    torch.cuda.synchronize()
    assert bool((short == 0x5A).all())
    # a packed stream may be any dtype; its bytes are what count
    out, _ = rca.dequant_reduce_requant([p.view(torch.int32)[: pb // 4]], rca.INT3, n)
    assert torch.equal(out, rca.dequant_reduce_requant([p], rca.INT3, n)[0])


def test_binding_rejects_a_stream_of_another_device():
    class OtherDeviceStream:
        device = torch.device("cuda", 1)
        cuda_stream = 0
    x = torch.ones(2048, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        rca.quantize_pack(x, rca.INT3, stream=OtherDeviceStream())


# -------------------------------------------------------- configurations ----

def test_config_int4_fp16_64_tiles_roundtrip_and_k2():
    """64 tiles x 2048 fp16 ~ N(0,1) (seeds 0, 1): INT4 pack, 2-stream reduce, unpack."""
    xs = [datagen.fp16_normal_64x2048(s) for s in (0, 1)]
    n = xs[0].size
    refs = [oracle_pack("int4", x, "fp16") for x in xs]
    for x, ref in zip(xs, refs):
        got = host_u8(rca.quantize_pack(to_dev(x, "fp16"), rca.INT4))
        assert np.array_equal(got, ref)
        assert got.size == 64 * 1152
    ref, ref_sum = oracle.dequant_reduce_requant(oracle.INT4, refs, n, want_sum=True)
    out, sums = rca.dequant_reduce_requant([torch.from_numpy(r).to(DEV) for r in refs], rca.INT4, n,
                                           sum_out=True)
    assert np.array_equal(host_u8(out), ref)
    assert_sums(sums.cpu().numpy(), ref_sum)
    y = rca.unpack_dequant(out, rca.INT4, n, torch.float16)
    assert np.array_equal(y.cpu().numpy().view(np.uint16),
                          oracle.unpack_dequant(oracle.INT4, ref, n, oracle.DT_FP16).view(np.uint16))


def test_config_int3_bf16_activation_4mb():
    """256 x 8192 bf16 activation, N(0,1) with 0.1% outliers x20: INT3 pack,
    unpack, and a 4-stream reduce of the message and three tile-shifted copies."""
    x = datagen.bf16_act_256x8192_outl()
    n = x.size
    ref = oracle.quantize_pack_parallel(oracle.INT3, x, dtype=oracle.DT_BF16)
    got = host_u8(rca.quantize_pack(to_dev(x, "bf16"), rca.INT3))
    assert np.array_equal(got, ref) and got.size == 1024 * 896
    y = rca.unpack_dequant(torch.from_numpy(ref).to(DEV), rca.INT3, n, torch.bfloat16)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle.unpack_dequant(oracle.INT3, ref, n, oracle.DT_BF16))
    tb = 896
    streams = [np.roll(ref.reshape(-1, tb), j, axis=0).ravel().copy() for j in range(4)]
    rref, rsum = oracle.dequant_reduce_requant_parallel(oracle.INT3, streams, n, want_sum=True)
    out, sums = rca.dequant_reduce_requant([torch.from_numpy(s).to(DEV) for s in streams], rca.INT3, n,
                                           sum_out=True)
    assert np.array_equal(host_u8(out), rref)
    assert_sums(sums.cpu().numpy(), rsum)


def test_config_fp8_eight_fp32_streams_16mb():
    """8 fp32 streams of 4M elements ~ N(0, 0.5): FP8 pack each, K=8 reduce."""
    n = 4 * 1024 * 1024
    refs = []
    for k in range(8):
        say(f"case fp8 config stream {k}")
        x = datagen.fp32_normal_4m(k)
        ref = oracle.quantize_pack_parallel(oracle.FP8, x)
        got = host_u8(rca.quantize_pack(to_dev(x, "fp32"), rca.FP8))
        assert np.array_equal(got, ref)
        refs.append(ref)
    say("case fp8 config reduce k=8")
    rref, rsum = oracle.dequant_reduce_requant_parallel(oracle.FP8, refs, n, want_sum=True)
    out, sums = rca.dequant_reduce_requant([torch.from_numpy(r).to(DEV) for r in refs], rca.FP8, n,
                                           sum_out=True)
    assert np.array_equal(host_u8(out), rref)
    assert_sums(sums.cpu().numpy(), rsum)
    # 4:1 payload: code bytes are a quarter of the fp32 input bytes
    assert (n // 2048) * 2048 * 4 / ((n // 2048) * 2048) == 4


def test_config_mxfp4_bf16_weight_4096():
    """bf16 4096x4096 weight, 0.02 N(0,1) with U[0.5,2] row drift: MXFP4 pack and unpack."""
    x = datagen.bf16_weight_4096x4096()
    n = x.size
    ref = oracle.quantize_pack_parallel(oracle.MXFP4, x, dtype=oracle.DT_BF16)
    got = host_u8(rca.quantize_pack(to_dev(x, "bf16"), rca.MXFP4))
    assert np.array_equal(got, ref) and got.size == 8192 * 1088
    y = rca.unpack_dequant(torch.from_numpy(ref).to(DEV), rca.MXFP4, n, torch.bfloat16)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle.unpack_dequant(oracle.MXFP4, ref, n, oracle.DT_BF16))


# ----------------------------------------- size sweep, sampled tiles ----

SWEEP_MIB = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]


def sample_tiles(tiles: int, rng) -> list:
    pick = {0, tiles - 1, tiles // 2}
    pick.update(int(t) for t in rng.integers(0, tiles, 40))
    return sorted(pick)


@pytest.mark.parametrize("mib", SWEEP_MIB)
@pytest.mark.parametrize("fmt", ["int4", "int3"])
def test_sweep_sampled_tiles(fmt, mib):
    """Student-t (nu=4) bf16 messages at full size in the launch shape the
    benchmark uses: quantize_pack of the message, a K=4 reduce of four
    tile-shifted messages and unpack_dequant of the reduced stream to bf16,
    checked on sampled tiles (first, middle, last and 40 random) the oracle
    computes."""
    n = mib * (1 << 20) // 2
    say(f"case sweep fmt={fmt} size={mib}MiB")
    base = datagen.bf16_student4(mib * (1 << 20) + 3 * 4096)        # n + 3 tiles
    streams_x = [base[j * 2048: j * 2048 + n] for j in range(4)]
    c, oc = rca.CODECS[fmt], oracle.CODECS[fmt]
    tb = oracle.tile_bytes(oc)
    tiles = -(-n // 2048)
    rng = np.random.default_rng(mib)
    picks = sample_tiles(tiles, rng)
    dev_packed = []
    ref_packed = []
    for j, xs in enumerate(streams_x):
        p = rca.quantize_pack(to_dev(xs, "bf16"), c)
        dev_packed.append(p)
        refp = np.zeros(oracle.packed_bytes(oc, n), dtype=np.uint8)
        for t in picks:
            oracle.quantize_pack(oc, xs, dtype=oracle.DT_BF16, tiles=(t, t + 1), out=refp)
        hp = host_u8(p)
        for t in picks:
            assert np.array_equal(hp[t * tb:(t + 1) * tb], refp[t * tb:(t + 1) * tb]), f"stream {j} tile {t}"
        ref_packed.append(refp)
    out, _ = rca.dequant_reduce_requant(dev_packed, c, n)
    hout = host_u8(out)
    refo = np.zeros_like(ref_packed[0])
    for t in picks:
        oracle.dequant_reduce_requant(oc, ref_packed, n, tiles=(t, t + 1), out=refo)
        assert np.array_equal(hout[t * tb:(t + 1) * tb], refo[t * tb:(t + 1) * tb]), f"reduce tile {t}"
    del dev_packed
    say(f"case sweep fmt={fmt} size={mib}MiB unpack")
    y = rca.unpack_dequant(out, c, n, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    for t in picks:
        m = min(2048, n - t * 2048)
        ref_y = oracle.unpack_dequant(oc, refo[t * tb:(t + 1) * tb], m, oracle.DT_BF16)
        assert np.array_equal(y[t * 2048:t * 2048 + m], ref_y), f"unpack tile {t}"
    del out, y
    torch.cuda.empty_cache()


# ------------------------------------------------- format / scale variants ----

VARIANTS = sorted(rca.ALL_CODECS)


@pytest.mark.parametrize("name", VARIANTS)
@pytest.mark.parametrize("dt", DTYPES)
def test_variant_quantize_bit_exact(name, dt):
    n = 2 * 2048 + 777
    say(f"case variant quantize {name} dt={dt} n={n}")
    x = mixed(n, seed=len(name) * 31 + n, dt=dt)
    ref = oracle.quantize_pack(oracle.ALL_CODECS[name], x, dtype=ORACLE_DT[dt])
    c = rca.ALL_CODECS[name]
    pb = rca.packed_bytes(c, n)
    buf = torch.full((pb + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    rca.quantize_pack(to_dev(x, dt), c, out=buf[:pb])
    got = host_u8(buf)
    assert_same(got[:pb], ref, name)
    assert (got[pb:] == 0xA5).all(), "wrote past the packed size"


@pytest.mark.parametrize("name", VARIANTS)
@pytest.mark.parametrize("odt", DTYPES)
def test_variant_unpack_bit_exact(name, odt):
    n = 2048 + 1000
    say(f"case variant unpack {name} odt={odt}")
    x = mixed(n, seed=7 + len(name), dt="fp32")
    packed = oracle.quantize_pack(oracle.ALL_CODECS[name], x, dtype=oracle.DT_FP32)
    ref = oracle.unpack_dequant(oracle.ALL_CODECS[name], packed, n, ORACLE_DT[odt])
    got = rca.unpack_dequant(torch.from_numpy(packed).to(DEV), rca.ALL_CODECS[name], n, TORCH_DT[odt])
    g = got.cpu()
    g = g.view(torch.int16).numpy().view(np.uint16) if odt == "bf16" else g.numpy()
    assert_same(g, ref, name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", VARIANTS)
def test_unpack_around_65536_tiles(name):
    """unpack_dequant reads its packed tiles with another cache policy from
    65,536 tiles on (3- and 4-bit codecs into any dtype, FP8 into fp32):
    streams of 65,535 (ragged), 65,536 and 65,537 (ragged) tiles of every
    codec into every output dtype, checked on sampled tiles.  The packed stream is the oracle's: picked tiles hold the
    oracle's codes of mixed values, every other tile is zero bytes."""
    c, oc = rca.ALL_CODECS[name], oracle.ALL_CODECS[name]
    tb = oracle.tile_bytes(oc)
    pool = mixed(61 * 2048, seed=len(name) * 7 + 3, dt="fp32")
    rng = np.random.default_rng(len(name))
    for n in (65535 * 2048 - 1000, 65536 * 2048, 65536 * 2048 + 777):
        tiles = -(-n // 2048)
        say(f"case unpack around 65536 tiles {name} n={n} tiles={tiles}")
        picks = sample_tiles(tiles, rng)
        packed = np.zeros(oracle.packed_bytes(oc, n), dtype=np.uint8)
        ref_tiles = {}
        for t in picks:
            cnt = min(2048, n - t * 2048)
            src = pool[(t % 61) * 2048:(t % 61) * 2048 + cnt]
            ref_tiles[t] = (oracle.quantize_pack(oc, src, dtype=oracle.DT_FP32), cnt)
            packed[t * tb:(t + 1) * tb] = ref_tiles[t][0]
        dev_packed = torch.from_numpy(packed).to(DEV)
        for odt in DTYPES:
            y = rca.unpack_dequant(dev_packed, c, n, TORCH_DT[odt])
            assert y.numel() == n
            for t in picks:
                ref_p, cnt = ref_tiles[t]
                ref = oracle.unpack_dequant(oc, ref_p, cnt, ORACLE_DT[odt])
                g = y[t * 2048:t * 2048 + cnt].cpu()
                g = g.numpy() if odt == "fp32" else g.view(torch.int16).numpy().view(np.uint16)
                assert_same(g, ref, f"{name} n={n} odt={odt} tile {t}")
            del y
        del dev_packed
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", VARIANTS)
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 8])
def test_variant_reduce_bit_exact(name, k):
    n = 2 * 2048 + 300
    say(f"case variant reduce {name} k={k}")
    c_or = oracle.ALL_CODECS[name]
    streams = []
    for j in range(k):
        x = mixed(n, 50 * k + 13 * j, "fp32") if j % 2 == 0 else \
            (np.random.default_rng(j).standard_normal(n) * (j + 1)).astype(np.float32)
        streams.append(oracle.quantize_pack(c_or, x, dtype=oracle.DT_FP32))
    ref, ref_sum = oracle.dequant_reduce_requant(c_or, streams, n, want_sum=True)
    c = rca.ALL_CODECS[name]
    pb = rca.packed_bytes(c, n)
    buf = torch.full((pb + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    _, sums = rca.dequant_reduce_requant([torch.from_numpy(s).to(DEV) for s in streams], c, n,
                                         out=buf[:pb], sum_out=True)
    got = host_u8(buf)
    assert_same(got[:pb], ref, name)
    assert (got[pb:] == 0xA5).all()
    assert_sums(sums.cpu().numpy(), ref_sum)


def same_values(got: np.ndarray, ref: np.ndarray, what: str):
    """Equal as values: bit for bit, except that any NaN matches any NaN."""
    g, r = np.asarray(got, dtype=np.float32), np.asarray(ref, dtype=np.float32)
    ok = (g.view(np.uint32) == r.view(np.uint32)) | (np.isnan(g) & np.isnan(r))
    if not ok.all():
        bad = np.nonzero(~ok)[0]
        raise AssertionError(f"{what}: {bad.size} differ; first (index, got, ref): "
                             f"{[(int(i), float(g[i]), float(r[i])) for i in bad[:6]]}")


@pytest.mark.parametrize("name", VARIANTS)
def test_decode_of_arbitrary_bytes(name):
    """Decoding is defined for every bit pattern of codes and scales (NaN,
    infinite, negative and subnormal scales, FP8 NaN / infinity codes, the
    E8M0 NaN byte and the E8M0 exponents whose products overflow binary32,
    planted in the first tile): packed streams of random bytes unpack to
    fp32, bf16 and fp16, and two of them reduce to the FP32 sums, as the
    oracle decodes them (a NaN matching any NaN).  The requantized codes of
    non-finite sums are unspecified and not compared."""
    n = 16 * 2048 + 100
    say(f"case decode of arbitrary bytes {name}")
    oc, c = oracle.ALL_CODECS[name], rca.ALL_CODECS[name]
    rng = np.random.default_rng(len(name) * 131)
    streams = [rng.integers(0, 256, oracle.packed_bytes(oc, n), dtype=np.uint8) for _ in range(2)]
    sp, at = SPECIAL_SCALES[oc[1]], brute.CODE_BYTES[oc[0]]
    streams[0][at:at + sp.size] = sp                  # the scale extremes in tile 0 of both streams,
    streams[1][at:at + sp.size] = sp.reshape(-1, brute.SCALE_SIZE[oc[1]])[::-1].reshape(-1)  # other pairings
    d0 = torch.from_numpy(streams[0]).to(DEV)
    same_values(rca.unpack_dequant(d0, c, n, torch.float32).cpu().numpy(),
                oracle.unpack_dequant(oc, streams[0], n, oracle.DT_FP32), f"{name} -> fp32")
    for odt, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        g = rca.unpack_dequant(d0, c, n, tdt).cpu().float().numpy()
        r = oracle.widen_to_f32(oracle.unpack_dequant(oc, streams[0], n, ORACLE_DT[odt]), ORACLE_DT[odt])
        same_values(g, r, f"{name} -> {odt}")
    _, want_sum = oracle.dequant_reduce_requant(oc, streams, n, want_sum=True)
    _, sums = rca.dequant_reduce_requant([torch.from_numpy(t).to(DEV) for t in streams], c, n, sum_out=True)
    same_values(sums.cpu().numpy(), want_sum, f"{name} sums")


@pytest.mark.parametrize("name", E8M0_CODECS)
def test_e8m0_every_code_with_every_scale_byte(name):
    """Every code pattern under every E8M0 scale byte, products beyond
    binary32 and the NaN byte included: unpack to fp32, bf16 and fp16 and the
    FP32 sums of two such streams (the codes paired differently) equal the
    oracle's (a NaN matching any NaN)."""
    oc, c = oracle.ALL_CODECS[name], rca.ALL_CODECS[name]
    a, n = e8m0_every_pair_stream(oc)
    b, _ = e8m0_every_pair_stream(oc, rot=(1 << CODE_BITS[oc[0]]) // 2 + 1)
    say(f"case e8m0 every pair {name} n={n}")
    da = torch.from_numpy(a).to(DEV)
    same_values(rca.unpack_dequant(da, c, n, torch.float32).cpu().numpy(),
                oracle.unpack_dequant(oc, a, n, oracle.DT_FP32), f"{name} -> fp32")
    for odt, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        g = rca.unpack_dequant(da, c, n, tdt).cpu().float().numpy()
        r = oracle.widen_to_f32(oracle.unpack_dequant(oc, a, n, ORACLE_DT[odt]), ORACLE_DT[odt])
        same_values(g, r, f"{name} -> {odt}")
    _, want = oracle.dequant_reduce_requant(oc, [a, b], n, want_sum=True)
    _, sums = rca.dequant_reduce_requant([da, torch.from_numpy(b).to(DEV)], c, n, sum_out=True)
    same_values(sums.cpu().numpy(), want, f"{name} sums")


FP8_SCALED = [n for n in VARIANTS if n.startswith(("e4m3_f", "e5m2_f"))]      # FP32 and FP16 scales


def fp8_tie_values(name: str, dt: str, n: int, seed: int, shift: int = 0) -> np.ndarray:
    """n values of dt (bf16 bit patterns, float16 or float32) in blocks with
    planted exact FP8 midpoint ties; fp32 messages hold bf16-valued ties.
    shift scales them by 2^shift (exact for bf16 and fp32 at -80)."""
    elem, scale, b = name.split("_")
    x, _ = fp8_ties.tie_message(elem, scale, "fp16" if dt == "fp16" else "bf16", int(b[1:]), n, seed)
    return datagen.narrow(np.ldexp(x, shift).astype(np.float32), dt)


@pytest.mark.parametrize("name", FP8_SCALED)
@pytest.mark.parametrize("dt", DTYPES)
def test_fp8_exact_midpoint_ties(name, dt):
    """Blocks whose quotients land exactly on FP8 rounding midpoints, on every
    side of the scale's rounding: bf16 / fp16 input takes the encoder's
    per-block tie rule, fp32 input (the same values) its exact fallback; then
    a 2-stream reduce of the packed stream with itself, whose sums are twice
    decoded values and so ties again."""
    n = 3 * 2048 + 320
    say(f"case fp8 ties {name} dt={dt} n={n}")
    xs = fp8_tie_values(name, dt, n, seed=len(name) * 101 + DTYPES.index(dt))
    oc, c = oracle.ALL_CODECS[name], rca.ALL_CODECS[name]
    ref = oracle.quantize_pack(oc, xs, dtype=ORACLE_DT[dt])
    assert_same(host_u8(rca.quantize_pack(to_dev(xs, dt), c)), ref, f"{name} codes")
    want, want_sum = oracle.dequant_reduce_requant(oc, [ref, ref], n, want_sum=True)
    dref = torch.from_numpy(ref).to(DEV)
    out, sums = rca.dequant_reduce_requant([dref, dref], c, n, sum_out=True)
    assert_same(host_u8(out), want, f"{name} reduce of two equal streams")
    assert_sums(sums.cpu().numpy(), want_sum)


@pytest.mark.parametrize("name", [n for n in FP8_SCALED if "_f32_" in n])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_fp8_ties_with_scales_below_2_pow_64(name, dt):
    """The tie messages times 2^-80: block scales from about 2^-108 up, many
    below 2^-64, where a wave holding such a lane encodes every code with the
    exact round-to-odd sequence (x and s times 2^64 in those lanes)."""
    n = 2 * 2048 + 320
    say(f"case fp8 ties tiny scales {name} dt={dt}")
    xs = fp8_tie_values(name, dt, n, seed=len(name) * 7 + 5, shift=-80)
    oc, c = oracle.ALL_CODECS[name], rca.ALL_CODECS[name]
    ref = oracle.quantize_pack(oc, xs, dtype=ORACLE_DT[dt])
    assert_same(host_u8(rca.quantize_pack(to_dev(xs, dt), c)), ref, f"{name} codes")
    want, want_sum = oracle.dequant_reduce_requant(oc, [ref, ref], n, want_sum=True)
    dref = torch.from_numpy(ref).to(DEV)
    out, sums = rca.dequant_reduce_requant([dref, dref], c, n, sum_out=True)
    assert_same(host_u8(out), want, f"{name} reduce of two equal streams")
    assert_sums(sums.cpu().numpy(), want_sum)


@pytest.mark.parametrize("name", [n for n in VARIANTS if n.startswith(("int4_e8m0", "int3_e8m0"))])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_int_e8m0_reduce_huge_block_exponents(name, k):
    """E8M0 scales near the top of the exponent range (blocks of ~1e37, shared
    exponent above 118) in the first tile only: the wave that holds them and
    the waves that do not take different decode and encode paths; both must
    match the oracle.  Sums stay finite."""
    n = 3 * 2048 + 500
    say(f"case e8m0 huge exponents {name} k={k}")
    c_or = oracle.ALL_CODECS[name]
    streams = []
    for j in range(k):
        r = np.random.default_rng(900 + 7 * j + k)
        x = r.standard_normal(n).astype(np.float32)
        for b in (0, 5, 6, 40, 63):                  # blocks of the first tile
            x[32 * b:32 * b + 32] *= np.float32(1e37 / (k + 1))
        x[32 * 7:32 * 7 + 32] *= np.float32(3e-39)   # and a denormal block beside them
        streams.append(oracle.quantize_pack(c_or, x, dtype=oracle.DT_FP32))
    ref, ref_sum = oracle.dequant_reduce_requant(c_or, streams, n, want_sum=True)
    assert np.isfinite(ref_sum).all()
    c = rca.ALL_CODECS[name]
    out, sums = rca.dequant_reduce_requant([torch.from_numpy(s).to(DEV) for s in streams], c, n, sum_out=True)
    assert_same(host_u8(out), ref, name)
    assert_sums(sums.cpu().numpy(), ref_sum)


# ------------------------------------------------ fused all-reduce emulation ----

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("two_shot", [True, False])
@pytest.mark.parametrize("k", [1, 2, 4, 5])
def test_allreduce_emulate_bit_exact(fmt, dt, two_shot, k):
    n = 2 * 2048 + 900
    say(f"case allreduce fmt={fmt} dt={dt} two_shot={two_shot} k={k}")
    msgs = [mixed(n, seed=300 * k + 17 * j + len(fmt), dt=dt) for j in range(k)]
    ref, ref_packed = oracle.allreduce_emulate(oracle.CODECS[fmt], msgs, ORACLE_DT[dt], two_shot=two_shot)
    out, packed = rca.allreduce_emulate([to_dev(m, dt) for m in msgs], rca.CODECS[fmt], two_shot=two_shot,
                                        packed_out=two_shot)
    g = out.cpu()
    g = g.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else g.numpy()
    assert_same(g, ref, f"allreduce {fmt} {dt}")
    if two_shot:
        assert_same(host_u8(packed), ref_packed, "packed sum")


@pytest.mark.parametrize("name", VARIANTS)
@pytest.mark.parametrize("two_shot", [True, False])
def test_allreduce_emulate_variants_bit_exact(name, two_shot):
    """The fused emulation for every codec (the message dtype and the
    message count vary with the codec): output and requantized sum equal the
    oracle's composition of quantize, reduce and unpack."""
    i = VARIANTS.index(name)
    dt, k = sorted(DTYPES)[i % 3], 2 + i % 3
    n = 2 * 2048 + 700
    say(f"case allreduce variant {name} dt={dt} two_shot={two_shot} k={k}")
    msgs = [mixed(n, seed=700 + 13 * i + j, dt=dt) for j in range(k)]
    ref, ref_packed = oracle.allreduce_emulate(oracle.ALL_CODECS[name], msgs, ORACLE_DT[dt], two_shot=two_shot)
    out, packed = rca.allreduce_emulate([to_dev(m, dt) for m in msgs], rca.ALL_CODECS[name], two_shot=two_shot,
                                        packed_out=two_shot)
    g = out.cpu()
    g = g.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else g.numpy()
    assert_same(g, ref, f"allreduce {name} {dt}")
    if two_shot:
        assert_same(host_u8(packed), ref_packed, "packed sum")


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("two_shot", [True, False])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_allreduce_emulate_fp8_ties(dt, two_shot, k):
    """The fused kernel's FP8 encodes on messages with planted exact midpoint
    ties (per-rank encodes of bf16 / fp16 take the per-block tie rule); the
    second message repeats the first, so the sums hold ties as well."""
    n = 2 * 2048 + 640
    say(f"case allreduce fp8 ties dt={dt} two_shot={two_shot} k={k}")
    msgs = [fp8_tie_values("e4m3_f32_b32", dt, n, seed=900 + j) for j in range(k)]
    if k >= 2:
        msgs[1] = msgs[0].copy()
    ref, ref_packed = oracle.allreduce_emulate(oracle.CODECS["fp8"], msgs, ORACLE_DT[dt], two_shot=two_shot)
    out, packed = rca.allreduce_emulate([to_dev(m, dt) for m in msgs], rca.FP8, two_shot=two_shot,
                                        packed_out=two_shot)
    g = out.cpu()
    g = g.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else g.numpy()
    assert_same(g, ref, f"allreduce fp8 ties {dt}")
    if two_shot:
        assert_same(host_u8(packed), ref_packed, "packed sum")


# ------------------------------------------------------------ MXFP4 GEMV ----

def gemv_bound(y: np.ndarray, exact: np.ndarray, mag: np.ndarray, cols: int, what: str):
    """|y - W x| <= (38 + T) 2^-24 sum |W_ij x_j| (T = cols / 2048), the
    tolerance of rc_mxfp4_gemv: every term passes through at most 38 + T
    binary32 roundings on its way to y, whatever the summation order.  A tiny
    absolute term covers block terms that underflow below 2^-126."""
    T = cols // 2048
    err = np.abs(y.astype(np.float64) - exact)
    tol = (38 + T) * 2.0 ** -24 * mag + 64 * 2.0 ** -149
    bad = np.nonzero(~(err <= tol))[0]
    if bad.size:
        show = [(int(i), float(y[i]), float(exact[i]), float(err[i] / max(mag[i], 1e-300))) for i in bad[:6]]
        raise AssertionError(f"{what}: {bad.size} rows beyond the bound; (row, y, exact, err/sum|Wx|): {show}")


@pytest.mark.parametrize("rows,cols", [(1, 2048), (7, 2048), (9, 4096), (33, 6144), (5, 10240), (300, 8192)])
@pytest.mark.parametrize("xt", DTYPES)
def test_mxfp4_gemv_within_bound_of_exact_dot_product(rows, cols, xt):
    """y (fp32) against the exact dot product of the decoded weights and x
    (the oracle's definition), within the stated bound; bf16 and fp16 y are
    the fp32 result rounded to nearest even."""
    say(f"case gemv rows={rows} cols={cols} x={xt}")
    r = np.random.default_rng(rows * 131 + cols)
    w = mixed(rows * cols, seed=rows + cols, dt="fp32")
    p = oracle.quantize_pack(oracle.MXFP4, w, dtype=oracle.DT_FP32)
    x = datagen.narrow((r.standard_normal(cols) * np.exp(r.uniform(-3, 3, cols))).astype(np.float32), xt)
    exact, mag = oracle.mxfp4_gemv(p, rows, cols, x, x_dtype=ORACLE_DT[xt])
    pd, xd = torch.from_numpy(p).to(DEV), to_dev(x, xt)
    y32 = rca.mxfp4_gemv(pd, rows, cols, xd, out_dtype=torch.float32).cpu().numpy()
    gemv_bound(y32, exact, mag, cols, f"gemv rows={rows} cols={cols} x={xt}")
    yb = rca.mxfp4_gemv(pd, rows, cols, xd, out_dtype=torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    assert_same(yb, oracle.f32_to_bf16_bits(y32), "gemv bf16 y = RN(fp32 y)")
    yh = rca.mxfp4_gemv(pd, rows, cols, xd, out_dtype=torch.float16).cpu().numpy().view(np.uint16)
    with np.errstate(over="ignore"):
        assert_same(yh, oracle.f32_to_f16_bits(y32), "gemv fp16 y = RN(fp32 y)")


def test_mxfp4_gemv_weight_4096x4096_all_rows_within_bound():
    """The 4096 x 4096 bf16 weight recipe packed on the GPU, bf16 x: every
    row against the exact dot product, within the bound."""
    rows = cols = 4096
    wbits = datagen.bf16_weight_4096x4096()
    p = rca.quantize_pack(to_dev(wbits, "bf16"), rca.MXFP4)
    assert np.array_equal(host_u8(p), oracle.quantize_pack_parallel(oracle.MXFP4, wbits, dtype=oracle.DT_BF16))
    x = datagen.narrow(np.random.default_rng(5).standard_normal(cols).astype(np.float32), "bf16")
    y = rca.mxfp4_gemv(p, rows, cols, to_dev(x, "bf16")).cpu().numpy()
    exact, mag = oracle.mxfp4_gemv(host_u8(p), rows, cols, x, x_dtype=oracle.DT_BF16)
    gemv_bound(y, exact, mag, cols, "gemv 4096x4096 recipe")


@pytest.mark.parametrize("case", ["x_bf16_subnormal", "x_bf16_mixed_magnitudes", "w_tiny_blocks"])
@pytest.mark.parametrize("xt", DTYPES)
def test_mxfp4_gemv_edge_magnitudes_within_bound(case, xt):
    """Inputs at the edges of the number range, every x dtype: x made of
    subnormal values (bf16 / fp16 / fp32 subnormals), x spanning 2^-60..2^60
    with zeros and -0, and weight blocks whose E8M0 exponent is near -127; y
    within the bound of the exact dot product."""
    rows, cols = 40, 4096
    say(f"case gemv edge {case} x={xt}")
    r = np.random.default_rng(hash(case) % 1000)
    w = r.standard_normal(rows * cols).astype(np.float32)
    if case == "w_tiny_blocks":
        w[: rows * cols // 2] *= np.float32(2.0 ** -120)
    p = oracle.quantize_pack(oracle.MXFP4, w)
    if case == "x_bf16_subnormal":
        tiny = {"bf16": 2.0 ** -130, "fp16": 2.0 ** -20, "fp32": 2.0 ** -140}[xt]
        x = (r.standard_normal(cols) * tiny).astype(np.float32)
    elif case == "x_bf16_mixed_magnitudes":
        x = (r.standard_normal(cols) * 2.0 ** r.integers(-60, 60, cols)).astype(np.float32)
        if xt == "fp16":
            x = (r.standard_normal(cols) * 2.0 ** r.integers(-20, 12, cols)).astype(np.float32)
        x[::7] = 0.0
        x[3::7] = -0.0
    else:
        x = (r.standard_normal(cols)).astype(np.float32)
    x = datagen.narrow(x, xt)
    exact, mag = oracle.mxfp4_gemv(p, rows, cols, x, x_dtype=ORACLE_DT[xt])
    y = rca.mxfp4_gemv(torch.from_numpy(p).to(DEV), rows, cols, to_dev(x, xt)).cpu().numpy()
    gemv_bound(y, exact, mag, cols, f"gemv edge {case} x={xt}")


@pytest.mark.parametrize("cols", [2048, 6144])
def test_mxfp4_gemv_exact_sums_and_one_hot(cols):
    """Order-free exact cases: dyadic weights (block maximum 6, so every E8M0
    exponent is 0) with integer x make every partial sum exact, so y equals
    the exact sum bit for bit; a one-hot x returns the decoded weight column."""
    rows = 70
    r = np.random.default_rng(cols)
    idx = r.integers(0, 8, rows * cols)
    w = (np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[idx] * r.choice([-1, 1], rows * cols)).astype(np.float32)
    w[::32] = 6.0
    p = oracle.quantize_pack(oracle.MXFP4, w)
    pd = torch.from_numpy(p).to(DEV)
    x = r.integers(-50, 51, cols).astype(np.float32)
    y = rca.mxfp4_gemv(pd, rows, cols, to_dev(x, "fp32")).cpu().numpy()
    exact, _ = oracle.mxfp4_gemv(p, rows, cols, x)
    assert np.array_equal(y.astype(np.float64), exact)
    wd = oracle.unpack_dequant(oracle.MXFP4, p, rows * cols).reshape(rows, cols)
    for j in (0, 33, cols - 1):
        e = np.zeros(cols, dtype=np.float32)
        e[j] = 1.0
        yj = rca.mxfp4_gemv(pd, rows, cols, to_dev(e, "fp32")).cpu().numpy()
        assert np.array_equal(yj, wd[:, j])


# ---------------------------------------------------------- beyond 4 GiB ----

def _big_message(n: int, seed: int) -> np.ndarray:
    """n bf16 values: one seeded Student-t chunk repeated, each repetition
    with different low mantissa bits, so no two regions of the message are
    alike (an access that lands in the wrong 4 GiB window shows)."""
    chunk = datagen.bf16_student4(1 << 24, seed)                       # 8M values
    x = np.empty(n, dtype=np.uint16)
    for r, i in enumerate(range(0, n, chunk.size)):
        m = min(chunk.size, n - i)
        np.bitwise_xor(chunk[:m], np.uint16(1 + r % 127), out=x[i:i + m])
    return x


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["int3", "fp8"])
def test_message_beyond_4gib(fmt):
    """A bf16 message of 2^31 + 3 tiles + 777 elements (4 GiB + of input and of
    unpacked output; 2.4 GB of FP8 codes): quantize, a 2-stream reduce and
    unpack, checked against the oracle on tiles around the 2^30 and 2^31
    element (2 GiB and 4 GiB byte) boundaries, random tiles and the ragged
    last tile."""
    n = (1 << 31) + 3 * 2048 + 777
    say(f"case beyond 4 GiB fmt={fmt} n={n}")
    c, oc = rca.CODECS[fmt], oracle.CODECS[fmt]
    tb = oracle.tile_bytes(oc)
    tiles = -(-n // 2048)
    xa, xb = _big_message(n, 31), _big_message(n, 32)
    pa = rca.quantize_pack(torch.from_numpy(xa.view(np.int16)).view(torch.bfloat16).to(DEV), c)
    xbd = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    pb_ = rca.quantize_pack(xbd, c)
    del xbd
    out, _ = rca.dequant_reduce_requant([pa, pb_], c, n)
    y = rca.unpack_dequant(out, c, n, torch.bfloat16)
    torch.cuda.synchronize()
    t2g, t4g = (1 << 30) // 2048, (1 << 31) // 2048
    picks = {0, t2g - 1, t2g, t4g - 1, t4g, t4g + 1, tiles - 1}
    picks.update(int(t) for t in np.random.default_rng(5).integers(0, tiles, 12))
    for t in sorted(picks):
        lo, cnt = t * 2048, min(2048, n - t * 2048)
        ra = oracle.quantize_pack(oc, xa[lo:lo + cnt], dtype=oracle.DT_BF16)
        rb = oracle.quantize_pack(oc, xb[lo:lo + cnt], dtype=oracle.DT_BF16)
        assert np.array_equal(host_u8(pa[t * tb:(t + 1) * tb]), ra), f"quantize tile {t}"
        assert np.array_equal(host_u8(pb_[t * tb:(t + 1) * tb]), rb), f"quantize tile {t} (stream b)"
        ro, _ = oracle.dequant_reduce_requant(oc, [ra, rb], cnt)
        assert np.array_equal(host_u8(out[t * tb:(t + 1) * tb]), ro), f"reduce tile {t}"
        ry = oracle.unpack_dequant(oc, ro, cnt, oracle.DT_BF16)
        got = y[lo:lo + cnt].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ry), f"unpack tile {t}"
    del pa, pb_, out, y
    torch.cuda.empty_cache()
