"""Property-based parity fuzzing of the HIP path against the CPU oracle.

Hypothesis draws the codec (any of the 33), the input dtype, the length
(ragged tails included), the stream count and a per-block mix of value kinds
(zero and negative-zero blocks, half-step ties on a grid, blocks whose scale
is an fp16 subnormal or flushes to zero, fp32 denormals, saturating and huge
blocks, outliers); every example quantizes K streams, reduces them with the
FP32 sums and unpacks the result, each step compared byte for byte with the
oracle.  Further tests fuzz the fused all-reduce emulation, the decode of
streams of random bytes and the MXFP4 GEMV.  By default the 120-example
sequence is derandomized, so a run is reproducible; RC_FUZZ_EXAMPLES=N runs N
examples with fresh random draws (N/2 for the emulation, N/3 for the others).
"""
import os

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import datagen
import oracle
import reduction_codec_amd as rca

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DTYPES = {"bf16": (torch.bfloat16, oracle.DT_BF16), "fp16": (torch.float16, oracle.DT_FP16),
          "fp32": (torch.float32, oracle.DT_FP32)}
CODECS = sorted(rca.ALL_CODECS)
EXAMPLES = int(os.environ.get("RC_FUZZ_EXAMPLES", "120"))


def make_values(rng: np.random.Generator, n: int, kinds, k: int, dt: str) -> np.ndarray:
    v = rng.standard_normal(n).astype(np.float32)
    for b in range((n + 31) // 32):
        sl = slice(32 * b, min(n, 32 * b + 32))
        m = sl.stop - sl.start
        kind = kinds[b % len(kinds)]
        if kind == 0:
            v[sl] = 0.0
            v[sl.start] = -0.0
        elif kind == 1:
            step = np.float32(2.0 ** rng.integers(-8, 8))
            v[sl] = (rng.integers(-15, 16, m) * step / 2).astype(np.float32)     # half-step ties
        elif kind == 2:
            v[sl] *= np.float32(1e-5)                                           # fp16-subnormal scales
        elif kind == 3:
            v[sl] *= np.float32(3e-8)                                           # scales that flush
        elif kind == 4:
            v[sl] = (rng.uniform(-1, 1, m) * 1e-39).astype(np.float32)          # fp32 denormals
        elif kind == 5:
            v[sl] *= np.float32(2e5)                                            # saturating fp16 scales
        elif kind == 6:
            v[sl] *= np.float32(1e36 / (k + 1))                                 # E8M0 exponents near the top
        elif kind == 7:
            v[sl.start + int(rng.integers(0, m))] *= np.float32(50)             # one outlier
        # kinds 8, 9: plain normal values
    if dt == "fp16":
        v = np.clip(v, -60000, 60000).astype(np.float32)
    return datagen.narrow(v, dt)


def to_dev(x: np.ndarray, dt: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16) if dt != "fp32" else np.ascontiguousarray(x))
    return (t.view(DTYPES[dt][0]) if dt != "fp32" else t).to(DEV)


@settings(max_examples=EXAMPLES, deadline=None, derandomize=EXAMPLES == 120, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(name=st.sampled_from(CODECS), dt=st.sampled_from(sorted(DTYPES)),
       n=st.integers(min_value=1, max_value=3 * 2048 + 200), k=st.integers(min_value=1, max_value=6),
       seed=st.integers(min_value=0, max_value=2**31 - 1),
       kinds=st.lists(st.integers(min_value=0, max_value=9), min_size=1, max_size=9))
def test_fuzz_quantize_reduce_unpack(name, dt, n, k, seed, kinds):
    print(f"case fuzz {name} dt={dt} n={n} k={k} seed={seed} kinds={kinds}", flush=True)
    rng = np.random.default_rng(seed)
    c_or, c = oracle.ALL_CODECS[name], rca.ALL_CODECS[name]
    xs = [make_values(rng, n, kinds[j % len(kinds):] + kinds[:j % len(kinds)], k, dt) for j in range(k)]
    ref_packed = [oracle.quantize_pack(c_or, x, dtype=DTYPES[dt][1]) for x in xs]
    got_packed = [rca.quantize_pack(to_dev(x, dt), c) for x in xs]
    for j in range(k):
        assert np.array_equal(got_packed[j].cpu().numpy(), ref_packed[j]), f"quantize stream {j}"
    ref_out, ref_sums = oracle.dequant_reduce_requant(c_or, ref_packed, n, want_sum=True)
    out, sums = rca.dequant_reduce_requant(got_packed, c, n, sum_out=True)
    assert np.array_equal(out.cpu().numpy(), ref_out), "reduce"
    s, r = sums.cpu().numpy(), ref_sums
    assert ((s.view(np.uint32) == r.view(np.uint32)) | (np.isnan(s) & np.isnan(r))).all(), "FP32 sums"
    ref_y = oracle.unpack_dequant(c_or, ref_out, n, oracle.DT_FP32)
    y = rca.unpack_dequant(out, c, n, torch.float32).cpu().numpy()
    assert ((y.view(np.uint32) == ref_y.view(np.uint32)) | (np.isnan(y) & np.isnan(ref_y))).all(), "unpack"


FUSED = CODECS


@settings(max_examples=max(1, EXAMPLES // 2), deadline=None, derandomize=EXAMPLES == 120, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(fmt=st.sampled_from(FUSED), dt=st.sampled_from(sorted(DTYPES)),
       n=st.integers(min_value=1, max_value=3 * 2048 + 200), k=st.integers(min_value=1, max_value=6),
       two_shot=st.booleans(), seed=st.integers(min_value=0, max_value=2**31 - 1),
       kinds=st.lists(st.integers(min_value=0, max_value=9), min_size=1, max_size=9))
def test_fuzz_allreduce_emulate(fmt, dt, n, k, two_shot, seed, kinds):
    """The one-kernel all-reduce emulation against the oracle's composition
    (quantize every message, reduce, then unpack the requantized sum or round
    the FP32 sums to the message dtype), on the same value mixes."""
    print(f"case fuzz allreduce {fmt} dt={dt} n={n} k={k} two_shot={two_shot} seed={seed} kinds={kinds}",
          flush=True)
    rng = np.random.default_rng(seed)
    xs = [make_values(rng, n, kinds[j % len(kinds):] + kinds[:j % len(kinds)], k, dt) for j in range(k)]
    ref, ref_packed = oracle.allreduce_emulate(oracle.ALL_CODECS[fmt], xs, DTYPES[dt][1], two_shot=two_shot)
    out, packed = rca.allreduce_emulate([to_dev(x, dt) for x in xs], rca.ALL_CODECS[fmt], two_shot=two_shot,
                                        packed_out=two_shot)
    g = out.cpu()
    g = g.numpy() if dt == "fp32" else g.view(torch.int16).numpy().view(np.uint16)
    r = np.asarray(ref)
    r = r if dt == "fp32" else r.view(np.uint16)
    if dt == "fp32":
        assert ((g.view(np.uint32) == r.view(np.uint32)) | (np.isnan(g) & np.isnan(r))).all(), "output"
    else:
        assert np.array_equal(g, r), "output"
    if two_shot:
        assert np.array_equal(packed.cpu().numpy(), ref_packed), "packed sum"


@settings(max_examples=max(1, EXAMPLES // 3), deadline=None, derandomize=EXAMPLES == 120, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(name=st.sampled_from(CODECS), n=st.integers(min_value=1, max_value=4 * 2048 + 200),
       k=st.integers(min_value=1, max_value=5), seed=st.integers(min_value=0, max_value=2**31 - 1))
def test_fuzz_decode_of_random_bytes(name, n, k, seed):
    """Packed streams of random bytes (any code, any scale bits): unpack to
    fp32 and the FP32 sums of k of them equal the oracle's, a NaN matching
    any NaN; the requantized codes of non-finite sums are unspecified."""
    print(f"case fuzz random bytes {name} n={n} k={k} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    c_or, c = oracle.ALL_CODECS[name], rca.ALL_CODECS[name]
    streams = [rng.integers(0, 256, oracle.packed_bytes(c_or, n), dtype=np.uint8) for _ in range(k)]
    dev = [torch.from_numpy(t).to(DEV) for t in streams]
    y, ref_y = rca.unpack_dequant(dev[0], c, n, torch.float32).cpu().numpy(), \
        oracle.unpack_dequant(c_or, streams[0], n, oracle.DT_FP32)
    assert ((y.view(np.uint32) == ref_y.view(np.uint32)) | (np.isnan(y) & np.isnan(ref_y))).all(), "unpack"
    _, ref_sums = oracle.dequant_reduce_requant(c_or, streams, n, want_sum=True)
    _, sums = rca.dequant_reduce_requant(dev, c, n, sum_out=True)
    s = sums.cpu().numpy()
    assert ((s.view(np.uint32) == ref_sums.view(np.uint32)) | (np.isnan(s) & np.isnan(ref_sums))).all(), "sums"


@settings(max_examples=max(1, EXAMPLES // 3), deadline=None, derandomize=EXAMPLES == 120, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(rows=st.integers(min_value=1, max_value=40), t=st.integers(min_value=1, max_value=5),
       xt=st.sampled_from(sorted(DTYPES)), yt=st.sampled_from(sorted(DTYPES)),
       seed=st.integers(min_value=0, max_value=2**31 - 1),
       wspread=st.integers(min_value=0, max_value=30), xspread=st.integers(min_value=0, max_value=30))
def test_fuzz_mxfp4_gemv(rows, t, xt, yt, seed, wspread, xspread):
    """y = W x from MXFP4-packed rows against the exact dot product of the
    decoded weights and x: |y - W x| <= (38 + T) 2^-24 sum |W_ij x_j| (plus
    a tiny absolute term), T = cols / 2048, for fp32 y; a bf16 / fp16 y must
    be that fp32 y rounded to nearest even.  Weights and x span 2^wspread and
    2^xspread in magnitude."""
    cols = 2048 * t
    print(f"case fuzz gemv rows={rows} cols={cols} x={xt} y={yt} seed={seed} w2^{wspread} x2^{xspread}",
          flush=True)
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(rows * cols) * np.exp2(rng.uniform(-wspread, 0, rows * cols))).astype(np.float32)
    x = (rng.standard_normal(cols) * np.exp2(rng.uniform(-xspread, 0, cols))).astype(np.float32)
    xn = datagen.narrow(x, xt)
    packed = oracle.quantize_pack(oracle.MXFP4, w, dtype=oracle.DT_FP32)
    exact, mag = oracle.mxfp4_gemv(packed, rows, cols, xn, x_dtype=DTYPES[xt][1])
    pd, xd = torch.from_numpy(packed).to(DEV), to_dev(xn, xt)
    y32 = rca.mxfp4_gemv(pd, rows, cols, xd, out_dtype=torch.float32).cpu().numpy()
    tol = (38 + t) * 2.0 ** -24 * mag + 64 * 2.0 ** -149
    err = np.abs(y32.astype(np.float64) - exact)
    assert (err <= tol).all(), float(np.max(err / np.maximum(tol, 1e-300)))
    if yt != "fp32":
        y = rca.mxfp4_gemv(pd, rows, cols, xd, out_dtype=DTYPES[yt][0]).cpu().view(torch.int16).numpy().view(np.uint16)
        with np.errstate(over="ignore"):
            want = oracle.f32_to_bf16_bits(y32) if yt == "bf16" else oracle.f32_to_f16_bits(y32)
        assert np.array_equal(y, want), f"{yt} y = RN(fp32 y)"
