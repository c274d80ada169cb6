"""Property-based pins of the oracle against the brute-force statement.

Hypothesis draws any of the 33 codecs, a length up to one tile plus a tail, and
a per-block mix of value kinds (zeros and negative zeros, half-step ties, tiny
blocks whose fp16 scale is subnormal or flushes, fp32 denormals, saturating
and huge blocks, outliers).  The oracle's packed bytes must equal
tests/brute.py's (exact rationals: argmin over every code), its decode must
equal brute force decode, and a 2-stream reduce must equal brute force.
Derandomized by default (the same 30 examples every run); RC_FUZZ_EXAMPLES=N
runs N examples with fresh random draws."""
import os

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from tests import brute

CODECS = sorted(oracle.ALL_CODECS)
EXAMPLES = int(os.environ.get("RC_FUZZ_EXAMPLES", "30"))


def values(rng: np.random.Generator, n: int, kinds) -> np.ndarray:
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
            v[sl] = (rng.integers(-15, 16, m) * step / 2).astype(np.float32)
        elif kind == 2:
            v[sl] *= np.float32(1e-5)
        elif kind == 3:
            v[sl] *= np.float32(3e-8)
        elif kind == 4:
            v[sl] = (rng.uniform(-1, 1, m) * 1e-39).astype(np.float32)
        elif kind == 5:
            v[sl] *= np.float32(2e5)
        elif kind == 6:
            v[sl] *= np.float32(1e36)
        elif kind == 7:
            v[sl.start + int(rng.integers(0, m))] *= np.float32(50)
    return v


@settings(max_examples=EXAMPLES, deadline=None, derandomize=EXAMPLES == 30, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(name=st.sampled_from(CODECS), n=st.integers(min_value=1, max_value=2048 + 300),
       seed=st.integers(min_value=0, max_value=2**31 - 1),
       kinds=st.lists(st.integers(min_value=0, max_value=9), min_size=1, max_size=9))
def test_fuzz_oracle_equals_brute_force(name, n, seed, kinds):
    c = oracle.ALL_CODECS[name]
    rng = np.random.default_rng(seed)
    x = values(rng, n, kinds)
    p = oracle.quantize_pack(c, x)
    assert p.tobytes() == brute.encode_codec(c, x)
    tb = oracle.tile_bytes(c)
    ours = oracle.unpack_dequant(c, p, n, oracle.DT_FP32)
    ref = np.concatenate([brute.decode_codec(c, p[t * tb:(t + 1) * tb].tobytes()) for t in range(len(p) // tb)])[:n]
    assert ((ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))).all()
    y = (values(rng, n, kinds[::-1]) * np.float32(0.5)).astype(np.float32)
    streams = [p, oracle.quantize_pack(c, y)]
    out, sums = oracle.dequant_reduce_requant(c, streams, n, want_sum=True)
    ref_out, ref_sums = brute.reduce_codec(c, streams, n)
    assert out.tobytes() == ref_out
    assert ((sums.view(np.uint32) == ref_sums.view(np.uint32)) | (np.isnan(sums) & np.isnan(ref_sums))).all()
