"""Exhaustive GPU check of the exact-quotient encoders on narrow inputs.

For every positive finite bf16 (or fp16) value a, blocks of 32 elements hold
a followed by every bf16 (fp16) value x in [0, a] (negated at odd positions),
31 per block, padded with zeros: every pair (x, block maximum a) the format
allows.  The GPU's E4M3 / E5M2 codes with FP32 and FP16 block scales must
equal the oracle's byte for byte -- the exact-quotient rounding of "FP8
Formats for Deep Learning" (abstract) under the block scales of "RCCLX:
Innovating GPU communications on AMD platforms" (Low-Precision Collectives)
-- and so must the INT3 / INT4 codes with FP16 block scales (round half to
even of the exact quotient, "QuickReduce INT3 Quantization and Benchmarking
on MI355", Method), and every element format under E8M0 block scales
("Microscaling Data Formats for Deep Learning", abstract: the nearest code
of the value times a power of two).  The bf16 pairs also run as fp32 input, which takes the
FP8 encoder's exact fallback wherever a quotient sits on a rounding
midpoint.  This checks on the hardware what tests/device_arith.c checks by
emulation.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import reduction_codec_amd as rca

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOP = {"bf16": 0x7F7F, "fp16": 0x7BFF}           # largest finite positive bit pattern
CHUNK_BLOCKS = 1 << 20                             # 32 Mi elements per launch
# every block maximum (all 33 cases: about 90 s on an MI355X machine);
# RC_FP8_PAIR_STEP=17 takes every 17th, with every x below it, for a quick run
A_STEP = int(os.environ.get("RC_FP8_PAIR_STEP", "1"))


def pair_blocks(dt: str):
    """Chunks of blocks (uint16 bit patterns, 32 per block): [a, x, x, ...]
    for every A_STEP-th a in 1..TOP[dt] and every x in 0..a."""
    a = np.arange(1, TOP[dt] + 1, A_STEP, dtype=np.int64)
    counts = (a + 31) // 31                        # blocks of a: x = 0 .. a, 31 per block
    cum = np.cumsum(counts)
    start = 0
    while start < a.size:
        base = cum[start - 1] if start else 0
        end = max(int(np.searchsorted(cum, base + CHUNK_BLOCKS, side="right")), start + 1)
        aa, cc = a[start:end], counts[start:end]
        ba = np.repeat(aa, cc)
        bc = np.arange(ba.size) - np.repeat(np.cumsum(cc) - cc, cc)
        x = bc[:, None] * 31 + np.arange(31)[None, :]
        x = np.where(x <= ba[:, None], x, 0).astype(np.uint16)
        x[:, 1::2] |= np.uint16(0x8000)
        yield np.concatenate([ba[:, None].astype(np.uint16), x], axis=1).reshape(-1)
        start = end


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["e4m3_f32_b32", "e4m3_f16_b32", "e5m2_f32_b32", "e5m2_f16_b32",
                                  "int3_f16_b32", "int4_f16_b32", "e4m3_e8m0_b32", "e5m2_e8m0_b32",
                                  "int3_e8m0_b32", "int4_e8m0_b32", "e2m1_e8m0_b32"])
@pytest.mark.parametrize("src,dt", [("bf16", "bf16"), ("fp16", "fp16"), ("bf16", "fp32")])
def test_every_narrow_pair(name, src, dt):
    c, oc = rca.ALL_CODECS[name], oracle.ALL_CODECS[name]
    for i, bits in enumerate(pair_blocks(src)):
        print(f"case every pair {name} {src} values as {dt}, chunk {i} ({bits.size} elements)", flush=True)
        if dt == "fp32":
            host = oracle.widen_to_f32(bits, oracle.DT_BF16)
            odt = oracle.DT_FP32
            dev = torch.from_numpy(host).to(DEV)
        else:
            host = bits if dt == "bf16" else bits.view(np.float16)
            odt = oracle.DT_BF16 if dt == "bf16" else oracle.DT_FP16
            dev = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16 if dt == "bf16" else torch.float16)
        ref = oracle.quantize_pack_parallel(oc, host, dtype=odt)
        got = rca.quantize_pack(dev, c).cpu().numpy()
        if not np.array_equal(got, ref):
            bad = np.nonzero(got != ref)[0]
            raise AssertionError(f"{name} {src}->{dt} chunk {i}: {bad.size} bytes differ, first at {bad[:8]}")
        del dev
