"""Proofs, on the CPU, of the binary32 sequences the gfx950 kernels use in
place of IEEE division (tests/device_arith.c restates each sequence with C's
fmaf and compares it with the exact rule it stands for):

* ``div``: a * RN(1/B) plus one residual correction equals the IEEE quotient
  a / B for every finite binary32 a and B = 3, 7, 448, 57344 (the INT and FP8
  block-scale divisions);
* ``recip``: the hardware reciprocal (either binary32 neighbour of 1/s) plus
  one Newton step is RN(1/s) for every positive finite fp16 scale s;
* ``int``: INT3 / INT4 codes from fma(x, r, x r_lo) and the RNE conversions
  equal round-half-even of the exact quotient x / s -- every fp16 scale with
  every bf16 x a block can hold, binary32 x within 16 ulp of every half step
  of every scale, random binary32 x -- while the single product x r differs
  there (control);
* ``fp8``: the encoder's two stages together equal the RNE E4M3 / E5M2 code
  of the exact quotient next to every rounding midpoint, at random
  magnitudes and far into saturation, for FP32 scales (also below 2^-64) and
  every fp16 scale.  The first stage converts x times the reciprocal rounded
  down and up by 2^-21 and keeps the code where both agree; the second, the
  round-to-odd quotient followed by the RNE conversion, decides the rest.
  Both stages must be exercised.
* ``fp8narrow``: for inputs of at most 11 significant bits (every bf16 and
  every fp16 pair x <= a, a the block maximum; FP32 and FP16 scales; both
  formats; both reciprocal neighbours) the bracket's undecided elements are
  exact ties, and the per-block rule gives the code of the exact quotient:
  the upper code when a - s fmax > 0 (FP32 scale rounded down), the lower
  when < 0, the even one when the quotient is the midpoint itself.  Every
  undecided pair is compared with the exact code, and a sample of the
  decided ones.

The scale rules are those of "QuickReduce INT3 Quantization and Benchmarking
on MI355" (Method: block FP16 scale) and "RCCLX: Innovating GPU
communications on AMD platforms" (Low-Precision Collectives: FP8 with FP32
computation).  Nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    exe = tmp_path_factory.mktemp("device_arith") / "device_arith"
    r = subprocess.run(["gcc", "-std=c11", "-O2", "-Wall", "-ffp-contract=off", "-fno-fast-math", "-pthread",
                        "-o", str(exe), os.path.join(HERE, "device_arith.c"), "-lm"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return str(exe)


@pytest.mark.slow
@pytest.mark.parametrize("check", ["recip", "div", "int", "fp8", "fp8narrow"])
def test_device_arithmetic_equals_exact_rule(checker, check):
    threads = str(min(16, os.cpu_count() or 4))
    r = subprocess.run([checker, check, threads], capture_output=True, text=True, timeout=900)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [ln for ln in r.stdout.splitlines() if "cases" in ln]
    assert lines and all(" differ 0" in ln for ln in lines if "must differ" not in ln)
    if check == "fp8narrow":
        res = [ln.split() for ln in r.stdout.splitlines() if ln.startswith("undecided pairs")]
        assert res and int(res[0][-1]) > 0
    if check == "fp8":
        stage = [ln.split() for ln in r.stdout.splitlines() if ln.startswith("bracket decided")]
        assert stage and int(stage[0][2].rstrip(",")) > 0 and int(stage[0][5]) > 0


def test_kernel_uses_the_proved_fp8_constants():
    """The FP8 encoder in the kernel sources uses the factors and the scale
    threshold that the fp8 / fp8narrow checks above prove: the reciprocal
    rounded down and up by 2^-21 (0x1.fffffp-1, 0x1.000008p0) and the exact
    sequence for scales below 2^-64, in the same binary32 spelling."""
    dev = open(os.path.join(HERE, "..", "reduction_codec_amd", "csrc", "rc_device.hpp")).read()
    proof = open(os.path.join(HERE, "device_arith.c")).read()
    for lit in ("0x1.fffffp-1f", "0x1.000008p0f", "0x1p-64f", "0x1p64f"):
        assert lit in dev, f"{lit} not in the kernel"
        assert lit in proof, f"{lit} not in the proof"
