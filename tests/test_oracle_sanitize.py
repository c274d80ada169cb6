"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds oracle/rcodec_oracle.c with the driver tests/oracle_sanitize.c (every
operation, every supported codec and dtype, ragged lengths, 1..3 streams, the
tile-range entry points, the MXFP4 GEMV, non-finite inputs and the error
paths) with gcc's sanitizers, and runs it: any out-of-bounds access, use of
freed memory, leak, out-of-range shift or float-to-int conversion fails the
test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    flags = ["-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all"]
    cmd = ["gcc", *flags, "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "rcodec_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle sanitizer run clean: 33 codecs" in r.stdout
