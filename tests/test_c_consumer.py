"""The C ABI from a C program: include/rcodec.h compiled as strict C99
(-pedantic -Werror) in tests/abi_consumer.c, linked against the built
librcodec.so, whose sizes, version, status strings and validation errors it
checks (calls that return before any HIP call, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "reduction_codec_amd")
LIB = os.path.join(LIBDIR, "librcodec.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_uses_the_abi(tmp_path):
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    exe = tmp_path / "abi_consumer"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_consumer.c"),
           "-o", str(exe), LIB, f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath-link,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks held" in r.stdout
