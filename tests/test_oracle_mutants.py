"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case below plants one mistake in a copy of oracle/rcodec_oracle.c (a
single exact text replacement), compiles the copy with the oracle's own flags,
and runs the oracle pin suites against it in a subprocess (RC_ORACLE_LIB points
the oracle package at the broken build).  The suites must fail: a mistake they
let through would mean the oracle is pinned only to itself in that place.  The
mistakes are on the CPU only; nothing here touches the GPU or the HIP library.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
PIN_SUITES = ["tests/test_oracle_formats.py", "tests/test_oracle_quant.py",
              "tests/test_oracle_fp8_ties.py", "tests/test_oracle_reduce.py",
              "tests/test_oracle_variants.py", "tests/test_oracle_fuzz.py"]
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-tree-vectorize",
          "-fPIC", "-shared"]

# name -> (text in rcodec_oracle.c, replacement): each a slip a careful reader
# of the pages could still make.
MUTANTS = {
    "ties_away_from_zero_exact_path": ("(frac == 0.5 && m % 2 == 1)", "(frac == 0.5)"),
    "absmax_skips_first_element": ("if (m > a) a = m;", "if (m > a && e > 0) a = m;"),
    "fp16_subnormal_exponent": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "e4m3_max_416": ("float s = amax / 448.0f;", "float s = amax / 416.0f;"),
    "e2m1_subnormal_step": ("double v = (e == 0) ? 0.5 * m :", "double v = (e == 0) ? 1.0 * m :"),
    "reduce_drops_last_stream": ("for (int s = 1; s < k; ++s)\n                a = a +",
                                 "for (int s = 1; s < k - 1; ++s)\n                a = a +"),
    "reduce_subtracts": ("a = a + decode_elem(", "a = a - decode_elem("),
    "ties_away_from_zero_int_path": ("return (m % 2 == 0) ? m : m + 1;", "return m + 1;"),
    "int_truncates": ("const double mid = (m + 0.5) * sd;", "const double mid = (m + 1.0) * sd;"),
    "int_ties_down_by_reciprocal": ("if (x > mid) return m + 1;\n    if (x < mid) return m;",
                                    "if (x * (float)(1.0f / s) > m + 0.5) return m + 1;\n    if (x < mid) return m;"),
    "int_scale_over_qmax_plus_one": ("float s32 = amax / (float)qmax;",
                                     "float s32 = amax / (float)(qmax + 1);"),
    "minifloat_ties_round_down": ("return (c % 2 == 0) ? c : c + 1;", "return c;"),
    "e4m3_saturates_one_code_low": ("nearest_of_quotient(e4m3_mag, 127,", "nearest_of_quotient(e4m3_mag, 126,"),
    "mx_exponent_off_by_one": ("return rco_e8m0_exponent(amax, 2);", "return rco_e8m0_exponent(amax, 1);"),
    "fp8_single_plane_order": ("return e < 16 ? 16 * g + e : 1024 + 16 * g + (e - 16);", "return i;"),
    "int3_pair_order_swapped": ("4 * (p / 2) + 2 * (e % 2);", "4 * (p / 2) + 2 * (1 - e % 2);"),
    "minifloat_ties_away_from_zero": ("return (c % 2 == 0) ? c : c + 1;", "return c + 1;"),
    "e8m0_decode_saturates": ("return (float)ldexp(val, (int)sp[0] - 127);",
                              "return (float)fmax(-3.4028234663852886e38, "
                              "fmin(3.4028234663852886e38, ldexp(val, (int)sp[0] - 127)));"),
    "e8m0_nan_byte_read_as_exponent": ("if (sp[0] == 0xFF) return NAN;", "if (sp[0] == 0x100) return NAN;"),
    "fp16_scale_sign_dropped": ("return (float)(val * rco_f16_to_f32(get_u16(sp)));",
                                "return (float)(val * fabs(rco_f16_to_f32(get_u16(sp))));"),
    "fp8_quotient_rounded_to_binary32_first": (
        "(unsigned)mag_of(fabs((double)vb[e]), den));",
        "(unsigned)mag_of((double)(float)(fabs((double)vb[e]) / den), 1.0));"),
}


def _build(tmp_path, name):
    src = open(os.path.join(ORACLE, "rcodec_oracle.c")).read()
    if name != "unmutated":
        old, new = MUTANTS[name]
        assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
        src = src.replace(old, new)
    d = tmp_path / name
    d.mkdir()
    shutil.copy(os.path.join(ORACLE, "rcodec_oracle.h"), d / "rcodec_oracle.h")
    (d / "rcodec_oracle.c").write_text(src)
    lib = d / "librcodec_oracle.so"
    r = subprocess.run(["gcc", *CFLAGS, "-o", str(lib), str(d / "rcodec_oracle.c"), "-lm"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return lib


def _run_pins(lib):
    env = dict(os.environ, RC_ORACLE_LIB=str(lib), RC_FUZZ_EXAMPLES="40")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PIN_SUITES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout, (r.stdout + r.stderr)[-1500:]


@pytest.fixture(scope="module")
def mutant_runs(tmp_path_factory):
    """Every mutant built, and the pin suites run against each, several at a
    time (each run is its own process)."""
    tmp = tmp_path_factory.mktemp("mutants")
    libs = {name: _build(tmp, name) for name in sorted(MUTANTS)}
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        futs = {name: ex.submit(_run_pins, lib) for name, lib in libs.items()}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(mutant_runs, name):
    rc, out, tail = mutant_runs[name]
    assert rc == 1 and " failed" in out, f"mutant {name} survived the pins:\n{tail}"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_unmutated_copy_passes_and_is_the_one_loaded(tmp_path):
    """Control for the cases above: the same build of the unchanged source
    passes the format and quantizer pins, and RC_ORACLE_LIB is the library the
    oracle package then loads (so the failures above are the mutants' own)."""
    lib = _build(tmp_path, "unmutated")
    env = dict(os.environ, RC_ORACLE_LIB=str(lib))
    probe = "import oracle; oracle._load(); print(oracle._LIB_PATH)"
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == str(lib), r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PIN_SUITES[:2]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-1500:]
