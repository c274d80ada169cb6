"""Host logic of bench.py that runs without a GPU: the one-GPU guard, the
counter summary (FETCH_SIZE / WRITE_SIZE scaled by the copy kernel's reading,
VALU count, source-hash guard) and the kernel-trace table."""
import csv
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_dir(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_pmc_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    copy_kib = bench.COPY_BYTES / 1024.0
    # FETCH_SIZE reads half the true bytes on the copy kernel, WRITE_SIZE all of them
    _counter_dir(tmp_path / "f", "FETCH_SIZE", [("rc::copy_kernel(...)", copy_kib / 2),
                                                ("void rc::reduce_kernel<2, 1, 32, 4>(...)", 1000.0),
                                                ("void rc::reduce_kernel<2, 1, 32, 4>(...)", 1002.0),
                                                ("void rc::quantize_kernel<2, 1, 32, 3>(...)", 500.0)])
    _counter_dir(tmp_path / "w", "WRITE_SIZE", [("rc::copy_kernel(...)", copy_kib),
                                                ("void rc::reduce_kernel<2, 1, 32, 4>(...)", 300.0),
                                                ("void rc::quantize_kernel<2, 1, 32, 3>(...)", 200.0)])
    _counter_dir(tmp_path / "s", "SQ_INSTS_VALU", [("void rc::reduce_kernel<2, 1, 32, 4>(...)", 5898240.0)])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "s"))
    t = json.loads(traffic.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    red = t["kernels"]["reduce_kernel"]
    assert red["fetch_kib"] == pytest.approx(1001.0)                     # averaged over dispatches
    assert red["bytes"] == pytest.approx(1001.0 * 1024 * 2 + 300.0 * 1024)
    assert red["valu_insts"] == 5898240.0
    assert "valu_insts" not in t["kernels"]["quantize_kernel"]
    assert bench.traffic_for("reduce_kernel") == pytest.approx(red["bytes"])
    # figures taken on other kernel sources are not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "another-tree")
    assert bench.traffic_for("reduce_kernel") is None
    assert bench.counters_for("reduce_kernel") == {}


def test_summarize_trace_table(tmp_path, capsys):
    db = tmp_path / "r.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, end integer)")
    con.executemany("insert into kernels values (?, ?, ?)",
                    [("void rc::reduce_kernel<2, 1, 32, 4>(rc::StreamPtrs, int)", 0, 15000),
                     ("void rc::reduce_kernel<2, 1, 32, 4>(rc::StreamPtrs, int)", 20000, 36000),
                     ("rc::copy_kernel(...)", 40000, 41000)])
    con.commit()
    con.close()
    assert bench.summarize_trace(str(db)) == 0
    out = capsys.readouterr().out.splitlines()
    assert out[0].startswith("| kernel | calls | avg ns")
    assert out[2] == "| void rc::reduce_kernel<2, 1, 32, 4> | 2 | 15500 | 15000 | 16000 | 31000 |"
    assert out[3] == "| rc::copy_kernel | 1 | 1000 | 1000 | 1000 | 1000 |"


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hpp"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hpp"])
    src.write_text('// header\nint f(int x) { return x + 1; }  /* note */\nconst char* s = "a // b";\n')
    h0 = bench.kernel_source_hash()
    src.write_text('// another header\n\nint f(int x)  { return x + 1; }\n/* longer\n note */ const char* s = "a // b";\n')
    assert bench.kernel_source_hash() == h0                      # comments and layout only
    src.write_text('// header\nint f(int x) { return x + 2; }  /* note */\nconst char* s = "a // b";\n')
    assert bench.kernel_source_hash() != h0                      # code
    src.write_text('// header\nint f(int x) { return x + 1; }  /* note */\nconst char* s = "a /// b";\n')
    assert bench.kernel_source_hash() != h0                      # a string literal is code


def test_committed_counters_are_for_these_kernels():
    """The stored HBM traffic and VALU counts were taken on the kernel code of
    this tree (bench.py drops them from its JSON line otherwise), and they say
    that the dominant kernels move what the method must move and no more."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["kernel_source_sha"] == bench.kernel_source_hash()
    for name, alg in (("reduce_kernel", 73400320), ("quantize_kernel", 81788928)):
        k = t["kernels"][name]
        assert 1.0 <= k["bytes"] / alg < 1.01, name
        assert k["valu_insts"] > 0, name
