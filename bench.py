"""Benchmark of the codec hot path on one MI355X.

One step = one pass of the whole hot path over one message: INT3
quantize_pack of a 64 MiB bf16 message (33,554,432 Student-t values) into the
first of four packed stream buffers, then a 4-stream dequant_reduce_requant of
that stream and three pre-packed peer streams into one packed output.  Inputs
are resident in HBM before timing starts; eight buffer sets are rotated so the
working set (about 1 GiB) defeats the 256 MiB Infinity Cache.  After the
eager warmup steps, the timed steps are recorded into one HIP graph and
replayed once, so the timed region holds GPU work only.

Prints one JSON line: value = uncompressed GB/s (input bytes of the quantize
plus K x message bytes of the reduce, per second), a `roofline` object for the
dominant kernel (algorithmic bytes per launch / average launch time, from HIP
events around a graph of back-to-back launches, against 8 TB/s) and a
`cpu_baseline` object (the plain C oracle on the host cores over a sample of
the same workload).

Extra modes:
  --table                               per-kernel table over codecs (--table-codecs),
                                        sizes (--table-mib), stream counts
                                        (--table-k) and message dtypes (--table-dt)
  --fused                               the one-kernel all-reduce emulation against
                                        the separate kernels
  --gemv                                the MXFP4 GEMV on the 4096 x 4096 weight recipe
  --summarize-trace RESULTS_DB          kernel-duration table of a rocprofv3 trace
  --summarize-pmc FETCH_DIR WRITE_DIR [SQ_DIR]
                                        turn `rocprofv3 --pmc` runs of this
                                        script into profiles/traffic_*.json
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
VALU_PEAK_GINST = 256 * 4 * 2.4 / 4          # 256 CUs x 4 SIMDs, a wave64 instruction per 4 cycles at 2.4 GHz
METRIC = "codec GB/s (uncompressed bytes) and % of HBM peak, 64 MB INT3 quant+reduce"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_int3_64MiB.json")
KERNEL_SOURCES = ["reduction_codec_amd/csrc/rc_device.hpp", "reduction_codec_amd/csrc/rc_kernels.hpp",
                  "reduction_codec_amd/csrc/rc_inst_default.hip"]
COPY_BYTES = 256 << 20


def strip_comments(src: str) -> str:
    """C/C++ source without its comments and with whitespace runs collapsed,
    string and character literals kept as written."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored): the
    stored counter figures are reported only while it matches."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--mib", type=int, default=64, help="message size in MiB of bf16")
    ap.add_argument("--k", type=int, default=4, help="streams in the reduce")
    ap.add_argument("--fmt", default="int3", choices=["int3", "int4", "fp8", "mxfp4"])
    ap.add_argument("--sets", type=int, default=0, help="rotation buffer sets (0 = enough for 1 GiB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR [SQ_DIR]: rocprofv3 --pmc runs of FETCH_SIZE, WRITE_SIZE "
                         "and (optionally) SQ_INSTS_VALU")
    ap.add_argument("--summarize-trace", metavar="RESULTS_DB",
                    help="per-kernel duration table from a rocprofv3 --kernel-trace results database")
    ap.add_argument("--table", action="store_true",
                    help="per-kernel table over every format and --table-mib sizes (no JSON line)")
    ap.add_argument("--table-mib", default="16,64,256,1024")
    ap.add_argument("--table-codecs", default="int3,int4,fp8,mxfp4",
                    help="comma list of codec names (default names or <elem>_<scale>_b<block>), or 'all'")
    ap.add_argument("--table-k", default="2,4,8", help="stream counts of the reduce rows")
    ap.add_argument("--table-dt", default="bf16", choices=["bf16", "fp16", "fp32"],
                    help="message dtype of the table: quantize input, unpack output, copy and fill")
    ap.add_argument("--gemv", action="store_true",
                    help="MXFP4 GEMV on the 4096x4096 weight recipe (no JSON line)")
    ap.add_argument("--fused", action="store_true",
                    help="fused all-reduce emulation against the separate kernels (no JSON line)")
    return ap.parse_args()


# --------------------------------------------------------------- PMC ----

def _read_counter_rows(d: str):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True):
        import csv
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def summarize_pmc(fetch_dir: str, write_dir: str, sq_dir: str | None = None):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, scaled by
    what the same counters read for the plain copy kernel of known size; with
    sq_dir (a run that collected SQ_INSTS_VALU), also the wave64 VALU
    instructions each launch issues."""
    def per_kernel(d, counter):
        acc = {}
        for r in _read_counter_rows(d):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            acc.setdefault(name, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    valu = per_kernel(sq_dir, "SQ_INSTS_VALU") if sq_dir else {}

    def find(table, key):
        hits = [v for k, v in table.items() if key in k]
        return hits[0] if hits else None

    copy_f, copy_w = find(fetch, "copy_kernel"), find(write, "copy_kernel")
    fscale = COPY_BYTES / (copy_f * 1024.0) if copy_f else None
    wscale = COPY_BYTES / (copy_w * 1024.0) if copy_w else None
    out = {"kernel_source_sha": kernel_source_hash(), "copy_bytes": COPY_BYTES,
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "fetch_scale": fscale, "write_scale": wscale,
           "kernels": {}}
    for key in ("reduce_kernel", "quantize_kernel"):
        f, w = find(fetch, key), find(write, key)
        if f is None or w is None or fscale is None or wscale is None:
            continue
        out["kernels"][key] = {"fetch_kib": f, "write_kib": w,
                               "bytes": f * 1024.0 * fscale + w * 1024.0 * wscale}
        v = find(valu, key)
        if v is not None:
            out["kernels"][key]["valu_insts"] = v
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def summarize_trace(db_path: str) -> int:
    """Markdown table of kernel dispatch durations (count, average, min, max
    in ns) from the SQLite database rocprofv3 writes with --kernel-trace."""
    import sqlite3
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, count(*), avg(end - start), min(end - start), max(end - start), "
                       "sum(end - start) from kernels group by name order by sum(end - start) desc").fetchall()
    print("| kernel | calls | avg ns | min ns | max ns | total ns |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, cnt, avg, lo, hi, tot in rows:
        print(f"| {name.split('(')[0]} | {cnt} | {avg:.0f} | {lo} | {hi} | {tot} |")
    return 0


def counters_for(kernel_key: str) -> dict:
    """The stored counter figures of one kernel, or {} when they were taken
    from other kernel sources than the ones in this tree."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return {}
    if t.get("kernel_source_sha") != kernel_source_hash():
        return {}
    return t.get("kernels", {}).get(kernel_key) or {}


def traffic_for(kernel_key: str):
    return counters_for(kernel_key).get("bytes")


# -------------------------------------------------------------- bench ----

def main():
    args = parse_args()
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3):
            sys.stderr.write("--summarize-pmc takes FETCH_DIR WRITE_DIR [SQ_DIR]\n")
            return 2
        summarize_pmc(*args.summarize_pmc)
        return 0
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.table:
        return table(args)
    if args.fused:
        return fused_table(args)
    if args.gemv:
        return gemv_table(args)
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only: this codec build has no multi-GPU path "
                         "(run with --gpus 1)\n")
        return 2

    import numpy as np
    import torch

    import datagen
    import reduction_codec_amd as rca

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    codec = rca.CODECS[args.fmt]
    n = args.mib * (1 << 20) // 2
    K = args.k
    pb = rca.packed_bytes(codec, n)
    tiles = -(-n // 2048)
    set_bytes = 2 * n + (K + 1) * pb
    sets = args.sets or max(2, -(-(1 << 30) // set_bytes))

    # seeded inputs: message k = Student-t nu=4 bf16, seed 500+k
    host = [datagen.bf16_student4(2 * n, k) for k in range(K)]
    dev_msgs = [torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev) for h in host]
    peers = [rca.quantize_pack(m, codec) for m in dev_msgs]           # what the peers would send
    bufs = []
    for s in range(sets):
        x = dev_msgs[0].clone()
        streams = [torch.empty(pb, dtype=torch.uint8, device=dev)] + [p.clone() for p in peers[1:]]
        out = torch.empty(pb, dtype=torch.uint8, device=dev)
        bufs.append((x, streams, out))
    torch.cuda.synchronize()

    def step(i):
        x, streams, out = bufs[i % sets]
        rca.quantize_pack(x, codec, out=streams[0])
        rca.dequant_reduce_requant(streams, codec, n, out=out)

    def q_only(i):
        x, streams, _ = bufs[i % sets]
        rca.quantize_pack(x, codec, out=streams[0])

    def r_only(i):
        _, streams, out = bufs[i % sets]
        rca.dequant_reduce_requant(streams, codec, n, out=out)

    # W eager warmup steps; then the K timed steps are recorded once into a
    # HIP graph (buffer sets rotating) and replayed, so the timed region holds
    # GPU work only, without per-call host overhead.  Per-kernel durations come
    # from graphs of back-to-back launches of one kernel.  Events are recorded
    # on the replay stream.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def capture(fn, count, first=0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + count):
                fn(i)
        return g

    timed_steps = capture(step, args.steps, args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    timed_steps.replay()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    del timed_steps

    def timed(fn, reps):
        g = capture(fn, reps)
        g.replay()                                  # warm
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(20, args.steps)
    q_ms = timed(q_only, reps)
    r_ms = timed(r_only, reps)

    # the replayed graphs computed what the eager calls compute
    capture(step, 1).replay()
    torch.cuda.synchronize()
    x, streams, out = bufs[0]
    q_eager = rca.quantize_pack(x, codec)
    r_eager, _ = rca.dequant_reduce_requant([q_eager] + streams[1:], codec, n)
    torch.cuda.synchronize()
    if not (torch.equal(q_eager, streams[0]) and torch.equal(r_eager, out)):
        raise RuntimeError("graph replay output differs from the eager launch")

    # plain copy of 256 MiB: the achievable-bandwidth reference in this run
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    c_ms = timed(lambda i: rca.copy(dst, src), 20)
    del src, dst

    q_bytes = 2 * n + pb                      # algorithmic HBM bytes of one quantize launch
    r_bytes = (K + 1) * pb                    # K packed streams in, one packed stream out
    unc = 2 * n + K * 2 * n                   # uncompressed bytes processed per step
    value = unc / (ms * 1e-3) / 1e9
    step_hbm = (q_bytes + r_bytes) / (ms * 1e-3) / 1e9
    def kernel_roof(key, nbytes, kms):
        achieved = nbytes / (kms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(key),
             "kernel": f"{key}<{args.fmt}" + (f", K={K}>" if key == "reduce_kernel" else ", bf16>"),
             "bytes_per_launch": nbytes, "avg_launch_ms": round(kms, 5)}
        valu = counters_for(key).get("valu_insts")
        if valu:
            # the same launch against the vector-ALU issue limit: wave64 VALU
            # instructions (SQ_INSTS_VALU) per launch / launch time, against one
            # instruction per 4 cycles on each of 256 x 4 SIMDs at 2.4 GHz
            rate = valu / (kms * 1e-3) / 1e9
            r["alu"] = {"valu_insts_per_launch": int(valu), "achieved": round(rate, 1),
                        "peak": VALU_PEAK_GINST, "unit": "G wave64 VALU instructions/s",
                        "frac": round(rate / VALU_PEAK_GINST, 4)}
        return r

    # the dominant kernel is the longer of the two launches; both are listed,
    # since at some sizes they take about the same time
    per_kernel = {"quantize_kernel": kernel_roof("quantize_kernel", q_bytes, q_ms),
                  "reduce_kernel": kernel_roof("reduce_kernel", r_bytes, r_ms)}
    dom_key = "reduce_kernel" if r_ms >= q_ms else "quantize_kernel"
    roof = dict(per_kernel[dom_key])
    roof["per_kernel"] = per_kernel

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args, host, n, K)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.mib} MiB bf16 Student-t(nu=4) message: {args.fmt.upper()} quantize_pack + "
                               f"{K}-stream dequant_reduce_requant", "format": args.fmt, "n": n, "k": K,
                   "tiles": tiles, "rotation_sets": sets, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "breakdown": {
            "quantize_ms": round(q_ms, 5), "quantize_hbm_gbs": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "quantize_uncompressed_gbs": round(2 * n / (q_ms * 1e-3) / 1e9, 1),
            "reduce_ms": round(r_ms, 5), "reduce_hbm_gbs": round(r_bytes / (r_ms * 1e-3) / 1e9, 1),
            "reduce_uncompressed_gbs": round(K * 2 * n / (r_ms * 1e-3) / 1e9, 1),
            "step_hbm_gbs": round(step_hbm, 1), "step_hbm_frac": round(step_hbm / HBM_PEAK_GBS, 4),
            "copy_256MiB_gbs": round(2 * COPY_BYTES / (c_ms * 1e-3) / 1e9, 1),
            "host_wall_ms_per_step": round(wall_ms, 5),
            "timing": "HIP graph replays; events on the replay stream",
        },
    }
    print(json.dumps(line), flush=True)
    return 0


def table(args):
    """Average launch time of every kernel family per format and message size
    (messages of --table-dt, bf16 by default; K packed streams for the
    reduce), from a HIP graph of 30 back-to-back launches, with algorithmic
    HBM bytes per launch / time against the 8 TB/s peak."""
    import numpy as np
    import torch

    import datagen
    import reduction_codec_amd as rca

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def timed(fn, reps=30):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()                  # back-to-back launches, no host overhead
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    print("| MiB | format | kernel | us | HBM GB/s | % of peak | uncompressed GB/s |")
    print("|---:|---|---|---:|---:|---:|---:|")
    dt = args.table_dt
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dt]
    es = 4 if dt == "fp32" else 2                   # bytes per element of the message
    for mib in [int(v) for v in args.table_mib.split(",")]:
        n = mib * (1 << 20) // es
        x0 = torch.from_numpy(datagen.bf16_student4(2 * n, 0).view(np.int16)).view(torch.bfloat16).to(dev).to(tdt)
        names = sorted(rca.ALL_CODECS) if args.table_codecs == "all" else args.table_codecs.split(",")
        ks = [int(v) for v in args.table_k.split(",")]
        # the achievable-bandwidth reference at this size: a plain copy of the message
        csets = max(1, -(-(1 << 30) // (2 * es * n)))
        cbufs = [(x0.clone(), torch.empty_like(x0)) for _ in range(csets)]
        ms = timed(lambda i: rca.copy(cbufs[i % csets][1], cbufs[i % csets][0]))
        g = 2 * es * n / (ms * 1e-3) / 1e9
        print(f"| {mib} | - | copy {dt} (reference) | {ms * 1e3:.2f} | {g:.0f} | {100 * g / HBM_PEAK_GBS:.1f} | "
              f"{es * n / (ms * 1e-3) / 1e9:.0f} |", flush=True)
        # and a write-only reference for the write-heavy unpack: torch's fill of
        # the same bytes
        ms = timed(lambda i: cbufs[i % csets][1].fill_(1.0))
        g = es * n / (ms * 1e-3) / 1e9
        print(f"| {mib} | - | fill {dt}, write only (reference) | {ms * 1e3:.2f} | {g:.0f} | "
              f"{100 * g / HBM_PEAK_GBS:.1f} | - |", flush=True)
        del cbufs
        for fmt in names:
            codec = rca.CODECS[fmt] if fmt in rca.CODECS else rca.ALL_CODECS[fmt]
            pb = rca.packed_bytes(codec, n)
            kmax = max(ks)
            sets = max(1, -(-(1 << 30) // (2 * es * n + (kmax + 1) * pb)))
            bufs = []
            for _ in range(sets):
                x = x0.clone()
                p = rca.quantize_pack(x, codec)
                streams = [p] + [p.clone() for _ in range(kmax - 1)]
                bufs.append((x, streams, torch.empty(pb, dtype=torch.uint8, device=dev),
                             torch.empty(n, dtype=tdt, device=dev)))
            torch.cuda.synchronize()
            rows = [(f"quantize_pack {dt}", lambda i: rca.quantize_pack(bufs[i % sets][0], codec, out=bufs[i % sets][2]),
                     es * n + pb, es * n)]
            for K in ks:
                rows.append((f"dequant_reduce_requant K={K}",
                             (lambda K: lambda i: rca.dequant_reduce_requant(bufs[i % sets][1][:K], codec, n,
                                                                              out=bufs[i % sets][2]))(K),
                             (K + 1) * pb, K * es * n))
            # unpack reads nothing but a packed stream: it walks over all the
            # packed streams of the sets, cloned up to 1 GiB, so that the
            # streams one graph reads (30 launches) exceed the 256 MiB
            # Infinity Cache (its plain loads of large streams would hit there)
            packs = [st for b in bufs for st in b[1]]
            while len(packs) * pb < (1 << 30) and len(packs) < 30:
                packs.append(packs[len(packs) % (sets * kmax)].clone())
            npk = len(packs)
            rows.append((f"unpack_dequant {dt}",
                         lambda i: rca.unpack_dequant(packs[i % npk], codec, n, tdt, out=bufs[i % sets][3]),
                         pb + es * n, es * n))
            for name, fn, hbm, unc in rows:
                ms = timed(fn)
                g = hbm / (ms * 1e-3) / 1e9
                print(f"| {mib} | {fmt} | {name} | {ms * 1e3:.2f} | {g:.0f} | {100 * g / HBM_PEAK_GBS:.1f} | "
                      f"{unc / (ms * 1e-3) / 1e9:.0f} |", flush=True)
            del bufs, packs
            torch.cuda.empty_cache()
    return 0


def fused_table(args):
    """The fused one-GPU all-reduce emulation (rc_allreduce_emulate, two-shot
    and one-shot) against the same pipeline as separate kernels (K quantizes,
    one K-stream reduce, one unpack), for bf16 messages of --table-mib MiB
    per emulated rank.  HBM bytes count what each variant must move: fused =
    K messages in + output (+ the packed sum for two-shot); separate = every
    kernel's inputs and outputs."""
    import numpy as np
    import torch

    import datagen
    import reduction_codec_amd as rca

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def timed(fn, reps=20):
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    print("| MiB/rank | codec | K | variant | us | HBM GB/s | % of peak | uncompressed GB/s | vs separate |")
    print("|---:|---|---:|---|---:|---:|---:|---:|---:|")
    for mib in [int(v) for v in args.table_mib.split(",")]:
        n = mib * (1 << 20) // 2
        for K in [int(v) for v in args.table_k.split(",")]:
            msgs = [torch.from_numpy(datagen.bf16_student4(2 * n, 500 + j).view(np.int16)).view(torch.bfloat16).to(dev)
                    for j in range(K)]
            names = sorted(rca.ALL_CODECS) if args.table_codecs == "all" else args.table_codecs.split(",")
            for fmt in names:
                c = rca.CODECS[fmt] if fmt in rca.CODECS else rca.ALL_CODECS[fmt]
                pb = rca.packed_bytes(c, n)
                out = torch.empty(n, dtype=torch.bfloat16, device=dev)
                packed = torch.empty(pb, dtype=torch.uint8, device=dev)
                streams = [torch.empty(pb, dtype=torch.uint8, device=dev) for _ in range(K)]

                def separate(i):
                    for j in range(K):
                        rca.quantize_pack(msgs[j], c, out=streams[j])
                    rca.dequant_reduce_requant(streams, c, n, out=packed)
                    rca.unpack_dequant(packed, c, n, torch.bfloat16, out=out)

                t_sep = timed(separate)
                b_sep = K * (2 * n + pb) + (K + 1) * pb + (pb + 2 * n)
                t2 = timed(lambda i: rca.allreduce_emulate(msgs, c, True, out=out, packed_out=packed))
                t1 = timed(lambda i: rca.allreduce_emulate(msgs, c, False, out=out))
                unc = K * 2 * n
                for name, t, b in (("separate kernels", t_sep, b_sep), ("fused two-shot", t2, K * 2 * n + 2 * n + pb),
                                   ("fused one-shot", t1, K * 2 * n + 2 * n)):
                    g = b / (t * 1e-3) / 1e9
                    print(f"| {mib} | {fmt} | {K} | {name} | {t * 1e3:.2f} | {g:.0f} | {100 * g / HBM_PEAK_GBS:.1f} | "
                          f"{unc / (t * 1e-3) / 1e9:.0f} | {t_sep / t:.2f}x |", flush=True)
                del streams, out, packed
            del msgs
            torch.cuda.empty_cache()
    return 0


def gemv_table(args):
    """y = W x with W the 4096 x 4096 bf16 weight recipe packed as MXFP4
    (8.9 MB): one weight matrix (resident in the 256 MiB Infinity Cache after
    the first call) and a rotation over 64 copies (570 MB, so every call reads
    HBM).  HBM bytes per call = packed weights + x + y.  torch's bf16 matrix
    vector product of the unquantized weights is printed for context."""
    import numpy as np
    import torch

    import datagen
    import reduction_codec_amd as rca

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = cols = 4096
    wb = torch.from_numpy(datagen.bf16_weight_4096x4096().view(np.int16)).view(torch.bfloat16).to(dev)
    p = rca.quantize_pack(wb, rca.MXFP4)
    x = torch.from_numpy(np.random.default_rng(5).standard_normal(cols).astype(np.float32)).to(dev).to(torch.bfloat16)
    copies = [p] + [p.clone() for _ in range(63)]
    ys = [torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(64)]
    torch.cuda.synchronize()

    def timed(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    pb = p.numel()
    hbm = pb + 2 * cols + 4 * rows
    print("| case | us | GB/s (packed weights + x + y) | % of peak | weights/s |")
    print("|---|---:|---:|---:|---:|")
    for name, fn in (("MXFP4 GEMV, one weight matrix (cache-resident)",
                      lambda i: rca.mxfp4_gemv(p, rows, cols, x, out=ys[0])),
                     ("MXFP4 GEMV, 64 rotating weight matrices (HBM)",
                      lambda i: rca.mxfp4_gemv(copies[i % 64], rows, cols, x, out=ys[i % 64]))):
        t = timed(fn, 64)
        g = hbm / (t * 1e-3) / 1e9
        print(f"| {name} | {t * 1e3:.2f} | {g:.0f} | {100 * g / HBM_PEAK_GBS:.1f} | {rows * cols / (t * 1e-3) / 1e12:.2f} T |",
              flush=True)
    wm = wb.view(rows, cols)
    wcopies = [wm] + [wm.clone() for _ in range(15)]
    xv = x.view(cols, 1)
    t = timed(lambda i: torch.mm(wcopies[i % 16], xv), 32)
    g = (2 * rows * cols + 2 * cols + 2 * rows) / (t * 1e-3) / 1e9
    print(f"| torch bf16 mm (unquantized weights, 16 rotating copies), context | {t * 1e3:.2f} | {g:.0f} | "
          f"{100 * g / HBM_PEAK_GBS:.1f} | {rows * cols / (t * 1e-3) / 1e12:.2f} T |", flush=True)
    return 0


def cpu_baseline(args, host, n, K):
    """The oracle as it stands, over the same workload on the host cores:
    quantize the message, then reduce it with the peers (packed by the oracle,
    untimed), tile ranges split over all host threads; the whole step is
    repeated until about 1.5 s of wall time (10-30 s of CPU work) has passed."""
    import oracle
    c = oracle.CODECS[args.fmt]
    threads = max(1, len(os.sched_getaffinity(0)))
    tiles = -(-n // 2048)
    # bounded sample: whole tiles from the start of the message, at most 64 MiB of bf16
    sample_tiles = min(tiles, 16384)
    ns = min(n, sample_tiles * 2048)
    msgs = [h[:ns] for h in host]
    peers = [oracle.quantize_pack_parallel(c, m, dtype=oracle.DT_BF16, threads=threads) for m in msgs]
    reps, t0 = 0, time.perf_counter()
    while True:
        p0 = oracle.quantize_pack_parallel(c, msgs[0], dtype=oracle.DT_BF16, threads=threads)
        oracle.dequant_reduce_requant_parallel(c, [p0] + peers[1:], ns, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 1.5 or reps >= 50:
            break
    unc = reps * (2 * ns + K * 2 * ns)
    # and one thread on a smaller sample of the same message (about 1.5 s)
    ns1 = min(ns, 1024 * 2048)
    peers1 = [p[:oracle.packed_bytes(c, ns1)] for p in peers]
    reps1, t1 = 0, time.perf_counter()
    while True:
        p0 = oracle.quantize_pack_parallel(c, msgs[0][:ns1], dtype=oracle.DT_BF16, threads=1)
        oracle.dequant_reduce_requant_parallel(c, [p0] + peers1[1:], ns1, threads=1)
        reps1 += 1
        dt1 = time.perf_counter() - t1
        if dt1 >= 1.5 or reps1 >= 50:
            break
    unc1 = reps1 * (2 * ns1 + K * 2 * ns1)
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(unc / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu": model,
            "sample": f"{sample_tiles} tiles ({ns} elements) of the same message and peers, {reps} repetitions of "
                      f"quantize + {K}-stream reduce, tile ranges over {threads} threads, {dt:.2f} s wall",
            "single_thread": {"value": round(unc1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"the first {ns1 // 2048} tiles, {reps1} repetitions, {dt1:.2f} s wall"}}


if __name__ == "__main__":
    sys.exit(main())
