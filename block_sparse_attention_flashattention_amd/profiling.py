"""rocprofv3 evidence harness: per-workload kernel traces and hardware counters
of the forward kernels, reduced to short markdown summaries.

Two steps, both driven from the command line:

  collect    runs rocprofv3 on ``bench.py`` for one workload and tile shape:
             a kernel trace with stats, then one counter pass each for
             FETCH_SIZE, WRITE_SIZE and the MFMA / LDS counters (counter
             passes never combine with tracing domains); ``collect-copy``
             profiles a plain 1 GiB device copy for the byte-counter scale.
  summarize  reads those CSVs and writes ``profiles/<kernel>_<tile>_<workload>.md``
             (trace averages, the bench line of the traced run, MFMA flops and
             busy fraction, LDS bank conflicts, HBM bytes and GB/s) and the
             traffic JSON that ``bench.py`` reports as ``roofline.traffic``.

Reductions (per dispatch of the kernel, averaged over its dispatches):
  * MFMA flops          = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (one MOP is 512
                          flops of a bf16 MFMA), set beside the sparse-aware
                          algorithmic flops of the launch;
  * MFMA busy fraction  = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs
                          x SIMDs): GRBM_GUI_ACTIVE sums the active cycles of
                          the XCDs, the busy counter sums over every SIMD;
  * LDS bank conflicts  = SQ_LDS_BANK_CONFLICT over SQ_ACTIVE_INST_LDS cycles;
  * HBM bytes           = FETCH_SIZE and WRITE_SIZE (KiB) x the factor that
                          makes the copy kernel read and write exactly the
                          bytes it moves.

Nothing here touches the GPU itself: ``collect`` starts rocprofv3 as a child
process with ``python3 bench.py`` directly after ``--``.
"""

from __future__ import annotations

import argparse
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")
PROFILES = os.path.join(ROOT, "profiles")

SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT",
               "SQ_ACTIVE_INST_LDS", "SQ_BUSY_CYCLES", "SQ_WAVES", "GRBM_GUI_ACTIVE")
FLOPS_PER_MOP = 512
XCDS, SIMDS = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
COPY_BYTES = 1 << 30   # bench.py --copy-calibration


def bench_common(workload, tile, extra=()):
    """bench.py flags shared by every pass: the workload, no CPU leg, no other
    configs, no MFMA rate measurement, no clock sampling or flush launches, a
    short pre-warm."""
    return ["--no-cpu-baseline", "--no-configs", "--no-mfma-ceiling", "--clock-seconds", "0", "--flush-steps", "0",
            "--prewarm-seconds", "0.3", "--workload", workload, "--tile", tile, *extra]


def passes(workload, tile, extra=()):
    """(name, rocprofv3 options, bench flags) of the four passes, in order."""
    common = bench_common(workload, tile, extra)
    # the counter passes keep the bench's backward leg, whose kernels get a
    # section of their own (a few launches of each)
    short = [*common, "--steps", "2", "--warmup", "1"]
    return [
        ("trace", ["--kernel-trace", "--stats"], [*common, "--steps", "20", "--warmup", "5"]),
        ("fetch", ["--pmc", "FETCH_SIZE"], short),
        ("write", ["--pmc", "WRITE_SIZE"], short),
        ("sq", ["--pmc", *SQ_COUNTERS], short),
    ]


def command(out_dir, opts, bench_flags):
    return ["rocprofv3", *opts, "--output-format", "csv", "-d", out_dir, "-o", "run", "--",
            sys.executable, BENCH, *bench_flags]


def display_command(out_dir, opts, bench_flags):
    """The command of one pass as it is printed in a summary."""
    return " ".join(["rocprofv3", *opts, "--output-format", "csv", "-d", out_dir, "-o", "run", "--", "python3",
                     "<repo>/bench.py", *bench_flags])


def _run(cmd, log, timeout):
    print("[profiling] " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        try:
            r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=timeout, cwd="/tmp",
                               env={**os.environ, "TMPDIR": "/tmp"})
        except subprocess.TimeoutExpired:
            print(f"[profiling] timed out after {timeout} s: see {log}", flush=True)
            return 124
    return r.returncode


def collect(out, tag, workload, tile, extra=(), timeout=240):
    """Run the four passes into out/tag/{trace,fetch,write,sq}; stops at the
    first failure. The traced run's bench JSON line is kept as bench_line.json."""
    d = os.path.join(os.path.abspath(out), tag)
    os.makedirs(d, exist_ok=True)
    for name, opts, flags in passes(workload, tile, extra):
        log = os.path.join(d, f"{name}.log")
        rc = _run(command(os.path.join(d, name), opts, flags), log, timeout if name == "trace" else 120)
        if rc != 0:
            print(f"[profiling] {tag} {name} failed (rc={rc})", flush=True)
            return rc
        if name == "trace":
            lines = [ln for ln in open(log) if ln.startswith('{"metric"')]
            if not lines:
                print(f"[profiling] {tag}: no bench line in {log}", flush=True)
                return 1
            with open(os.path.join(d, "bench_line.json"), "w") as f:
                f.write(lines[-1])
        print(f"[profiling] {tag} {name} done", flush=True)
    return 0


def collect_copy(out, timeout=120):
    """FETCH_SIZE and WRITE_SIZE of a plain 1 GiB device copy (the scale)."""
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    for name, ctr in (("copy_fetch", "FETCH_SIZE"), ("copy_write", "WRITE_SIZE")):
        cmd = ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", os.path.join(out, name), "-o", "run", "--",
               sys.executable, BENCH, "--copy-calibration"]
        rc = _run(cmd, os.path.join(out, f"{name}.log"), timeout)
        if rc != 0:
            return rc
    return 0


# ------------------------------------------------------------------ reduction

def _norm(name):
    return name.replace(" ", "")


def short_name(name):
    """Kernel name without return type, namespaces and argument list."""
    n = name.replace("void ", "")
    for p in ("vsa::(anonymous namespace)::", "(anonymous namespace)::", "vsa::"):
        n = n.replace(p, "")
    return n.split("(")[0]


def kernel_stats(path):
    """Rows of run_kernel_stats.csv: name, calls, avg/min/max in microseconds."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "short": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3})
    return rows


MEASUREMENT_KERNELS = ("mfma_rate_kernel", "mfma_pingpong_kernel")  # vsa_measure_mfma, not the attention path


def is_ours(row):
    name = row["name"]
    return "at::" not in name and not name.startswith("__amd") and not any(k in name for k in MEASUREMENT_KERNELS)


def counter_values(path, counter, kernel):
    """Per-dispatch values of `counter` for the dispatches of `kernel` (a full
    template name such as vsa_fwd_pp_kernel<128,128,false>, spaces ignored)."""
    want = _norm(kernel)
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and _norm(short_name(r["Kernel_Name"])) == want:
                vals.append(float(r["Counter_Value"]))
    return vals


def _main_dispatches(mops):
    """Indices of the launches that did the work (an entry point that chooses
    its schedule on the device also launches kernels that exit at once)."""
    big = max(mops) if mops else 0.0
    return [i for i, m in enumerate(mops) if m > 0.5 * big] if big > 0 else list(range(len(mops)))


def sq_summary(sq_csv, kernel):
    """MFMA flops, MFMA busy fraction, LDS conflict rate and waves per
    dispatch, averaged over the kernel's working dispatches."""
    vals = {c: counter_values(sq_csv, c, kernel) for c in SQ_COUNTERS}
    sel = _main_dispatches(vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
    if not sel:
        raise ValueError(f"no dispatches of {kernel} in {sq_csv}")

    def avg(c):
        return sum(vals[c][i] for i in sel) / len(sel)

    grbm = avg("GRBM_GUI_ACTIVE")
    lds = avg("SQ_ACTIVE_INST_LDS")
    return {
        "dispatches": len(sel),
        "mfma_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_BF16") * FLOPS_PER_MOP,
        "mfma_busy": avg("SQ_VALU_MFMA_BUSY_CYCLES") / (grbm / XCDS * SIMDS) if grbm > 0 else 0.0,
        "lds_conflicts": avg("SQ_LDS_BANK_CONFLICT"),
        "lds_active": lds,
        "lds_conflict_rate": avg("SQ_LDS_BANK_CONFLICT") / lds if lds > 0 else 0.0,
        "waves": avg("SQ_WAVES"),
        "gui_active_cycles_per_xcd": grbm / XCDS,
    }


def copy_scale(copy_dir, counter):
    """Bytes per counter KiB: COPY_BYTES over what the counter reads for the
    copy kernel (averaged over its dispatches)."""
    vals = []
    with open(os.path.join(copy_dir, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower():
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} rows of a copy kernel in {copy_dir}")
    return COPY_BYTES / (1024.0 * sum(vals) / len(vals))


def traffic(fetch_csv, write_csv, copy_fetch_dir, copy_write_dir, kernel):
    """HBM bytes per launch of `kernel`, scaled by the copy calibration."""
    fs, ws = copy_scale(copy_fetch_dir, "FETCH_SIZE"), copy_scale(copy_write_dir, "WRITE_SIZE")
    fv, wv = counter_values(fetch_csv, "FETCH_SIZE", kernel), counter_values(write_csv, "WRITE_SIZE", kernel)
    if not fv or not wv:
        raise ValueError(f"no FETCH_SIZE / WRITE_SIZE dispatches of {kernel}")
    # the working launches read the most (skipped schedules exit at once)
    fbig, wbig = max(fv), max(wv)
    fetch = sum(x for x in fv if x > 0.5 * fbig) / len([x for x in fv if x > 0.5 * fbig]) * 1024.0 * fs
    write = sum(x for x in wv if x > 0.5 * wbig) / len([x for x in wv if x > 0.5 * wbig]) * 1024.0 * ws
    return {"fetch_bytes": round(fetch), "write_bytes": round(write), "bytes_per_launch": round(fetch + write),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}


def backward_kernel_lines(out, d, ours):
    """Per backward kernel of the counter passes (if they ran the backward
    leg): trace average, executed MFMA flops and their rate, MFMA busy, LDS
    conflicts and HBM bytes per launch; no lines if the counters hold none."""
    sq_csv = os.path.join(d, "sq", "run_counter_collection.csv")
    rows = []
    for r in sorted((r for r in ours if r["short"].startswith("vsa_bwd_")), key=lambda r: r["short"]):
        kname = _norm(r["short"])
        if not counter_values(sq_csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16", kname):
            continue
        try:
            sq = sq_summary(sq_csv, kname)
            tr = traffic(os.path.join(d, "fetch", "run_counter_collection.csv"),
                         os.path.join(d, "write", "run_counter_collection.csv"),
                         os.path.join(out, "copy_fetch"), os.path.join(out, "copy_write"), kname)
        except ValueError:
            continue
        rate = sq["mfma_flops"] / (r["avg_us"] * 1e-6) / 1e12
        rows.append(f"| {r['short']} | {r['avg_us']:.1f} | {sq['mfma_flops']:.4g} | {rate:.1f} | "
                    f"{100 * sq['mfma_busy']:.1f}% | {100 * sq['lds_conflict_rate']:.2f}% | "
                    f"{tr['fetch_bytes'] / 1e9:.3f} + {tr['write_bytes'] / 1e9:.3f} |")
    if not rows:
        return []
    return ["", "Backward kernels (trace average; counters per working dispatch, reduced as below; the flops are "
            "what the MFMAs executed, S and dP included in both kernels):", "",
            "| kernel | avg us | MFMA flop | executed TFLOP/s | MFMA busy | LDS conflicts | HBM GB (fetch + write) |",
            "|---|---|---|---|---|---|---|", *rows]


def summarize(out, tag, workload, tile, extra=(), profiles=PROFILES, write_files=True):
    """Write profiles/<kernel>_<tile>_<workload>.md and the traffic JSON from
    out/tag (collect) and out/copy_{fetch,write} (collect-copy); returns the
    markdown text and the traffic record."""
    sys.path.insert(0, ROOT)
    import bench

    d = os.path.join(out, tag)
    with open(os.path.join(d, "bench_line.json")) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    kname = b["roofline"]["kernel"]
    stats = kernel_stats(os.path.join(d, "trace", "run_kernel_stats.csv"))
    ours = [r for r in stats if is_ours(r)]
    main = [r for r in ours if _norm(r["short"]) == _norm(kname)]
    if not main:
        raise ValueError(f"{kname} not in the kernel trace of {d}")
    trace_us = max(main, key=lambda r: r["calls"] * r["avg_us"])["avg_us"]
    sq = sq_summary(os.path.join(d, "sq", "run_counter_collection.csv"), kname)
    tr = traffic(os.path.join(d, "fetch", "run_counter_collection.csv"),
                 os.path.join(d, "write", "run_counter_collection.csv"),
                 os.path.join(out, "copy_fetch"), os.path.join(out, "copy_write"), kname)
    tr = {"kernel": kname, "workload": workload, "tile": tile, **tr, "source_hash": bench.kernel_source_hash(kname)}
    flops = b["roofline"]["achieved"] * 1e12 * b["kernel_ms"] / 1e3
    ev_us = b["kernel_ms"] * 1e3
    ragged = "--ragged" in extra
    flags = " ".join(extra)
    common = " ".join(bench_common(workload, tile, extra))
    lines = [f"# {kname} on {workload}, tiles {tile}" + (f" ({flags})" if flags else ""), "",
             "One MI355X. Made by `python -m block_sparse_attention_flashattention_amd.profiling collect` and "
             "`... summarize` (rocprofv3 run from /tmp with TMPDIR=/tmp; `<repo>` is the repository root, "
             "`<out>` the output directory):", ""]
    for name, opts, bflags in passes(workload, tile, extra):
        lines.append("    " + display_command(f"<out>/{name}", opts, bflags))
    lines += ["    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/copy_fetch -o run -- python3 <repo>/bench.py "
              "--copy-calibration",
              "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/copy_write -o run -- python3 <repo>/bench.py "
              "--copy-calibration", "",
              f"Every pass runs bench.py with `{common}`.", "",
              "## Kernel trace (`run_kernel_stats.csv`; calls include the pre-warm steps)", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in ours:
        lines.append(f"| {r['short']} | {r['calls']} | {r['avg_us']:.1f} | {r['min_us']:.1f} | {r['max_us']:.1f} |")
    lines += ["", f"bench.py in the traced run (HIP events on the launch stream): kernel {ev_us:.1f} us = "
              f"{b['roofline']['achieved']:.1f} TFLOP/s sparse-aware ({flops:.4g} flop per launch"
              + (", valid pairs only" if ragged else "") + f"), {100 * b['roofline']['frac']:.1f}% of the "
              f"{b['roofline']['peak']:.0f} TFLOP/s dense bf16 peak; whole step {b['ms_per_step'] * 1e3:.1f} us.",
              f"Trace average {trace_us:.1f} us = {flops / (trace_us * 1e-6) / 1e12:.1f} TFLOP/s "
              f"({100 * flops / (trace_us * 1e-6) / 1e12 / b['roofline']['peak']:.1f}% of peak); "
              f"against the events {100 * (trace_us / ev_us - 1):+.1f}%."]
    bw = b.get("backward")
    if bw:
        lines += ["", "## Backward leg of the traced run (`vsa_csr_transpose` + `vsa_attn_bwd`)", "",
                  f"{bw['ms'] * 1e3:.1f} us per backward = {bw['tflops']:.1f} TFLOP/s at {bw['flops_per_pair']} "
                  f"flops per selected pair ({bw['pct_of_bf16_peak']:.1f}% of peak)."]
        lines += backward_kernel_lines(out, d, ours)
    lines += ["", "## Counters (mean per working dispatch of this kernel)", "",
              f"- MFMA: SQ_INSTS_VALU_MFMA_MOPS_BF16 x {FLOPS_PER_MOP} = {sq['mfma_flops']:.4g} flop "
              f"(sparse-aware algorithmic {flops:.4g}"
              + ("; valid pairs only, tiles are computed whole" if ragged else "") + "); MFMA busy "
              f"{100 * sq['mfma_busy']:.1f}% of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
              f"{XCDS} x {SIMDS})).",
              f"- LDS: SQ_LDS_BANK_CONFLICT = {sq['lds_conflicts']:.4g} over {sq['lds_active']:.4g} active LDS "
              f"instruction cycles ({100 * sq['lds_conflict_rate']:.2f}%).",
              f"- HBM: FETCH_SIZE x {tr['fetch_scale']:.3f} = {tr['fetch_bytes'] / 1e9:.3f} GB, WRITE_SIZE x "
              f"{tr['write_scale']:.3f} = {tr['write_bytes'] / 1e9:.3f} GB per launch "
              f"({tr['bytes_per_launch'] / (trace_us * 1e-6) / 1e12:.2f} TB/s at the trace average; "
              f"algorithmic {b['roofline'].get('algorithmic_bytes', 0) / 1e9:.3f} GB); the scale factors make a "
              f"1 GiB device copy read 1 GiB and write 1 GiB.",
              f"- Waves per launch: {sq['waves']:.0f}.", ""]
    text = "\n".join(lines)
    if write_files:
        os.makedirs(profiles, exist_ok=True)
        stem = kname.split("<")[0] + ("_partial" if kname.endswith("true>") else "")
        suffix = "_paired" if "--paired" in extra else ("_coalesced" if "--coalesce" in extra else "")
        with open(os.path.join(profiles, f"{stem}{suffix}_{tile}_{workload}.md"), "w") as f:
            f.write(text)
        tpath = bench.default_traffic_path(kname, workload, *(int(x) for x in
                                                               (b["config"].get("paired_onto") or tile).split("x")))
        with open(tpath, "w") as f:
            json.dump(tr, f, indent=1)
            f.write("\n")
    return text, tr


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    for name in ("collect", "summarize"):
        p = sub.add_parser(name)
        p.add_argument("--out", required=True)
        p.add_argument("--tag", required=True)
        p.add_argument("--workload", required=True)
        p.add_argument("--tile", required=True)
        p.add_argument("extra", nargs=argparse.REMAINDER, help="further bench.py flags (after --)")
    p = sub.add_parser("collect-copy")
    p.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "collect-copy":
        return collect_copy(a.out)
    extra = [x for x in a.extra if x != "--"]
    if a.cmd == "collect":
        return collect(a.out, a.tag, a.workload, a.tile, extra)
    text, tr = summarize(a.out, a.tag, a.workload, a.tile, extra)
    print(text)
    print(json.dumps(tr))
    return 0


if __name__ == "__main__":
    sys.exit(main())
