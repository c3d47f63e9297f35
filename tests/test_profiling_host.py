"""Host tests of the rocprofv3 evidence harness (no GPU): the reductions of
block_sparse_attention_flashattention_amd.profiling on a small fixture cut
from this project's own rocprofv3 output of the VSA-256 workload (two
dispatches of the 256-row kernel and one other kernel per counter file, the
copy calibration, the kernel statistics and the traced run's bench line)."""

import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from block_sparse_attention_flashattention_amd import profiling as P  # noqa: E402

DATA = os.path.join(ROOT, "tests", "data", "rocprof")
KERNEL = "vsa_fwd_pp_kernel<128,128,false>"
WORKLOAD = "vsa256_b1h24s32768d128_keep13"


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _ours(rows, counter):
    return [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and "vsa_fwd_pp_kernel<128, 128, false>" in r["Kernel_Name"]]


def test_short_names_and_stats():
    assert P.short_name("void vsa::(anonymous namespace)::vsa_fwd_pp_kernel<128, 128, false>(vsa::FwdParams)") == \
        "vsa_fwd_pp_kernel<128, 128, false>"
    stats = P.kernel_stats(os.path.join(DATA, "c2", "trace", "run_kernel_stats.csv"))
    main = [r for r in stats if r["short"].replace(" ", "") == KERNEL]
    assert len(main) == 1 and main[0]["calls"] == 313
    assert main[0]["avg_us"] == pytest.approx(1115.216619808)
    assert not any(P.is_ours(r) for r in stats if "at::native" in r["name"] or r["name"].startswith("__amd"))
    assert not P.is_ours({"name": "void vsa::(anonymous namespace)::mfma_rate_kernel<false>(...)"})
    assert P.is_ours({"name": "void vsa::(anonymous namespace)::vsa_fwd_pp_kernel<128, 128, false>(vsa::FwdParams)"})


def test_sq_reduction_by_hand():
    path = os.path.join(DATA, "c2", "sq", "run_counter_collection.csv")
    rows = _rows(path)
    mops, busy, grbm = (_ours(rows, c) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
                                                  "GRBM_GUI_ACTIVE"))
    conf, lds = _ours(rows, "SQ_LDS_BANK_CONFLICT"), _ours(rows, "SQ_ACTIVE_INST_LDS")
    assert len(mops) == 2
    s = P.sq_summary(path, KERNEL)
    assert s["dispatches"] == 2
    assert s["mfma_flops"] == pytest.approx(512 * sum(mops) / 2)
    # the sparse-aware count of this workload: 4*D*pairs = 4*128*2617245696
    assert s["mfma_flops"] == pytest.approx(4 * 128 * 2617245696, rel=1e-9)
    assert s["mfma_busy"] == pytest.approx((sum(busy) / 2) / (sum(grbm) / 2 / 8 * 1024))
    assert 0.0 < s["mfma_busy"] < 1.0
    assert s["lds_conflict_rate"] == pytest.approx((sum(conf) / 2) / (sum(lds) / 2))
    with pytest.raises(ValueError):
        P.sq_summary(path, "vsa_fwd_iw_kernel<64,128,false>")


def test_traffic_scaled_by_the_copy():
    c = os.path.join(DATA, "c2")
    tr = P.traffic(os.path.join(c, "fetch", "run_counter_collection.csv"),
                   os.path.join(c, "write", "run_counter_collection.csv"),
                   os.path.join(DATA, "copy_fetch"), os.path.join(DATA, "copy_write"), KERNEL)
    cf = [float(r["Counter_Value"]) for r in _rows(os.path.join(DATA, "copy_fetch", "run_counter_collection.csv"))]
    cw = [float(r["Counter_Value"]) for r in _rows(os.path.join(DATA, "copy_write", "run_counter_collection.csv"))]
    fs, ws = (1 << 30) / (1024 * sum(cf) / len(cf)), (1 << 30) / (1024 * sum(cw) / len(cw))
    f = _ours(_rows(os.path.join(c, "fetch", "run_counter_collection.csv")), "FETCH_SIZE")
    w = _ours(_rows(os.path.join(c, "write", "run_counter_collection.csv")), "WRITE_SIZE")
    assert tr["fetch_bytes"] == round(sum(f) / len(f) * 1024 * fs)
    assert tr["write_bytes"] == round(sum(w) / len(w) * 1024 * ws)
    assert tr["bytes_per_launch"] == tr["fetch_bytes"] + tr["write_bytes"]
    # the kernel reads at least the compulsory Q, K, V bytes of the workload
    assert tr["fetch_bytes"] > 3 * 32768 * 24 * 128 * 2


def test_summary_text_carries_the_figures():
    text, tr = P.summarize(DATA, "c2", WORKLOAD, "256x128", write_files=False)
    b = json.loads(open(os.path.join(DATA, "c2", "bench_line.json")).read())
    assert text.startswith(f"# {KERNEL} on {WORKLOAD}, tiles 256x128")
    assert "rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o run -- python3 <repo>/bench.py" \
        in text
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    assert "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512" in text
    assert f"{b['roofline']['achieved']:.1f} TFLOP/s sparse-aware" in text
    assert f"{tr['fetch_bytes'] / 1e9:.3f} GB" in text
    assert "| vsa_fwd_pp_kernel<128, 128, false> | 313 | 1115.2 |" in text
    assert tr["kernel"] == KERNEL and tr["source_hash"]


def test_pass_commands_keep_counters_apart_from_tracing():
    for name, opts, flags in P.passes(WORKLOAD, "256x128"):
        if "--pmc" in opts:
            assert not any(o in opts for o in ("--kernel-trace", "--sys-trace", "--runtime-trace", "-s", "-r"))
            # at most 8 SQ counters and 4 TCC-style counters in one pass
            assert sum(o.startswith("SQ_") for o in opts) <= 8
        assert "--no-configs" in flags and "--no-cpu-baseline" in flags
        cmd = P.command("/tmp/x", opts, flags)
        assert cmd[cmd.index("--") + 1] == sys.executable  # the program itself follows "--"


def _write_counters(path, kernel, values):
    """A rocprofv3 counter CSV with one row per (dispatch, counter)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    head = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,Kernel_Name,"
            "Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,SGPR_Count,Counter_Name,"
            "Counter_Value,Start_Timestamp,End_Timestamp")
    with open(path, "w") as f:
        f.write(head + "\n")
        for disp, per in enumerate(values, start=1):
            for counter, val in per.items():
                f.write(f'{disp},{disp},Agent 1,1,1,1,1,1,"void vsa::(anonymous namespace)::{kernel}(vsa::BwdParams)",'
                        f"256,0,0,4,0,16,{counter},{val},0,1\n")


def test_backward_kernel_section_from_counters(tmp_path):
    """The backward section reduces each backward kernel's counters like the
    forward's: executed MFMA flops = MOPS x 512, their rate over the trace
    average, busy fraction and HBM bytes scaled by the copy."""
    import shutil
    out = str(tmp_path)
    shutil.copytree(os.path.join(DATA, "copy_fetch"), os.path.join(out, "copy_fetch"))
    shutil.copytree(os.path.join(DATA, "copy_write"), os.path.join(out, "copy_write"))
    d = os.path.join(out, "t")
    k = "vsa_bwd_dq_kernel<256, 128, false, false>"
    sq = {"SQ_VALU_MFMA_BUSY_CYCLES": 4.0e8, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 4.0e9, "SQ_LDS_BANK_CONFLICT": 0.0,
          "SQ_ACTIVE_INST_LDS": 1.0e7, "SQ_BUSY_CYCLES": 1.0e7, "SQ_WAVES": 24576.0, "GRBM_GUI_ACTIVE": 8.0e6}
    _write_counters(os.path.join(d, "sq", "run_counter_collection.csv"), k, [sq, sq])
    _write_counters(os.path.join(d, "fetch", "run_counter_collection.csv"), k, [{"FETCH_SIZE": 1.0e6}] * 2)
    _write_counters(os.path.join(d, "write", "run_counter_collection.csv"), k, [{"WRITE_SIZE": 2.0e5}] * 2)
    ours = [{"name": f"void vsa::{k}(vsa::BwdParams)", "short": k, "calls": 2, "avg_us": 2000.0, "min_us": 1.0,
             "max_us": 3.0}]
    lines = P.backward_kernel_lines(out, d, ours)
    row = [ln for ln in lines if ln.startswith(f"| {k} |")]
    assert len(row) == 1
    flops = 4.0e9 * 512
    busy = 4.0e8 / (8.0e6 / 8 * 1024)
    assert f"| {flops:.4g} | {flops / 2000e-6 / 1e12:.1f} | {100 * busy:.1f}% |" in row[0]
    fs = P.copy_scale(os.path.join(out, "copy_fetch"), "FETCH_SIZE")
    assert f"{1.0e6 * 1024 * fs / 1e9:.3f} + " in row[0]
    # no backward dispatches in the counters: no section
    assert P.backward_kernel_lines(out, os.path.join(DATA, "c2"), ours) == []
