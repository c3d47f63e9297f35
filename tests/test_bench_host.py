"""Host-side logic of bench.py (no GPU): the kernel it names for the roofline,
the staleness check of measured traffic, the sparse-aware pair count, the
refusal of more than one GPU, and the parsing of the clock and power sample."""

import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_items_per_cu_switch_matches_the_library():
    with open(os.path.join(ROOT, "block_sparse_attention_flashattention_amd", "csrc", "vsa_internal.h")) as f:
        m = re.search(r"constexpr int kIwItemsPerCu = (\d+);", f.read())
    assert m and int(m.group(1)) == bench.IW_ITEMS_PER_CU


def test_kernel_names_follow_the_dispatch():
    cus = bench.compute_units()
    assert bench.kernel_name(256, 128, 128) == "vsa_fwd_pp_kernel<128,128,false>"
    assert bench.kernel_name(256, 64, 128, partial=True) == "vsa_fwd_pp_kernel<64,128,true>"
    assert bench.kernel_name(128, 128, 128, n_items=cus) == "vsa_fwd_2t_kernel<128,false>"
    assert bench.kernel_name(128, 64, 64, n_items=cus) == "vsa_fwd_2s_kernel<64,false>"
    assert bench.kernel_name(64, 64, 128, n_items=cus) == "vsa_fwd_4s_kernel<128,false>"
    assert bench.kernel_name(64, 64, 128, n_items=cus, entry=True) == "vsa_fwd_iw_kernel<64,128,false>"
    many = bench.IW_ITEMS_PER_CU * cus
    assert bench.kernel_name(128, 64, 128, n_items=many) == "vsa_fwd_iw_kernel<128,128,false>"
    assert bench.kernel_name(64, 64, 128, n_items=many) == "vsa_fwd_iw_kernel<64,128,false>"
    assert bench.kernel_name(64, 64, 128, n_items=many - 1) == "vsa_fwd_4s_kernel<128,false>"


def test_traffic_is_used_only_for_the_sources_it_was_measured_on(tmp_path):
    kname = "vsa_fwd_pp_kernel<128,128,false>"
    path = tmp_path / "t.json"
    path.write_text(json.dumps({"bytes_per_launch": 123, "source_hash": bench.kernel_source_hash(kname)}))
    assert bench.read_traffic(str(path), kname) == 123
    path.write_text(json.dumps({"bytes_per_launch": 123, "source_hash": "0" * 64}))
    assert bench.read_traffic(str(path), kname) is None
    assert bench.read_traffic(str(tmp_path / "missing.json"), kname) is None
    # each kernel family hashes its own source file
    assert bench.kernel_source_hash(kname) != bench.kernel_source_hash("vsa_fwd_iw_kernel<64,128,false>")


def test_selected_pairs_matches_a_token_level_count():
    B, H, nq, nkv, bq, bkv = 1, 2, 4, 8, 64, 32
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=3)
    assert bench.selected_pairs(torch.from_numpy(idx), torch.from_numpy(cnt), bq, bkv) == int(cnt.sum()) * bq * bkv
    valid = np.random.default_rng(4).integers(0, bkv + 1, size=nkv).astype(np.int32)
    want = sum(int(valid[idx[b, h, p, j]]) * bq for b in range(B) for h in range(H) for p in range(nq)
               for j in range(int(cnt[b, h, p])))
    got = bench.selected_pairs(torch.from_numpy(idx), torch.from_numpy(cnt), bq, bkv, torch.from_numpy(valid))
    assert got == want


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def _smi_json(watts):
    clock = {f"gfx_{i}": {"clk": {"value": 1600 + 10 * i, "unit": "MHz"}} for i in range(8)}
    clock["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    power = {"socket_power": {"value": watts, "unit": "W"} if watts is not None else "N/A", "gfx_voltage": "N/A"}
    return json.dumps({"gpu_data": [{"gpu": 0, "clock": clock, "power": power}]})


@pytest.mark.parametrize("watts", [1400, None])
def test_clock_sample_reads_gfx_clocks_and_socket_power(monkeypatch, watts):
    """sample_clock parses the gfx clock of every XCD and the socket power
    from amd-smi's JSON (layout as the tool prints it on MI355X); a missing
    power reading leaves the field empty rather than failing the bench."""
    calls = []

    def fake_run(cmd, **kw):
        calls.append(cmd)
        return subprocess.CompletedProcess(cmd, 0, stdout=_smi_json(watts), stderr="")

    monkeypatch.setattr(subprocess, "run", fake_run)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    steps = []
    out = bench.sample_clock(lambda: steps.append(1), 0.05)
    assert calls and calls[0][:2] == ["amd-smi", "metric"] and "--power" in calls[0] and "--clock" in calls[0]
    assert out["gfx_mhz"] == [1600.0 + 10 * i for i in range(8)]
    assert out["gfx_mhz_mean"] == pytest.approx(1635.0)
    assert out["socket_power_w"] == (None if watts is None else float(watts))
    assert steps  # steps ran while the sample was taken
