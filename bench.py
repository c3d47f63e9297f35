#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

One step = the whole forward path over one batch of synthetic input that is
already resident in HBM: logical mask -> physical block CSR (exact
expansion), the count-sorted work list, then the fused attention kernel.

Default workload: VSA-256 mask, B=1 H=24 S=32768 D=128, Q256/KV256 logical
blocks keeping 13 of 128 per row (~90% sparse), run on physical 256x128
tiles. Throughput is sparse-aware: 4*D*(selected token pairs) per step.

Prints one JSON line. The `roofline` object rates the attention kernel alone
(HIP events around its launches on the stream it runs on) against the dense
bf16 MFMA peak; `cpu_baseline` times the CPU oracle on a bounded sample of
the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published figure)
METRIC = "sparse-aware TFLOP/s and % of bf16 MFMA peak, block-sparse attn fwd S=32k"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="vsa256_b1h24s32768d128_keep13")
    ap.add_argument("--tile", default=None, help="physical QxKV tile, e.g. 128x64 (default: workload's first)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (the oracle timing and the parity checks of the timed outputs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the headline workload (skip the `configs` object: dense, the VSA-256 mask "
                         "on finer tiles natively and coalesced, and the native Q64 masks)")
    ap.add_argument("--config-cpu-seconds", type=float, default=2.5,
                    help="target CPU time of the oracle sample that checks each entry of `configs`")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with measured HBM bytes per kernel launch (default: the one under profiles/ "
                         "for this kernel and workload, written by the profiling module's `summarize` and used "
                         "only if the kernel sources are unchanged)")
    ap.add_argument("--prewarm-seconds", type=float, default=0.5,
                    help="run steps back to back for this long before the warmup steps, so that the timed "
                         "steps see the sustained clock rather than the ramp out of idle")
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="seconds of extra steps during which amd-smi samples the gfx clock and socket power (0: skip)")
    ap.add_argument("--flush-steps", type=int, default=10,
                    help="kernel launches timed after writing a buffer larger than the last-level cache")
    ap.add_argument("--ragged", type=int, default=None, metavar="SEED",
                    help="partial KV tiles: ragged valid-token counts per logical KV block drawn with this seed "
                         "(the masked kernels run; throughput counts valid pairs only)")
    ap.add_argument("--paired", action="store_true",
                    help="64-row tiles through vsa_attn_fwd_paired: adjacent query tiles with identical lists run as "
                         "128-row tiles (decided on the device; the timed scope then includes the pairing and both "
                         "work lists)")
    ap.add_argument("--coalesce", action="store_true",
                    help="64- or 128-row tiles through vsa_attn_fwd_coalesced: adjacent query tiles with identical "
                         "lists run as one tile, level by level up to 256 rows (decided on the device; the timed "
                         "scope then includes the pairing, the gates and all work lists)")
    ap.add_argument("--scope", choices=("kernel", "entry"), default="kernel",
                    help="kernel: the attention kernel over the work list built in the step (vsa_build_worklist + "
                         "vsa_attn_fwd_worklist, the kernel alone is timed); entry: vsa_attn_fwd, which builds its own "
                         "work list and splits lists when there are few work items (all of it is timed)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward leg (dQ, dK, dV of the same workload; reported beside the headline)")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the MFMA rate measurement reported beside the roofline (what the matrix cores "
                         "sustain on random bf16 operands, alone and beside softmax-shaped vector work, and on "
                         "zero operands; vsa_measure_mfma, about 0.3 s after the timed steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (for counter calibration)")
    return ap.parse_args()


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (how it would shard is a design note).",
              file=sys.stderr)
        return 2

    import torch

    import block_sparse_attention_flashattention_amd as vsa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}), flush=True)
        return 0

    wl = W.WORKLOADS[args.workload]
    if args.tile:
        tile = tuple(int(x) for x in args.tile.lower().split("x"))
    else:
        tile = wl.physical[0]
    bq, bkv = tile
    lq, lkv = wl.logical_block
    B, H, S, D = wl.batch, wl.heads, wl.seqlen, wl.head_dim

    # ---- inputs, resident in HBM before timing ----
    q_cpu, k_cpu, v_cpu = wl.qkv()
    mask_cpu = wl.logical_mask()
    q, k, v = (t.to(dev) for t in (q_cpu, k_cpu, v_cpu))
    mask = torch.from_numpy(np.ascontiguousarray(mask_cpu).copy()).to(dev)
    nq = S // bq
    ld = int(mask_cpu.sum(-1).max()) * (lkv // bkv)
    idx = torch.zeros((B, H, nq, ld), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, nq), dtype=torch.int32, device=dev)
    work = torch.empty((B * H * nq,), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    scale = wl.scale
    stream = torch.cuda.current_stream(dev)
    vbs = kv_valid = None
    if args.ragged is not None:
        vbs = torch.from_numpy(W.ragged_block_sizes(S // lkv, lkv, seed=args.ragged)).to(dev)
        kv_valid = torch.empty((S // bkv,), dtype=torch.int32, device=dev)

    if args.paired and bq != 64:
        print("--paired needs 64-row query tiles", file=sys.stderr)
        return 2
    if args.coalesce and (bq not in (64, 128) or args.paired):
        print("--coalesce needs 64- or 128-row query tiles and excludes --paired", file=sys.stderr)
        return 2

    def attention():
        if args.paired:
            vsa.vsa_attn_fwd_paired(q, k, v, idx, cnt, bkv, scale, o, lse, stream=stream, kv_valid=kv_valid)
        elif args.coalesce:
            vsa.vsa_attn_fwd_coalesced(q, k, v, idx, cnt, bq, bkv, scale, o, lse, stream=stream, kv_valid=kv_valid)
        elif args.scope == "entry":
            vsa.vsa_attn_fwd(q, k, v, idx, cnt, bq, bkv, scale, o, lse, stream=stream, kv_valid=kv_valid)
        else:
            vsa.vsa_attn_fwd_worklist(q, k, v, idx, cnt, bq, bkv, work, scale, o, lse, stream=stream,
                                      kv_valid=kv_valid)

    def step(ev0=None, ev1=None):
        if vbs is not None:
            vsa.vsa_expand_valid(vbs, lkv, bkv, kv_valid, stream=stream)
        # tiles without a valid key are left out of the lists
        vsa.vsa_mask_to_csr(mask, (lq, lkv), (bq, bkv), ld, idx, cnt, stream=stream, kv_valid=kv_valid)
        if not (args.paired or args.coalesce) and args.scope == "kernel":
            vsa.vsa_build_worklist(cnt, ld, work, segment=nq, stream=stream)
        if ev0 is not None:
            ev0.record(stream)
        attention()
        if ev1 is not None:
            ev1.record(stream)

    step()
    torch.cuda.synchronize()
    pairs = selected_pairs(idx, cnt, bq, bkv, kv_valid)
    run_bq = bq
    if args.paired:  # which schedule the device will choose (read once, outside the timed region)
        run_bq = 128 if int(vsa.vsa_pair_q_tiles(idx, cnt)[2].item()) == 0 else 64
    if args.coalesce:  # the same, level by level up to 256 rows
        ri, rc = idx, cnt
        while run_bq < 256 and S % 256 == 0:
            pi, pc, un = vsa.vsa_pair_q_tiles(ri, rc)
            if int(un.item()) != 0:
                break
            ri, rc, run_bq = pi, pc, run_bq * 2
        del ri, rc
    flops = 4.0 * D * pairs
    t_pre = time.perf_counter() + args.prewarm_seconds
    while time.perf_counter() < t_pre:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in events:
        step(e0, e1)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # the outputs of the last timed step, checked against the oracle below
    o_timed, lse_timed = o.clone(), lse.clone()
    kernel_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in events]))
    value = flops / (ms_step * 1e-3) / 1e12
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12

    # Wrapper scope: mask front-end + the entry point that builds its own
    # work list (what a caller without a cached work list pays).
    def wrapper():
        if vbs is not None:
            vsa.vsa_expand_valid(vbs, lkv, bkv, kv_valid, stream=stream)
        vsa.vsa_mask_to_csr(mask, (lq, lkv), (bq, bkv), ld, idx, cnt, stream=stream, kv_valid=kv_valid)
        if args.paired or args.coalesce:
            attention()
        else:
            vsa.vsa_attn_fwd(q, k, v, idx, cnt, bq, bkv, scale, o, lse, stream=stream, kv_valid=kv_valid)

    for _ in range(2):
        wrapper()
    torch.cuda.synchronize()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(args.steps):
        wrapper()
    w1.record(stream)
    torch.cuda.synchronize()
    wrapper_ms = w0.elapsed_time(w1) / args.steps

    # Post-flush: the kernel alone after overwriting a buffer larger than the
    # 256 MB last-level cache, so Q/K/V start cold.
    kernel_ms_flush = None
    if args.flush_steps > 0:
        junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fl_events = []
        for i in range(args.flush_steps):
            junk.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            attention()
            e1.record(stream)
            fl_events.append((e0, e1))
        torch.cuda.synchronize()
        kernel_ms_flush = float(np.mean([e0.elapsed_time(e1) for e0, e1 in fl_events]))
        del junk

    clock = sample_clock(step, args.clock_seconds) if args.clock_seconds > 0 else None
    backward = None if args.no_backward else time_backward(vsa, q, k, v, o, lse, idx, cnt, bq, bkv, scale, D, pairs,
                                                           args.steps, stream, kv_valid, args.clock_seconds)

    # Algorithmic HBM bytes of one kernel launch: Q, K, V read once, O and
    # LSE written once, CSR indices and counts read once.
    alg_bytes = (3 * B * S * H * D + B * S * H * D) * 2 + B * H * S * 4 + (B * H * nq) * (ld + 2) * 4
    kname = kernel_name(run_bq, bkv, D, partial=kv_valid is not None, n_items=B * H * (S // run_bq),
                        entry=args.scope == "entry")
    traffic = read_traffic(args.traffic or default_traffic_path(kname, wl.name, run_bq, bkv), kname)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": B, "heads": H, "seq_len": S, "head_dim": D,
            "logical_block": f"{lq}x{lkv}", "tile": f"{bq}x{bkv}",
            "paired_onto": f"{run_bq}x{bkv}" if (args.paired or args.coalesce) else None,
            "timed_scope": "vsa_attn_fwd_paired" if args.paired else "vsa_attn_fwd_coalesced" if args.coalesce else (
                "vsa_attn_fwd" if args.scope == "entry" else "vsa_attn_fwd_worklist"),
            "selected_pairs": pairs,
            "density": round(pairs / (B * H * S * S), 5),
            "parallelism": "single_gpu",
            "partial_tiles": None if vbs is None else {
                "vbs_seed": args.ragged, "valid_token_fraction": round(float(vbs.float().mean().item()) / lkv, 4)},
        },
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "kernel_ms": round(kernel_ms, 4),
        "kernel_tflops": round(kernel_tflops, 2),
        "frontend_ms": round(ms_step - kernel_ms, 4),
        "wrapper_ms": round(wrapper_ms, 4),
        "wrapper_tflops": round(flops / (wrapper_ms * 1e-3) / 1e12, 2),
        "kernel_ms_post_flush": None if kernel_ms_flush is None else round(kernel_ms_flush, 4),
        "kernel_tflops_post_flush": None if kernel_ms_flush is None else round(flops / (kernel_ms_flush * 1e-3) / 1e12, 2),
        "clock": clock,
        "backward": backward,
        "roofline": {
            "bound": "mfma",
            "achieved": round(kernel_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kernel_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_bytes": alg_bytes,
            "kernel": kname,
        },
    }

    ok = True
    if not args.no_cpu_baseline:
        base, sample = cpu_baseline(wl, q_cpu, k_cpu, v_cpu, idx, cnt, bq, bkv, args.cpu_seconds,
                                    None if kv_valid is None else kv_valid.cpu().numpy())
        result["cpu_baseline"] = base
        result["parity"] = compare_rows(o_timed, lse_timed, sample, S, H)
        result["parity"]["scope"] = "outputs of the last timed step against the oracle rows of cpu_baseline"
        ok = result["parity"]["pass"]
    del o_timed, lse_timed

    if not args.no_configs:
        result["configs"] = time_configs(vsa, W, wl, (bq, bkv), args, stream, q, k, v, q_cpu, k_cpu, v_cpu, mask_cpu,
                                         kernel_tflops)
        ok = ok and all(c.get("parity", {}).get("pass", True) for c in result["configs"].values()
                        if isinstance(c, dict) and "kernel" in c)

    if not args.no_mfma_ceiling:
        result["mfma_ceiling"] = mfma_ceiling(vsa, kernel_tflops)

    print(json.dumps(result), flush=True)
    return 0 if ok else 1


def mfma_ceiling(vsa, kernel_tflops, iters=200000):
    """What the matrix cores sustain on v_mfma_f32_32x32x16_bf16 when every
    compute unit runs it back to back (vsa_measure_mfma): on operands drawn
    like Q, K, V (bf16 N(0,1)), on the same beside softmax-shaped vector work
    on the other wave of each SIMD (the forward kernels' phase split), and on
    zero operands. The published peak assumes the top clock, which a long run
    keeps only on zero operands; the fractions say how far the kernel is from
    what this part sustains on data like its own."""
    vsa.vsa_measure_mfma("random", iters=iters // 4)  # out of the idle clock state
    out = {"unit": "TFLOP/s", "mfma": "v_mfma_f32_32x32x16_bf16", "iters": iters}
    for mode in ("random", "pingpong_softmax", "zero"):
        r = vsa.vsa_measure_mfma(mode, iters=iters)
        out[mode] = {"value": round(r["tflops"], 1), "clock_mhz": round(r["clock_mhz"])}
    out["kernel_frac_of_random"] = round(kernel_tflops / out["random"]["value"], 4)
    out["kernel_frac_of_pingpong_softmax"] = round(kernel_tflops / out["pingpong_softmax"]["value"], 4)
    return out


# The other workloads and tile shapes timed beside the headline (kernel
# scope unless noted): dense S=4k, the VSA-256 mask on 128x64 and 64x64 tiles
# natively and coalesced to 256-row tiles, the native Q64 masks.
CONFIGS = [
    ("dense 128x128", "dense_b1h8s4096d128", (128, 128), "kernel"),
    ("vsa256 128x64", "vsa256_fine_b1h24s32768d128_keep13", (128, 64), "kernel"),
    ("vsa256 64x64", "vsa256_fine_b1h24s32768d128_keep13", (64, 64), "kernel"),
    ("vsa256 128x64 coalesced", "vsa256_fine_b1h24s32768d128_keep13", (128, 64), "coalesce"),
    ("vsa256 64x64 coalesced", "vsa256_fine_b1h24s32768d128_keep13", (64, 64), "coalesce"),
    ("native64 64x64", "native64_b1h24s32768d128_cnt10to92", (64, 64), "kernel"),
]


def coalesced_rows(vsa, idx, cnt, bq, S):
    """Query-tile height the coalesced entry point runs for this CSR (the
    device makes the same pairing test level by level)."""
    run_bq, ri, rc = bq, idx, cnt
    while run_bq < 256 and S % 256 == 0:
        pi, pc, un = vsa.vsa_pair_q_tiles(ri, rc)
        if int(un.item()) != 0:
            break
        ri, rc, run_bq = pi, pc, run_bq * 2
    return run_bq


def time_configs(vsa, W, head_wl, head_tile, args, stream, q0, k0, v0, q0_cpu, k0_cpu, v0_cpu, mask0_cpu,
                 head_kernel_tflops):
    """Kernel time, sparse-aware TFLOP/s and (with the CPU leg) sampled parity
    of every entry of CONFIGS, each on its own synthetic inputs resident in
    HBM; the entry equal to the headline is skipped."""
    import torch

    out = {}
    dev = q0.device
    for label, wname, tile, scope in CONFIGS:
        wl = W.WORKLOADS[wname]
        if tile == head_tile and scope == "kernel" and wl.mask_kind == head_wl.mask_kind and \
                wl.mask_seed() == head_wl.mask_seed() and wl.seqlen == head_wl.seqlen:
            continue
        B, H, S, D = wl.batch, wl.heads, wl.seqlen, wl.head_dim
        same_inputs = (B, S, H, D) == tuple(q0_cpu.shape)
        if same_inputs:
            q, k, v, q_cpu, k_cpu, v_cpu = q0, k0, v0, q0_cpu, k0_cpu, v0_cpu
        else:
            q_cpu, k_cpu, v_cpu = wl.qkv()
            q, k, v = (t.to(dev) for t in (q_cpu, k_cpu, v_cpu))
        same_mask = wl.mask_kind == head_wl.mask_kind and wl.mask_seed() == head_wl.mask_seed() and \
            wl.logical_block == head_wl.logical_block and same_inputs
        mask_cpu = mask0_cpu if same_mask else wl.logical_mask()
        mask = torch.from_numpy(np.ascontiguousarray(mask_cpu).copy()).to(dev)
        lq, lkv = wl.logical_block
        bq, bkv = tile
        nq = S // bq
        ld = int(mask_cpu.sum(-1).max()) * (lkv // bkv)
        idx, cnt = vsa.vsa_mask_to_csr(mask, wl.logical_block, tile, ld, stream=stream)
        work = vsa.vsa_build_worklist(cnt, ld, segment=nq, stream=stream)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)

        def attention():
            if scope == "coalesce":
                vsa.vsa_attn_fwd_coalesced(q, k, v, idx, cnt, bq, bkv, wl.scale, o, lse, stream=stream)
            else:
                vsa.vsa_attn_fwd_worklist(q, k, v, idx, cnt, bq, bkv, work, wl.scale, o, lse, stream=stream)

        for _ in range(max(args.warmup, 3)):
            attention()
        events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e0, e1 in events:
            e0.record(stream)
            attention()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in events]))
        pairs = selected_pairs(idx, cnt, bq, bkv)
        tflops = 4.0 * D * pairs / (ms * 1e-3) / 1e12
        run_bq = coalesced_rows(vsa, idx, cnt, bq, S) if scope == "coalesce" else bq
        kname = kernel_name(run_bq, bkv, D, n_items=B * H * (S // run_bq))
        # HBM bytes per launch from the committed counters (a workload with the
        # headline's mask shares the headline workload's profiles)
        traffic = read_traffic(default_traffic_path(kname, wl.name, run_bq, bkv), kname)
        if traffic is None and same_mask:
            traffic = read_traffic(default_traffic_path(kname, head_wl.name, run_bq, bkv), kname)
        entry = {
            "workload": wl.name, "tile": f"{bq}x{bkv}",
            "runs_as": f"{run_bq}x{bkv}",
            "timed_scope": "vsa_attn_fwd_coalesced" if scope == "coalesce" else "vsa_attn_fwd_worklist",
            "kernel": kname,
            "kernel_ms": round(ms, 4), "tflops": round(tflops, 2),
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "selected_pairs": pairs,
            "vs_headline_kernel": round(tflops / head_kernel_tflops, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": kname},
        }
        if not args.no_cpu_baseline and args.config_cpu_seconds > 0:
            _, sample = cpu_baseline(wl, q_cpu, k_cpu, v_cpu, idx, cnt, bq, bkv, args.config_cpu_seconds)
            entry["parity"] = compare_rows(o, lse, sample, S, H)
        out[label] = entry
        print(f"[bench] {label}: {ms:.4f} ms {tflops:.1f} TFLOP/s"
              + (f" parity {'ok' if entry['parity']['pass'] else 'FAILED'}" if "parity" in entry else ""),
              file=sys.stderr, flush=True)
        del o, lse, idx, cnt, work, mask
        if not same_inputs:
            del q, k, v
        torch.cuda.empty_cache()
    out["relative_efficiency"] = {
        "basis": "kernel TFLOP/s of each entry over the headline kernel's (the FastVideo page's efficiency "
                 "relative to the 256-row arm)",
        **{lbl: e["vs_headline_kernel"] for lbl, e in out.items() if isinstance(e, dict) and "vs_headline_kernel" in e},
    }
    return out


def selected_pairs(idx, cnt, bq, bkv, kv_valid=None):
    """Selected (query, key) token pairs of a block CSR: block_q times the
    valid keys of every listed KV tile (block_kv each without partial tiles)."""
    import torch
    if kv_valid is None:
        return int(cnt.to(torch.int64).sum().item()) * bq * bkv
    ld = idx.shape[-1]
    listed = torch.arange(ld, device=idx.device) < cnt[..., None]
    keys = kv_valid.to(torch.int64)[idx.to(torch.int64).clamp(0, kv_valid.numel() - 1)]
    return int((keys * listed).sum().item()) * bq


def time_backward(vsa, q, k, v, o, lse, idx, cnt, bq, bkv, scale, D, pairs, steps, stream, kv_valid=None,
                  clock_seconds=0.0):
    """Backward leg: the Q-direction CSR plus dQ, dK, dV of this workload,
    timed like the forward (HIP events on the launch stream). Throughput uses
    the usual 10*D flops per selected pair (QK^T, dO V^T, P^T dO, dS K,
    dS^T Q); the kernels recompute QK^T and dO V^T once more (14*D executed).
    With clock_seconds > 0 the gfx clock and socket power are sampled while
    backward steps run back to back, as for the forward."""
    import torch

    B, S, H, _ = q.shape
    nkv = S // bkv
    g = torch.Generator(device="cpu").manual_seed(4242)
    dout = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(q.device)
    q_idx = torch.empty((B, H, nkv, S // bq), dtype=torch.int32, device=q.device)
    q_cnt = torch.empty((B, H, nkv), dtype=torch.int32, device=q.device)
    grads = [torch.empty_like(q) for _ in range(3)]

    def run():
        vsa.vsa_csr_transpose(idx, cnt, nkv, S // bq, q_idx, q_cnt, stream=stream)
        vsa.vsa_attn_bwd(q, k, v, o, lse, dout, idx, cnt, q_idx, q_cnt, bq, bkv, scale, *grads, stream=stream,
                         kv_valid=kv_valid)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = 10.0 * D * pairs / (ms * 1e-3) / 1e12
    clock = sample_clock(run, clock_seconds) if clock_seconds > 0 else None
    return {"ms": round(ms, 4), "tflops": round(tflops, 2), "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
            "flops_per_pair": f"10*D={10 * D}", "scope": "vsa_csr_transpose + vsa_attn_bwd (dQ with D and LSE, then dK/dV)",
            "clock": clock}


IW_ITEMS_PER_CU = 8  # the library's switch to the independent-wave kernel


def compute_units():
    """Compute units of GPU 0 (MI355X's 256 when no GPU is visible)."""
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.get_device_properties(0).multi_processor_count
    except Exception:
        pass
    return 256


def kernel_name(bq, bkv, d, partial=False, n_items=None, entry=False):
    """Name of the forward kernel the library dispatches for this tile shape
    and number of work items (the last template argument: built for partial
    tiles); entry: through vsa_attn_fwd, which splits the lists of few 64-row
    items over the independent-wave kernel."""
    p = "true" if partial else "false"
    if bq == 256:
        return f"vsa_fwd_pp_kernel<{bkv},{d},{p}>"
    many = n_items is not None and n_items >= IW_ITEMS_PER_CU * compute_units()
    if many or (entry and bq == 64):
        return f"vsa_fwd_iw_kernel<{bq},{d},{p}>"
    if bq == 128:
        return f"vsa_fwd_2t_kernel<{d},{p}>" if bkv == 128 else f"vsa_fwd_2s_kernel<{d},{p}>"
    return f"vsa_fwd_4s_kernel<{d},{p}>"


CSRC = os.path.join(ROOT, "block_sparse_attention_flashattention_amd", "csrc")


def kernel_source_hash(kname):
    """sha256 over the sources a forward kernel is compiled from: its own
    file, the dispatcher and the headers they include."""
    import hashlib
    own = {"vsa_fwd_pp_kernel": "attn_fwd_pp.hip", "vsa_fwd_2s_kernel": "attn_fwd_2s.hip",
           "vsa_fwd_4s_kernel": "attn_fwd_4s.hip", "vsa_fwd_iw_kernel": "attn_fwd_iw.hip",
           "vsa_fwd_2t_kernel": "attn_fwd_2t.hip"}[kname.split("<")[0]]
    h = hashlib.sha256()
    for name in sorted([own, "attn_fwd.hip", "wave_engine.h", "device_common.h", "vsa_internal.h"]):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def default_traffic_path(kname, workload, bq, bkv):
    stem = kname.split("<")[0] + ("_partial" if kname.endswith("true>") else "")
    return os.path.join(ROOT, "profiles", f"traffic_{stem}_{bq}x{bkv}_{workload}.json")


def read_traffic(path, kname):
    """HBM bytes per launch from a traffic JSON, or None if it is missing or
    was measured on other kernel sources."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash(kname):
        return None
    return t.get("bytes_per_launch")


def sample_clock(step, seconds):
    """Run steps back to back for about `seconds` while amd-smi reads the gfx
    clock of every XCD and the socket power once, half-way through. The
    socket power shows whether the step runs at the board's power limit
    (1,400 W on MI355X), where its time follows its energy per step."""
    import subprocess
    import threading

    import torch
    box = {}

    def query():
        try:
            r = subprocess.run(["amd-smi", "metric", "--clock", "--power", "--json"], capture_output=True,
                               text=True, timeout=30)
            d = json.loads(r.stdout)
            d = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else d[0]
            clk = d["clock"]
            box["mhz"] = [float(clk[k]["clk"]["value"]) for k in sorted(clk) if k.startswith("gfx_")]
            pw = (d.get("power") or {}).get("socket_power")
            if isinstance(pw, dict) and isinstance(pw.get("value"), (int, float)):
                box["watts"] = float(pw["value"])
        except Exception as e:  # best effort: the tool may be missing or print another layout
            box["error"] = f"{type(e).__name__}: {e}"[:200]

    t_end = time.perf_counter() + seconds
    th = None
    while True:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        now = time.perf_counter()
        if th is None and now > t_end - seconds / 2:
            th = threading.Thread(target=query)
            th.start()
        if now > t_end and th is not None and not th.is_alive():
            break
        if now > t_end + 40:
            break
    if "mhz" not in box:
        return {"gfx_mhz_mean": None, "error": box.get("error", "no sample")}
    mhz = box["mhz"]
    return {"gfx_mhz_mean": round(sum(mhz) / len(mhz), 1), "gfx_mhz": mhz, "socket_power_w": box.get("watts"),
            "source": "amd-smi metric --clock --power, sampled while steps ran back to back"}


O_MAX_ABS, O_MEAN_ABS, LSE_REL = 2e-2, 2e-3, 1e-3  # forward tolerances (bf16 O, fp32 LSE)


def oracle_threads():
    """Host threads for the oracle: OMP_NUM_THREADS if set, else every CPU."""
    return int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)


def cpu_baseline(wl, q, k, v, idx, cnt, bq, bkv, seconds, kv_valid=None):
    """Time the CPU oracle on a bounded sample of whole query tiles of this
    workload (a fixed pseudo-random order, sized to about `seconds`); returns
    the timing and the sample (rows and the oracle's O and LSE for them)."""
    import oracle

    threads = oracle_threads()
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    B, S, H, D = q.shape
    nq = S // bq

    def rows_for(n_tiles):
        # whole query tiles, spread over heads, in a fixed pseudo-random order
        order = np.random.default_rng(0).permutation(B * H * nq)[:n_tiles]
        rows = []
        for item in order:
            bh, p = divmod(int(item), nq)
            rows.append(bh * S + p * bq + np.arange(bq))
        return np.concatenate(rows).astype(np.int64), order

    def run(n_tiles):
        rows, items = rows_for(n_tiles)
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attn_rows(q, k, v, idx_h, cnt_h, bq, bkv, wl.scale, rows, threads, kv_valid=kv_valid)
        dt = time.perf_counter() - t0
        if kv_valid is None:
            flops = 4.0 * D * float(cnt_h.reshape(-1)[items].sum()) * bq * bkv
        else:
            flat_idx, flat_cnt = idx_h.reshape(-1, idx_h.shape[-1]), cnt_h.reshape(-1)
            flops = 4.0 * D * bq * float(sum(kv_valid[flat_idx[i, :flat_cnt[i]]].sum() for i in items))
        return dt, flops, rows, o_ref, lse_ref

    probe = max(1, threads // 4)
    dt, fl, *_ = run(probe)
    n_tiles = max(1, min(B * H * nq, int(probe * seconds / max(dt, 1e-3))))
    dt, fl, rows, o_ref, lse_ref = run(n_tiles)
    base = {
        "value": round(fl / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_tiles} of {B * H * nq} query tiles ({rows.size} rows, {fl:.3e} sparse-aware flops) "
                  f"in {dt:.1f} s",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
    }
    return base, {"rows": rows, "o": o_ref, "lse": lse_ref, "tiles": n_tiles}


def compare_rows(o_gpu, lse_gpu, sample, S, H):
    """GPU O [B,S,H,D] / LSE [B,H,S] at the sample's flat rows (b*H + h)*S + i
    against the oracle's: max-abs and mean-abs of O, relative LSE error (floor
    1), and the FastVideo page's gate max(1e-2, 8 x the bf16 rounding floor of
    the reference)."""
    import torch

    rows = sample["rows"]
    i, h, b = rows % S, (rows // S) % H, rows // (S * H)
    ti, th, tb = (torch.from_numpy(x).to(o_gpu.device) for x in (i, h, b))
    og = o_gpu[tb, ti, th].float().cpu().numpy()
    lg = lse_gpu[tb, th, ti].cpu().numpy()
    o_ref, lse_ref = sample["o"], sample["lse"]
    fin = np.isfinite(lse_ref)
    d = np.abs(og - o_ref)
    max_abs, mean_abs = float(d.max()), float(d.mean())
    lse_rel = float((np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))).max()) if fin.any() else 0.0
    ref32 = torch.from_numpy(np.ascontiguousarray(o_ref, dtype=np.float32))
    floor = float((ref32 - ref32.to(torch.bfloat16).float()).abs().max())
    gate = max(1e-2, 8.0 * floor)
    finite_ok = bool(np.array_equal(fin, np.isfinite(lg)) and np.isfinite(og).all())
    ok = finite_ok and max_abs <= O_MAX_ABS and mean_abs <= O_MEAN_ABS and lse_rel <= LSE_REL and max_abs <= gate
    return {
        "rows": int(rows.size), "query_tiles": int(sample["tiles"]),
        "max_abs_o": max_abs, "mean_abs_o": mean_abs, "lse_rel": lse_rel,
        "page_gate": round(gate, 6), "tolerances": {"max_abs_o": O_MAX_ABS, "mean_abs_o": O_MEAN_ABS,
                                                    "lse_rel": LSE_REL},
        "pass": bool(ok),
    }


def cpu_model():
    """Model name of the host CPU (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    sys.exit(main())
