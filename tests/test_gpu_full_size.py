"""GPU parity at the full sizes of the workloads, on every output element.

The oracle runs once per workload over all rows (module fixtures). It is
bitwise invariant under the tile shape of an exact-expanded mask (pinned in
tests/test_oracle_pins.py), so the one VSA-256 reference checks that mask at
256x128, 128x64 and 64x64 and through the paired and coalesced schedules.

Tolerances, over all B*S*H*D elements of O (bf16, compared after conversion
to fp32) and all B*H*S rows of LSE: max |dO| <= 2e-2, mean |dO| <= 2e-3,
|dLSE| <= 1e-3 * max(1, |LSE|); and the FastVideo page's own gate, max |dO|
within max(1e-2, 8 x the largest bf16 rounding error of the reference).
"""

import os
import time

import numpy as np
import pytest
import torch

import oracle
from oracle import frontend as ofront
import workloads as W

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_REL = 1e-3


def say(msg):
    line = f"[gpu-full] {msg}"
    print(line, flush=True)
    path = os.environ.get("VSA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


@pytest.fixture(scope="module")
def vsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flashattention_amd as m

    m.load_library()
    return m


def dev(x):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.array(x, copy=True, order="C"))  # a writable copy (cached oracle arrays are read-only)
    return x.contiguous().to("cuda")


def check_all(o, lse, o_ref, lse_ref, label):
    """Every element of O [B,S,H,D] and every row of LSE [B,H,S] against the
    oracle's fp32 O and LSE."""
    og = o.float().cpu()
    lg = lse.cpu()
    orf = torch.from_numpy(o_ref)
    lrf = torch.from_numpy(lse_ref)
    fin = torch.isfinite(lrf)
    assert torch.equal(fin, torch.isfinite(lg)), f"{label}: LSE finiteness differs"
    assert torch.all(lg[~fin] == -float("inf")), f"{label}: empty rows must have LSE=-inf"
    empty_rows = (~fin).permute(0, 2, 1)  # [B, S, H]
    assert torch.all(og[empty_rows] == 0), f"{label}: empty rows must have O=0"
    assert torch.isfinite(og).all(), f"{label}: non-finite O"
    d = (og - orf).abs_()
    max_abs, mean_abs = float(d.max()), float(d.mean(dtype=torch.float64))
    del d
    lse_err = float(((lg[fin] - lrf[fin]).abs() / lrf[fin].abs().clamp_min(1.0)).max()) if bool(fin.any()) else 0.0
    floor = float((orf - orf.to(torch.bfloat16).float()).abs_().max())
    page_limit = max(1e-2, 8.0 * floor)
    say(f"{label}: all {og.numel()} elements: max|dO|={max_abs:.3e} mean|dO|={mean_abs:.3e} LSE rel={lse_err:.3e} "
        f"(page gate {page_limit:.3e})")
    assert max_abs <= O_MAX_ABS, f"{label}: max |dO| {max_abs}"
    assert max_abs <= page_limit, f"{label}: max |dO| {max_abs} above the page's gate {page_limit}"
    assert mean_abs <= O_MEAN_ABS, f"{label}: mean |dO| {mean_abs}"
    assert lse_err <= LSE_REL, f"{label}: LSE rel err {lse_err}"


class Reference:
    """One workload's inputs on the host and the device, its logical mask on
    the device, and the oracle over every row at one tile shape."""

    def __init__(self, wl, tile, ld):
        t0 = time.perf_counter()
        self.wl = wl
        self.q, self.k, self.v = wl.qkv()
        self.mask_h = wl.logical_mask()
        idx, cnt, ovf = ofront.mask_to_csr(self.mask_h, wl.logical_block, tile, ld)
        assert not ovf
        self.o, self.lse = oracle.attn_full(self.q, self.k, self.v, idx, cnt, tile[0], tile[1], wl.scale)
        say(f"oracle {wl.name} at {tile[0]}x{tile[1]}, every row: {time.perf_counter() - t0:.1f} s "
            f"on {os.cpu_count()} host CPUs")
        self.qd, self.kd, self.vd = dev(self.q), dev(self.k), dev(self.v)
        self.mask = dev(self.mask_h)

    def csr(self, vsa, tile, ld):
        return vsa.vsa_mask_to_csr(self.mask, self.wl.logical_block, tile, ld)


@pytest.fixture(scope="module")
def dense_ref(vsa):
    return Reference(W.DENSE, (128, 128), 32)


@pytest.fixture(scope="module")
def vsa256_ref(vsa):
    return Reference(W.VSA256, (256, 128), 26)


@pytest.fixture(scope="module")
def vsa256_d64_ref(vsa):
    return Reference(W.VSA256_D64, (256, 128), 26)


@pytest.fixture(scope="module")
def native64_ref(vsa):
    return Reference(W.NATIVE64, (64, 64), 92)


@pytest.mark.parametrize("tile", [(128, 128), (256, 128)], ids=["128x128", "256x128_split"])
def test_dense_every_element(vsa, dense_ref, tile):
    """Dense S=4k: 128-row tiles (256 work items, the whole-tile two-stream
    kernel) and 256-row tiles (128 items, so each list is split over two
    workgroups and the partial rows merged)."""
    r = dense_ref
    idx, cnt = r.csr(vsa, tile, 4096 // tile[1])
    o, lse = vsa.vsa_attn_fwd(r.qd, r.kd, r.vd, idx, cnt, tile[0], tile[1], r.wl.scale)
    torch.cuda.synchronize()
    check_all(o, lse, r.o, r.lse, f"dense {tile[0]}x{tile[1]}")


VSA256_RUNS = [
    # label, entry point, tile the CSR is built at, idx_ld, tile whose plain kernel it must equal bitwise
    ("256x128", "fwd", (256, 128), 26, None),
    ("256x128 worklist", "worklist", (256, 128), 26, None),
    ("128x64", "fwd", (128, 64), 52, None),
    ("64x64", "fwd", (64, 64), 52, None),
    ("64x64 paired", "paired", (64, 64), 52, (128, 64)),
    ("128x64 coalesced", "coalesced", (128, 64), 52, (256, 64)),
    ("64x64 coalesced", "coalesced", (64, 64), 52, (256, 64)),
]


@pytest.mark.parametrize("label,entry,tile,ld,equal_to", VSA256_RUNS, ids=[c[0] for c in VSA256_RUNS])
def test_vsa256_every_element(vsa, vsa256_ref, label, entry, tile, ld, equal_to):
    """The VSA-256 mask (B1 H24 S32768 D128, keep 13 of 128) at every tile
    shape and schedule, every element against the one oracle run. The paired
    and coalesced entry points must also equal, bit for bit, the kernel of
    the tile shape they coalesce to."""
    r = vsa256_ref
    idx, cnt = r.csr(vsa, tile, ld)
    say(f"vsa256 {label}: kernel")
    if entry == "fwd":
        o, lse = vsa.vsa_attn_fwd(r.qd, r.kd, r.vd, idx, cnt, tile[0], tile[1], r.wl.scale)
    elif entry == "worklist":
        work = vsa.vsa_build_worklist(cnt, ld, segment=r.wl.seqlen // tile[0])
        o, lse = vsa.vsa_attn_fwd_worklist(r.qd, r.kd, r.vd, idx, cnt, tile[0], tile[1], work, r.wl.scale)
    elif entry == "paired":
        o, lse = vsa.vsa_attn_fwd_paired(r.qd, r.kd, r.vd, idx, cnt, tile[1], r.wl.scale)
    else:
        o, lse = vsa.vsa_attn_fwd_coalesced(r.qd, r.kd, r.vd, idx, cnt, tile[0], tile[1], r.wl.scale)
    torch.cuda.synchronize()
    check_all(o, lse, r.o, r.lse, f"vsa256 {label}")
    if equal_to is not None:
        idx2, cnt2 = r.csr(vsa, equal_to, ld)
        o2, l2 = vsa.vsa_attn_fwd(r.qd, r.kd, r.vd, idx2, cnt2, equal_to[0], equal_to[1], r.wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2), f"{label}: not the {equal_to} kernel's result"
        del o2, l2
    del o, lse
    torch.cuda.empty_cache()


def test_vsa256_cross_shape_agreement(vsa, vsa256_ref):
    """The FastVideo page's cross-shape check (max-abs of the 128x64 and 64x64
    arms against the 256-row arm on one exact-expanded mask), GPU against GPU."""
    r = vsa256_ref
    idx, cnt = r.csr(vsa, (256, 128), 26)
    o0, l0 = vsa.vsa_attn_fwd(r.qd, r.kd, r.vd, idx, cnt, 256, 128, r.wl.scale)
    for tile in ((128, 64), (64, 64)):
        idx, cnt = r.csr(vsa, tile, 52)
        o1, l1 = vsa.vsa_attn_fwd(r.qd, r.kd, r.vd, idx, cnt, tile[0], tile[1], r.wl.scale)
        torch.cuda.synchronize()
        d = (o1.float() - o0.float()).abs()
        lrel = ((l1 - l0).abs() / l0.abs().clamp_min(1.0)).max().item()
        say(f"cross-shape {tile}: max|dO|={d.max().item():.3e} mean|dO|={d.mean().item():.3e} LSE rel={lrel:.3e}")
        assert d.max().item() <= O_MAX_ABS and d.mean().item() <= O_MEAN_ABS and lrel <= LSE_REL
        del o1, l1, d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tile,ld", [((256, 128), 26), ((128, 64), 52), ((64, 64), 52)],
                         ids=["256x128", "128x64", "64x64"])
def test_vsa256_head_dim_64_every_element(vsa, vsa256_d64_ref, tile, ld):
    """The VSA-256 mask at head_dim 64 (B1 H48 S32768): the 256-row, 128-row
    and 64-row kernels built for head_dim 64, every element against one
    oracle run."""
    r = vsa256_d64_ref
    idx, cnt = r.csr(vsa, tile, ld)
    o, lse = vsa.vsa_attn_fwd(r.qd, r.kd, r.vd, idx, cnt, tile[0], tile[1], r.wl.scale)
    torch.cuda.synchronize()
    check_all(o, lse, r.o, r.lse, f"vsa256 d64 {tile[0]}x{tile[1]}")
    del o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("entry", ["fwd", "worklist"])
def test_native64_every_element(vsa, native64_ref, entry):
    """Native Q64/KV64 masks (512x512 tile grid, 10..92 tiles per row): the
    count-sorted work list and the independent-wave 64-row kernel."""
    r = native64_ref
    idx, cnt = r.csr(vsa, (64, 64), 92)
    if entry == "fwd":
        o, lse = vsa.vsa_attn_fwd(r.qd, r.kd, r.vd, idx, cnt, 64, 64, r.wl.scale)
    else:
        work = vsa.vsa_build_worklist(cnt, 92, segment=r.wl.seqlen // 64)
        o, lse = vsa.vsa_attn_fwd_worklist(r.qd, r.kd, r.vd, idx, cnt, 64, 64, work, r.wl.scale)
    torch.cuda.synchronize()
    check_all(o, lse, r.o, r.lse, f"native64 64x64 {entry}")
    del o, lse
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def ragged_ref(vsa):
    """VSA-256 with ragged logical KV blocks (valid tokens per 256-token block
    uniform in [0, 256], 30% full): the oracle over every row at 256x128."""
    wl = W.VSA256
    t0 = time.perf_counter()
    q, k, v = wl.qkv()
    mask = wl.logical_mask()
    vbs = W.ragged_block_sizes(wl.seqlen // 256, 256, seed=2026)
    vbs[:3] = [0, 128, 1]
    idx, cnt, _ = ofront.mask_to_csr(mask, wl.logical_block, (256, 128), 26)
    val = ofront.expand_valid(vbs, 256, 128)
    o, lse = oracle.attn_full(q, k, v, idx, cnt, 256, 128, wl.scale, kv_valid=val)
    say(f"oracle ragged vsa256 at 256x128, every row: {time.perf_counter() - t0:.1f} s")
    return dict(qd=dev(q), kd=dev(k), vd=dev(v), mask=dev(mask), mask_h=mask, vbs=dev(vbs), vbs_h=vbs, o=o,
                lse=lse)


RAGGED_RUNS = [((256, 128), 26, False), ((256, 128), 26, True), ((128, 64), 52, True), ((64, 64), 52, True)]


@pytest.mark.parametrize("tile,ld,drop", RAGGED_RUNS,
                         ids=[f"{t[0]}x{t[1]}{'_dropped' if d else ''}" for t, _, d in RAGGED_RUNS])
def test_vsa256_ragged_every_element(vsa, ragged_ref, tile, ld, drop):
    """Partial KV tiles at full size: the valid counts per physical tile are
    expanded on the device from the per-block counts; every element against
    the one oracle run (the token-level selection is the same at every tile
    shape). With `drop`, the front-end leaves tiles without a valid key out of
    the lists (their counts shrink; the CSR is bit-exact against the
    oracle's front-end)."""
    r = ragged_ref
    val = vsa.vsa_expand_valid(r["vbs"], 256, tile[1])
    idx, cnt = vsa.vsa_mask_to_csr(r["mask"], (256, 256), tile, ld, kv_valid=val if drop else None)
    if drop:
        ridx, rcnt, _ = ofront.mask_to_csr(r["mask_h"], (256, 256), tile, ld,
                                           kv_valid=ofront.expand_valid(r["vbs_h"], 256, tile[1]))
        torch.cuda.synchronize()
        assert np.array_equal(cnt.cpu().numpy(), rcnt)
        listed = np.arange(ld)[None, None, None, :] < rcnt[..., None]
        assert np.array_equal(np.where(listed, idx.cpu().numpy(), -1), np.where(listed, ridx, -1))
        full = ofront.mask_to_csr(r["mask_h"], (256, 256), tile, ld)[1]
        say(f"ragged {tile}: {int(full.sum() - rcnt.sum())} of {int(full.sum())} listed tiles dropped")
    o, lse = vsa.vsa_attn_fwd(r["qd"], r["kd"], r["vd"], idx, cnt, tile[0], tile[1], W.VSA256.scale, kv_valid=val)
    torch.cuda.synchronize()
    check_all(o, lse, r["o"], r["lse"], f"ragged vsa256 {tile[0]}x{tile[1]}{' dropped' if drop else ''}")
    del o, lse
    torch.cuda.empty_cache()
