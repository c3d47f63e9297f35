"""vsa_attn_fwd_noalloc (the entry point for callers that cannot allocate)
through the C ABI: the same result as vsa_attn_fwd
(within the forward tolerances, bitwise where both split a list the same
way), every row also against the oracle, on two calls in a row of which the
second is smaller (the fixed scratch array keeps the first call's bytes)."""

import ctypes
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_REL = 1e-3


def say(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flashattention_amd as m

    return m.load_library()


def _call(fn, t, o, lse):
    B, S, H, D = t["q"].shape
    rc = fn(t["qd"].data_ptr(), t["kd"].data_ptr(), t["vd"].data_ptr(), t["idxd"].data_ptr(), t["cntd"].data_ptr(),
            None, B, S, H, D, t["idx"].shape[3], t["bq"], t["bkv"], ctypes.c_float(t["scale"]), o.data_ptr(),
            lse.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, rc


def _compare(o, lse, o2, l2, label):
    d = (o.float() - o2.float()).abs()
    fin = torch.isfinite(l2)
    assert torch.equal(fin, torch.isfinite(lse))
    lrel = float(((lse[fin] - l2[fin]).abs() / l2[fin].abs().clamp_min(1.0)).max())
    say(f"{label}: noalloc vs vsa_attn_fwd max|dO|={d.max().item():.3e} mean|dO|={d.mean().item():.3e} "
        f"LSE rel={lrel:.3e}")
    assert d.max().item() <= O_MAX_ABS and d.mean().item() <= O_MEAN_ABS and lrel <= LSE_REL


def _against_oracle(t, o, lse, label):
    B, S, H, D = t["q"].shape
    o_ref, lse_ref = oracle.attn_full(t["q"], t["k"], t["v"], t["idx"], t["cnt"], t["bq"], t["bkv"], t["scale"])
    og = o.float().cpu().numpy()
    d = np.abs(og - o_ref)
    lg = lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lg))
    lrel = float((np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))).max())
    say(f"{label}: noalloc vs oracle max|dO|={d.max():.3e} mean|dO|={d.mean():.3e} LSE rel={lrel:.3e}")
    assert d.max() <= O_MAX_ABS and d.mean() <= O_MEAN_ABS and lrel <= LSE_REL


def _case(B, H, S, D, bq, bkv, lo, hi, seed):
    q, k, v = W.qkv(B, S, H, D, seed=seed)
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, lo, hi, seed=seed + 1)
    cnt[0, 0, 0] = 0  # an empty query tile
    return dict(q=q, k=k, v=v, idx=idx, cnt=cnt, bq=bq, bkv=bkv, scale=1.0 / math.sqrt(D),
                qd=q.cuda(), kd=k.cuda(), vd=v.cuda(), idxd=torch.from_numpy(idx).cuda(),
                cntd=torch.from_numpy(cnt).cuda())


def test_noalloc_matches_vsa_attn_fwd_on_two_calls(lib):
    # first call: 32 work items of 256 rows (vsa_attn_fwd splits each list in
    # four; the array holds the partial states of two parts), then a smaller
    # one: 64 items of 64 rows, split in four by both entry points
    cases = [("256x128 D128 32 items", _case(1, 1, 8192, 128, 256, 128, 1, 64, 31)),
             ("64x64 D64 64 items", _case(1, 2, 2048, 64, 64, 64, 0, 32, 32))]
    for label, t in cases:
        say(label)
        o = torch.full_like(t["qd"], 7.0)
        lse = torch.full(t["q"].shape[:1] + (t["q"].shape[2], t["q"].shape[1]), 7.0, dtype=torch.float32,
                         device="cuda")
        o2, l2 = torch.empty_like(o), torch.empty_like(lse)
        _call(lib.vsa_attn_fwd_noalloc, t, o, lse)
        _call(lib.vsa_attn_fwd, t, o2, l2)
        torch.cuda.synchronize()
        _compare(o, lse, o2, l2, label)
        _against_oracle(t, o, lse, label)
        if t["bq"] == 64:  # same number of parts on both paths: the same kernel work, bit for bit
            assert torch.equal(o, o2) and torch.equal(lse, l2)
        # a repeated call must give the same bits (counters left at zero)
        o3, l3 = torch.empty_like(o), torch.empty_like(lse)
        _call(lib.vsa_attn_fwd_noalloc, t, o3, l3)
        torch.cuda.synchronize()
        assert torch.equal(o, o3) and torch.equal(lse, l3)


def test_noalloc_many_items_unsplit(lib):
    """Many 128-row work items (no split): bitwise equal to vsa_attn_fwd."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = 2048
    H = max(1, -(-8 * cus * 128 // S))
    t = _case(1, H, S, 64, 128, 64, 0, 8, 33)
    o = torch.empty_like(t["qd"])
    lse = torch.empty((1, H, S), dtype=torch.float32, device="cuda")
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    _call(lib.vsa_attn_fwd_noalloc, t, o, lse)
    _call(lib.vsa_attn_fwd, t, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
