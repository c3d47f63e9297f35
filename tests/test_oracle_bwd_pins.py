"""Pins for the CPU oracle's backward pass (dQ, dK, dV), without a GPU.

Checked against PyTorch float64 autograd through a masked softmax attention
built from an explicitly materialised token mask, closed forms, invariants
of the softmax derivative, and planted mistakes.
"""

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import frontend
from workloads import bf16_bits, qkv, random_csr

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _f64(t):
    return torch.from_numpy((bf16_bits(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def _token_mask(idx, cnt, S, bq, bkv, kv_valid=None):
    B, H, NQ, _ = idx.shape
    m = np.zeros((B, H, S, S), dtype=bool)
    for b in range(B):
        for h in range(H):
            for p in range(NQ):
                for e in range(int(cnt[b, h, p])):
                    t = int(idx[b, h, p, e])
                    n = bkv if kv_valid is None else int(kv_valid[t])
                    m[b, h, p * bq:(p + 1) * bq, t * bkv:t * bkv + n] = True
    return torch.from_numpy(m)


def _autograd(q, k, v, do, idx, cnt, bq, bkv, scale, kv_valid=None):
    """float64 reference gradients, [B, S, H, D] each."""
    qf, kf, vf, df = (_f64(t).permute(0, 2, 1, 3).contiguous() for t in (q, k, v, do))  # [B,H,S,D]
    qf.requires_grad_(True)
    kf.requires_grad_(True)
    vf.requires_grad_(True)
    B, H, S, D = qf.shape
    mask = _token_mask(idx, cnt, S, bq, bkv, kv_valid)
    s = torch.matmul(qf, kf.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    mx = s.amax(-1, keepdim=True)
    mx = torch.where(torch.isfinite(mx), mx, torch.zeros_like(mx)).detach()
    e = torch.exp(s - mx) * mask
    l = e.sum(-1, keepdim=True)
    p = e / torch.where(l > 0, l, torch.ones_like(l))
    o = torch.matmul(p, vf)
    o.backward(df)
    g = lambda t: t.grad.permute(0, 2, 1, 3).numpy()  # noqa: E731
    return g(qf), g(kf), g(vf)


CASES = [
    # B, H, S, D, block_q, block_kv, count range, partial tiles
    (1, 2, 128, 16, 32, 16, (0, 5), False),
    (2, 1, 128, 32, 16, 32, (1, 4), False),
    (1, 2, 256, 16, 64, 32, (0, 8), True),
    (1, 1, 192, 64, 64, 64, (1, 3), True),
]


@pytest.mark.parametrize("B,H,S,D,bq,bkv,cr,partial", CASES)
def test_backward_matches_float64_autograd(B, H, S, D, bq, bkv, cr, partial):
    q, k, v = qkv(B, S, H, D, seed=S + D + 11)
    do = qkv(B, S, H, D, seed=S + D + 12)[0]
    nq, nkv = S // bq, S // bkv
    idx, cnt = random_csr(B, H, nq, nkv, nkv, cr[0], min(cr[1], nkv), seed=S + bq + 13)
    val = None
    if partial:
        val = np.random.default_rng(S).integers(0, bkv + 1, size=nkv).astype(np.int32)
        val[0] = 0
    scale = D ** -0.5
    dq, dk, dv = oracle.bwd_full(q, k, v, do, idx, cnt, bq, bkv, scale, kv_valid=val)
    rq, rk, rv = _autograd(q, k, v, do, idx, cnt, bq, bkv, scale, val)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() < 2e-5 * max(1.0, np.abs(ref).max())


def test_zero_output_gradient_gives_zero_gradients():
    B, H, S, D, bq, bkv = 1, 2, 128, 16, 32, 32
    q, k, v = qkv(B, S, H, D, seed=5)
    do = torch.zeros_like(q)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 4, seed=6)
    for g in oracle.bwd_full(q, k, v, do, idx, cnt, bq, bkv, 0.3):
        assert np.all(g == 0.0)


def test_uniform_attention_closed_form():
    """K = 0: P_ij = 1/|A(i)|, so dQ = 0 exactly and dV_j = sum over the rows
    that see j of dO_i / |A(i)|."""
    B, H, S, D, bq, bkv = 1, 1, 128, 16, 32, 16
    q, _, v = qkv(B, S, H, D, seed=7)
    k = torch.zeros_like(q)
    do = qkv(B, S, H, D, seed=8)[0]
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 5, seed=9)
    dq, dk, dv = oracle.bwd_full(q, k, v, do, idx, cnt, bq, bkv, 0.5)
    assert np.all(dq == 0.0)
    mask = _token_mask(idx, cnt, S, bq, bkv).numpy()[0, 0]
    dof = _f64(do).numpy()[0, :, 0]
    expect = (mask / mask.sum(1, keepdims=True)).T @ dof
    assert np.abs(dv[0, :, 0] - expect).max() < 1e-5


def test_key_gradients_sum_to_zero_per_head():
    """Each softmax row's dS sums to zero, so sum_j dK_j = 0 for every head."""
    B, H, S, D, bq, bkv = 2, 2, 256, 32, 64, 32
    q, k, v = qkv(B, S, H, D, seed=21)
    do = qkv(B, S, H, D, seed=22)[0]
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 0, 8, seed=23)
    _, dk, _ = oracle.bwd_full(q, k, v, do, idx, cnt, bq, bkv, 0.2)
    assert np.abs(dk.sum(1)).max() < 1e-4 * np.abs(dk).max()


def test_row_subsets_match_full_and_tile_shapes_agree_bitwise():
    from workloads import anchor_uniform_mask

    B, H, S, D = 1, 1, 512, 32
    q, k, v = qkv(B, S, H, D, seed=31)
    do = qkv(B, S, H, D, seed=32)[0]
    base = anchor_uniform_mask(H, S // 256, S // 256, 1, seed=33)[None]
    vbs = np.array([256, 150], dtype=np.int32)
    res = []
    for shape in ((256, 256), (128, 64), (64, 64)):
        idx, cnt, _ = frontend.mask_to_csr(base, (256, 256), shape, S // shape[1])
        val = frontend.expand_valid(vbs, 256, shape[1])
        res.append(oracle.bwd_full(q, k, v, do, idx, cnt, shape[0], shape[1], 0.125, kv_valid=val))
        rows = np.array([0, 77, 300, 511], dtype=np.int64)
        dq_r = oracle.bwd_dq_rows(q, k, v, do, idx, cnt, shape[0], shape[1], 0.125, rows, kv_valid=val)
        dk_r, dv_r = oracle.bwd_dkv_rows(q, k, v, do, idx, cnt, shape[0], shape[1], 0.125, rows, kv_valid=val)
        assert np.array_equal(dq_r, res[-1][0][0, rows, 0])
        assert np.array_equal(dk_r, res[-1][1][0, rows, 0]) and np.array_equal(dv_r, res[-1][2][0, rows, 0])
    for other in res[1:]:
        for a, b in zip(other, res[0]):
            assert np.array_equal(a, b)


MUTATIONS = {
    "dq_without_D": ("const float ds = s[j] * (dp - di);", "const float ds = s[j] * dp;"),
    "dk_without_D": ("const float ds = pij * (dp - di);", "const float ds = pij * dp;"),
    "dk_unscaled": ("for (int d = 0; d < D; ++d) dkrow[d] *= scale;", ""),
    "dv_without_p": ("for (int d = 0; d < D; ++d) dvrow[d] += pij * bf16_to_f32(drow[d]);",
                     "for (int d = 0; d < D; ++d) dvrow[d] += bf16_to_f32(drow[d]);"),
    "dq_uses_v": ("for (int d = 0; d < D; ++d) dqrow[d] += ds * bf16_to_f32(krow[d]);",
                  "for (int d = 0; d < D; ++d) dqrow[d] += ds * bf16_to_f32(vrow[d]);"),
    "dkv_prob_of_wrong_key": ("const float pij = s[j];", "const float pij = s[i];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_backward_mistake_is_caught(tmp_path, name, monkeypatch):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "vsa_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, name  # planted in every backward routine that has the line
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", str(path), "-o",
                    str(so), "-lm"], check=True)
    import ctypes

    lib = ctypes.CDLL(str(so))
    base = oracle._load()
    for fn in ("vsa_oracle_bwd_dq_rows", "vsa_oracle_bwd_dkv_rows", "vsa_oracle_bwd_full"):
        getattr(lib, fn).argtypes = getattr(base, fn).argtypes
        getattr(lib, fn).restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", lib)
    B, H, S, D, bq, bkv = 1, 2, 128, 16, 32, 16
    q, k, v = qkv(B, S, H, D, seed=41)
    do = qkv(B, S, H, D, seed=42)[0]
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 6, seed=43)
    val = np.random.default_rng(44).integers(0, bkv + 1, size=S // bkv).astype(np.int32)
    caught = False
    for kv_valid in (None, val):
        flat = B * H * S
        dq = oracle.bwd_dq_rows(q, k, v, do, idx, cnt, bq, bkv, 0.3, kv_valid=kv_valid)
        dk, dv = oracle.bwd_dkv_rows(q, k, v, do, idx, cnt, bq, bkv, 0.3, kv_valid=kv_valid)
        shape = lambda a: a.reshape(B, H, S, D).transpose(0, 2, 1, 3)  # noqa: E731
        assert dq.shape[0] == flat
        got = (shape(dq), shape(dk), shape(dv))
        ref = _autograd(q, k, v, do, idx, cnt, bq, bkv, 0.3, kv_valid)
        caught |= any(not np.all(np.abs(g - r) < 2e-5 * max(1.0, np.abs(r).max())) for g, r in zip(got, ref))
    assert caught, f"mutation {name} went unnoticed"
