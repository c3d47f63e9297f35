"""Pins for the CPU attention oracle (runs without a GPU).

The oracle (oracle/vsa_oracle.c) is checked against things other than
itself: a float64 brute force that materialises the token mask, PyTorch's
float64 SDPA for the all-selected case, closed forms, invariants that the
definition implies, and planted mistakes that these checks must catch.
"""

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import frontend
from workloads import bf16_bits, qkv, random_csr

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _f64(x_bits):
    return (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _token_mask(idx, cnt, S, block_q, block_kv, kv_valid=None):
    """[B, H, S, S] bool: query i may see key j. Built by explicit loops; with
    kv_valid only the first kv_valid[t] keys of tile t exist."""
    B, H, NQ, _ = idx.shape
    m = np.zeros((B, H, S, S), dtype=bool)
    for b in range(B):
        for h in range(H):
            for p in range(NQ):
                for e in range(int(cnt[b, h, p])):
                    t = int(idx[b, h, p, e])
                    n = block_kv if kv_valid is None else int(kv_valid[t])
                    m[b, h, p * block_q:(p + 1) * block_q, t * block_kv:t * block_kv + n] = True
    return m


def _brute(q, k, v, idx, cnt, block_q, block_kv, scale, kv_valid=None):
    """float64 masked softmax attention; returns O [B,S,H,D], LSE [B,H,S]."""
    qf, kf, vf = (_f64(bf16_bits(t)).transpose(0, 2, 1, 3) for t in (q, k, v))  # [B,H,S,D]
    B, H, S, D = qf.shape
    tm = _token_mask(idx, cnt, S, block_q, block_kv, kv_valid)
    s = np.einsum("bhid,bhjd->bhij", qf, kf) * scale
    s = np.where(tm, s, -np.inf)
    mx = s.max(-1, keepdims=True)
    empty = ~np.isfinite(mx)
    mx = np.where(empty, 0.0, mx)
    e = np.exp(s - mx)
    l = e.sum(-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(empty, 0.0, e / l)
        lse = np.where(empty[..., 0], -np.inf, (mx + np.log(l))[..., 0])
    o = np.einsum("bhij,bhjd->bhid", p, vf)
    return o.transpose(0, 2, 1, 3), lse


CASES = [
    # B, H, S, D, block_q, block_kv, count range
    (2, 2, 128, 16, 16, 16, (0, 8)),
    (1, 2, 256, 64, 64, 64, (1, 4)),
    (1, 3, 256, 32, 32, 16, (0, 16)),
    (2, 1, 192, 16, 16, 32, (1, 6)),
    (1, 2, 256, 64, 128, 64, (1, 4)),
]


@pytest.mark.parametrize("B,H,S,D,bq,bkv,cr", CASES)
def test_matches_float64_brute_force(B, H, S, D, bq, bkv, cr):
    q, k, v = qkv(B, S, H, D, seed=S + D + bq)
    nq, nkv = S // bq, S // bkv
    idx, cnt = random_csr(B, H, nq, nkv, nkv, cr[0], min(cr[1], nkv), seed=7 * S + bkv)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale)
    o_ref, lse_ref = _brute(q, k, v, idx, cnt, bq, bkv, scale)
    assert np.abs(o - o_ref).max() < 2e-5
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(lse[~fin] == -np.inf)
    assert np.abs(lse[fin] - lse_ref[fin]).max() < 2e-5 * max(1.0, np.abs(lse_ref[fin]).max())
    # empty rows: O = 0 exactly
    empty_rows = ~fin  # [B,H,S]
    o_bhsd = o.transpose(0, 2, 1, 3)
    assert np.all(o_bhsd[empty_rows] == 0.0)


def _ragged(nkv, block_kv, seed, p_full=0.5):
    """Valid key counts per tile: full, empty, or anywhere in between."""
    rng = np.random.default_rng(seed)
    val = rng.integers(0, block_kv + 1, size=nkv).astype(np.int32)
    val[rng.random(nkv) < p_full] = block_kv
    val[rng.random(nkv) < 0.1] = 0
    return val


@pytest.mark.parametrize("B,H,S,D,bq,bkv,cr", CASES)
def test_partial_tiles_match_float64_brute_force(B, H, S, D, bq, bkv, cr):
    q, k, v = qkv(B, S, H, D, seed=S + D + bq + 1)
    nq, nkv = S // bq, S // bkv
    idx, cnt = random_csr(B, H, nq, nkv, nkv, cr[0], min(cr[1], nkv), seed=7 * S + bkv + 1)
    val = _ragged(nkv, bkv, seed=S + bkv)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=val)
    o_ref, lse_ref = _brute(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=val)
    assert np.abs(o - o_ref).max() < 2e-5
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - lse_ref[fin]).max() < 2e-5 * max(1.0, np.abs(lse_ref[fin]).max())
    assert np.all(o.transpose(0, 2, 1, 3)[~fin] == 0.0)
    # all tiles full is the same as no validity input, bit for bit
    full = np.full(nkv, bkv, np.int32)
    o2, l2 = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=full)
    o3, l3 = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


def test_partial_tiles_zero_keys_closed_form():
    """K = 0 with partial tiles: LSE = ln(#valid selected keys), O = their V mean."""
    B, H, S, D, bq, bkv = 1, 2, 256, 32, 64, 16
    q, _, v = qkv(B, S, H, D, seed=43)
    k = torch.zeros_like(q)
    nkv = S // bkv
    idx, cnt = random_csr(B, H, S // bq, nkv, nkv, 1, 9, seed=44)
    val = _ragged(nkv, bkv, seed=45)
    o, lse = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.2, kv_valid=val)
    vf = _f64(bf16_bits(v))
    for h in range(H):
        for p in range(S // bq):
            c = int(cnt[0, h, p])
            tok = np.concatenate([np.arange(t * bkv, t * bkv + val[t]) for t in idx[0, h, p, :c]])
            for i in range(p * bq, (p + 1) * bq, 13):
                if tok.size == 0:
                    assert lse[0, h, i] == -np.inf and np.all(o[0, i, h] == 0.0)
                    continue
                assert abs(lse[0, h, i] - math.log(tok.size)) < 1e-6 * math.log(tok.size) + 1e-7
                assert np.abs(o[0, i, h] - vf[0, tok, h].mean(0)).max() < 1e-5


def test_partial_tiles_are_bitwise_identical_across_tile_shapes():
    """Ragged logical blocks expanded to finer tiles select the same key tokens."""
    from workloads import anchor_uniform_mask

    B, H, S, D = 1, 2, 1024, 64
    q, k, v = qkv(B, S, H, D, seed=33)
    base = anchor_uniform_mask(H, S // 256, S // 256, 2, seed=34)[None]
    vbs = np.array([256, 200, 129, 64], dtype=np.int32)
    results = []
    for shape in ((256, 256), (256, 128), (128, 64), (64, 64)):
        ld = S // shape[1]
        idx, cnt, ovf = frontend.mask_to_csr(base, (256, 256), shape, ld)
        val = frontend.expand_valid(vbs, 256, shape[1])
        results.append(oracle.attn_full(q, k, v, idx, cnt, shape[0], shape[1], 0.125, kv_valid=val))
    for o, l in results[1:]:
        assert np.array_equal(o, results[0][0]) and np.array_equal(l, results[0][1])


def test_invalid_valid_counts_are_rejected():
    B, H, S, D, bq, bkv = 1, 1, 128, 16, 32, 32
    q, k, v = qkv(B, S, H, D, seed=3)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 2, seed=4)
    for bad in ([33, 32, 32, 32], [-1, 32, 32, 32]):
        with pytest.raises(ValueError):
            oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.1, kv_valid=np.array(bad, np.int32))


def test_dense_equals_torch_sdpa_float64():
    B, H, S, D = 1, 2, 512, 64
    q, k, v = qkv(B, S, H, D, seed=3)
    bq = bkv = 64
    nq, nkv = S // bq, S // bkv
    idx = np.broadcast_to(np.arange(nkv, dtype=np.int32), (B, H, nq, nkv)).copy()
    cnt = np.full((B, H, nq), nkv, dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale)
    q64, k64, v64 = (t.double().permute(0, 2, 1, 3) for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(q64, k64, v64, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    lse_ref = torch.logsumexp((q64 @ k64.transpose(-1, -2)) * scale, dim=-1).numpy()
    assert np.abs(o - ref).max() < 2e-5
    assert np.abs(lse - lse_ref).max() < 2e-5 * np.abs(lse_ref).max()


def test_lse_is_logsumexp_of_masked_scores():
    from scipy.special import logsumexp

    B, H, S, D, bq, bkv = 1, 2, 256, 32, 32, 32
    q, k, v = qkv(B, S, H, D, seed=11)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 5, seed=12)
    scale = 0.37
    _, lse = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale)
    qf, kf = (_f64(bf16_bits(t)) for t in (q, k))
    tm = _token_mask(idx, cnt, S, bq, bkv)
    for h in range(H):
        for i in range(0, S, 17):
            s = (kf[0, :, h] @ qf[0, i, h]) * scale
            ref = logsumexp(s[tm[0, h, i]])
            assert abs(lse[0, h, i] - ref) < 1e-5 * max(1.0, abs(ref))


def test_probability_rows_sum_to_one_and_vanish_outside_mask():
    B, H, S, D, bq, bkv = 1, 2, 256, 64, 64, 32
    q, k, _ = qkv(B, S, H, D, seed=5)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 8, seed=6)
    tm = _token_mask(idx, cnt, S, bq, bkv)
    for flat in (0, 1, 63, 64, 200, 255, 256 + 77, 2 * 256 - 1):
        h, i = divmod(flat, S)
        p = oracle.probs_row(q, k, idx, cnt, bq, bkv, 0.125, flat)
        assert abs(float(p.astype(np.float64).sum()) - 1.0) < 1e-5
        assert np.all(p[~tm[0, h, i]] == 0.0)
        assert np.all(p[tm[0, h, i]] > 0.0)


def test_idx_order_does_not_change_result_bitwise():
    B, H, S, D, bq, bkv = 1, 2, 256, 64, 32, 32
    q, k, v = qkv(B, S, H, D, seed=21)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 8, seed=22, shuffle=False)
    o1, l1 = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.125)
    rng = np.random.default_rng(0)
    idx2 = idx.copy()
    for pos in np.ndindex(cnt.shape):
        c = cnt[pos]
        idx2[pos][:c] = rng.permutation(idx2[pos][:c])
    o2, l2 = oracle.attn_full(q, k, v, idx2, cnt, bq, bkv, 0.125)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_exact_expansion_is_bitwise_identical_across_tile_shapes():
    from workloads import anchor_uniform_mask

    B, H, S, D = 1, 2, 1024, 64
    q, k, v = qkv(B, S, H, D, seed=31)
    base = anchor_uniform_mask(H, S // 256, S // 256, 2, seed=32)[None]
    results = []
    for shape in ((256, 256), (256, 128), (128, 64), (64, 64)):
        ld = S // shape[1]
        idx, cnt, ovf = frontend.mask_to_csr(base, (256, 256), shape, ld)
        assert not ovf
        results.append(oracle.attn_full(q, k, v, idx, cnt, shape[0], shape[1], 0.125))
    for o, l in results[1:]:
        assert np.array_equal(o, results[0][0]) and np.array_equal(l, results[0][1])


def test_zero_keys_closed_form():
    """K = 0: every score is 0, so LSE = ln(#keys) and O = mean of allowed V rows."""
    B, H, S, D, bq, bkv = 1, 2, 256, 32, 64, 16
    q, _, v = qkv(B, S, H, D, seed=41)
    k = torch.zeros_like(q)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 9, seed=42)
    o, lse = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.2)
    vf = _f64(bf16_bits(v))
    for h in range(H):
        for p in range(S // bq):
            c = int(cnt[0, h, p])
            tok = np.concatenate([np.arange(t * bkv, (t + 1) * bkv) for t in idx[0, h, p, :c]])
            mean = vf[0, tok, h].mean(0)
            for i in range(p * bq, (p + 1) * bq, 13):
                assert abs(lse[0, h, i] - math.log(c * bkv)) < 1e-6 * math.log(c * bkv) + 1e-7
                assert np.abs(o[0, i, h] - mean).max() < 1e-5


def test_token_index_values_pin_which_tiles_are_read():
    """K = 0 and V[j] = j: O_i is exactly the mean index of the allowed keys."""
    B, H, S, D, bq, bkv = 1, 1, 256, 16, 32, 16
    q, _, _ = qkv(B, S, H, D, seed=51)
    k = torch.zeros_like(q)
    v = torch.arange(S, dtype=torch.float32).view(1, S, 1, 1).expand(B, S, H, D).to(torch.bfloat16)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 5, seed=52)
    o, _ = oracle.attn_full(q, k, v.contiguous(), idx, cnt, bq, bkv, 1.0)
    for p in range(S // bq):
        c = int(cnt[0, 0, p])
        tiles = idx[0, 0, p, :c]
        expect = np.mean(np.concatenate([np.arange(t * bkv, (t + 1) * bkv) for t in tiles]))
        assert np.abs(o[0, p * bq:(p + 1) * bq, 0] - expect).max() < 1e-4 * max(1.0, expect)


def test_constant_values_give_constant_output():
    B, H, S, D, bq, bkv = 1, 2, 128, 16, 16, 16
    q, k, _ = qkv(B, S, H, D, seed=61)
    v = torch.full((B, S, H, D), 1.5, dtype=torch.bfloat16)
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 8, seed=62)
    o, _ = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.25)
    assert np.abs(o - 1.5).max() < 2e-6


@pytest.mark.parametrize("bad", ["dup", "range", "cnt"])
def test_invalid_csr_is_rejected(bad):
    B, H, S, D, bq, bkv = 1, 1, 64, 16, 16, 16
    q, k, v = qkv(B, S, H, D)
    idx, cnt = random_csr(B, H, 4, 4, 4, 2, 2, seed=1)
    if bad == "dup":
        idx[0, 0, 1, 1] = idx[0, 0, 1, 0]
    elif bad == "range":
        idx[0, 0, 2, 0] = 4
    else:
        cnt[0, 0, 3] = 5
    with pytest.raises(ValueError):
        oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.25)


# --- planted mistakes: each must make the brute-force pin fail ---------------

MUTATIONS = {
    "scale_dropped": ("s[j] = acc * scale;", "s[j] = acc;"),
    "key_from_query_row": ("const uint16_t* krow = k + ((int64_t)b * S + j) * tok + (int64_t)h * D;\n            float acc",
                           "const uint16_t* krow = k + ((int64_t)b * S + i) * tok + (int64_t)h * D;\n            float acc"),
    "value_tiles_use_block_q": ("if (!allowed(allow, block_kv, j)) continue;\n                        const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;\n                        float w",
                                "if (!allowed(allow, block_q, j)) continue;\n                        const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;\n                        float w"),
    "key_tile_offset": ("const uint16_t* krow = k + ((int64_t)b * S + j) * tok + (int64_t)h * D;\n            float acc",
                        "const uint16_t* krow = k + ((int64_t)b * S + (j + block_kv) % S) * tok + (int64_t)h * D;\n            float acc"),
    "value_wrong_head": ("const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;\n                        float w",
                         "const uint16_t* vrow = v + ((int64_t)b * S + j) * tok;\n                        float w"),
    "no_normalisation": ("if (allowed(allow, block_kv, j)) s[j] = s[j] / l;", "if (allowed(allow, block_kv, j)) s[j] = s[j];"),
    "valid_counts_ignored": ("allow[t] = kv_valid ? kv_valid[t] : block_kv;", "allow[t] = block_kv;"),
    "valid_count_off_by_one": ("return (j % block_kv) < allow[j / block_kv];", "return (j % block_kv) <= allow[j / block_kv];"),
    "lse_without_max": ("lse[r] = m + logf(l);", "lse[r] = logf(l);"),
    "max_not_subtracted": ("s[j] = expf(s[j] - m);", "s[j] = expf(s[j]);"),
}


def _build_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "vsa_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    str(path), "-o", str(so), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name, monkeypatch):
    so = _build_mutant(tmp_path, name)
    import ctypes

    lib = ctypes.CDLL(so)
    lib.vsa_oracle_attn_rows.argtypes = oracle._load().vsa_oracle_attn_rows.argtypes
    lib.vsa_oracle_attn_rows.restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", lib)
    B, H, S, D, bq, bkv = 1, 2, 128, 16, 32, 16
    q, k, v = qkv(B, S, H, D, seed=71)
    q = (q.float() * 3).to(torch.bfloat16)  # large scores so the max matters numerically
    idx, cnt = random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 6, seed=72)
    caught = False
    for val in (None, _ragged(S // bkv, bkv, seed=73)):  # full tiles, then partial tiles
        o, lse = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.3, kv_valid=val)
        o_ref, lse_ref = _brute(q, k, v, idx, cnt, bq, bkv, 0.3, kv_valid=val)
        with np.errstate(invalid="ignore"):
            caught |= not np.all(np.abs(o - o_ref) < 2e-5)
            caught |= not np.all(np.abs(lse - lse_ref) < 2e-5 * np.maximum(1.0, np.abs(lse_ref)))
    assert caught, f"mutation {name} went unnoticed"
