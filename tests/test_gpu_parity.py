"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances for the forward pass (bf16 O compared after conversion to fp32,
fp32 LSE): max |dO| <= 2e-2, mean |dO| <= 2e-3, |dLSE| <= 1e-3*max(1, |LSE|).
Integer front-end outputs must be bit-exact.
"""

import math
import os

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
    line = f"[gpu-parity] {msg}"
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
        x = torch.from_numpy(np.array(x, copy=True, order="C"))  # writable (oracle arrays may be read-only)
    return x.contiguous().to("cuda")


def check_rows(o_gpu, lse_gpu, rows, o_ref, lse_ref, S, H, label):
    """Compare GPU O [B,S,H,D] / LSE [B,H,S] at flat rows against oracle rows."""
    rows = np.asarray(rows, dtype=np.int64)
    i = rows % S
    h = (rows // S) % H
    b = rows // (S * H)
    og = o_gpu.float().cpu().numpy()[b, i, h]
    lg = lse_gpu.cpu().numpy()[b, h, i]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lg)), f"{label}: LSE finiteness differs"
    assert np.all(lg[~fin] == -np.inf), f"{label}: empty rows must have LSE=-inf"
    assert np.all(og[~fin] == 0.0), f"{label}: empty rows must have O=0"
    d = np.abs(og - o_ref)
    max_abs, mean_abs = float(d.max()), float(d.mean())
    lse_err = float((np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))).max()) if fin.any() else 0.0
    # the FastVideo page's own gate: max(1e-2, 8 x the bf16 output-rounding floor of the reference)
    ref32 = torch.from_numpy(np.ascontiguousarray(o_ref, dtype=np.float32))
    floor = float((ref32 - ref32.to(torch.bfloat16).float()).abs().max())
    page_limit = max(1e-2, 8.0 * floor)
    say(f"{label}: rows={rows.size} max|dO|={max_abs:.3e} mean|dO|={mean_abs:.3e} LSE rel={lse_err:.3e} "
        f"(page gate {page_limit:.3e})")
    assert np.isfinite(og).all()
    assert max_abs <= O_MAX_ABS, f"{label}: max |dO| {max_abs}"
    assert max_abs <= page_limit, f"{label}: max |dO| {max_abs} above the page's gate {page_limit}"
    assert mean_abs <= O_MEAN_ABS, f"{label}: mean |dO| {mean_abs}"
    assert lse_err <= LSE_REL, f"{label}: LSE rel err {lse_err}"


def sample_rows(B, H, S, bq, tiles_per_head=3, seed=0):
    rng = np.random.default_rng(seed)
    nq = S // bq
    out = []
    for b in range(B):
        for h in range(H):
            tiles = {0, nq - 1} | set(rng.integers(0, nq, size=tiles_per_head).tolist())
            for p in sorted(tiles):
                local = {0, 1, 31, 32, 33, bq - 1} | set(rng.integers(0, bq, size=2).tolist())
                for r in sorted(local):
                    out.append((b * H + h) * S + p * bq + r)
    return np.array(out, dtype=np.int64)


# ----------------------------------------------------------------- front-end

FRONT_CASES = [
    ("tiny", W.TINY, (64, 64), 16),
    ("vsa256->256x128", W.VSA256, (256, 128), 26),
    ("vsa256->128x64", W.VSA256, (128, 64), 52),
    ("vsa256->64x64", W.VSA256, (64, 64), 52),
    ("vsa256->256x256", W.VSA256, (256, 256), 128),
    ("native64 compact", W.NATIVE64, (64, 64), 92),
    ("native64 full", W.NATIVE64, (64, 64), 512),
    ("dense->128x128", W.DENSE, (128, 128), 32),
]


@pytest.mark.parametrize("label,wl,shape,ld", FRONT_CASES, ids=[c[0] for c in FRONT_CASES])
def test_mask_to_csr_bit_exact(vsa, label, wl, shape, ld):
    say(f"mask_to_csr {label}")
    mask = wl.logical_mask()
    idx_ref, cnt_ref, ovf_ref = ofront.mask_to_csr(mask, wl.logical_block, shape, ld)
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx, cnt = vsa.vsa_mask_to_csr(dev(mask), wl.logical_block, shape, ld, overflow=ovf)
    torch.cuda.synchronize()
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(cnt_h, cnt_ref)
    valid = np.arange(ld)[None, None, None, :] < np.minimum(cnt_ref, ld)[..., None]
    assert np.array_equal(np.where(valid, idx_h, -1), np.where(valid, idx_ref, -1))
    assert bool(ovf.item()) == ovf_ref


@pytest.mark.parametrize("lblock,shape", [((256, 256), (256, 128)), ((256, 256), (64, 64)), ((128, 64), (32, 16)),
                                          ((256, 256), (128, 256))])
def test_mask_to_csr_drops_empty_tiles_bit_exact(vsa, lblock, shape):
    """With valid keys per physical tile, tiles without one are left out:
    counts and lists bit-exact against the oracle's front-end (rows of more
    than 64 logical cells exercise the wave prefix sum across steps)."""
    say(f"mask_to_csr with valid counts {lblock} -> {shape}")
    S = 32768 if lblock[1] == 256 else 8192  # 128 logical cells per row
    rng = np.random.default_rng(shape[0] + shape[1])
    mask = (rng.random((2, 3, S // lblock[0], S // lblock[1])) < 0.6).astype(np.uint8)
    vbs = W.ragged_block_sizes(S // lblock[1], lblock[1], seed=shape[1], p_full=0.2)
    vbs[:4] = [0, 1, lblock[1], 0]
    val = ofront.expand_valid(vbs, lblock[1], shape[1])
    ld = S // shape[1]
    ridx, rcnt, _ = ofront.mask_to_csr(mask, lblock, shape, ld, kv_valid=val)
    idx, cnt = vsa.vsa_mask_to_csr(dev(mask), lblock, shape, ld, kv_valid=dev(val))
    torch.cuda.synchronize()
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    listed = np.arange(ld)[None, None, None, :] < rcnt[..., None]
    assert np.array_equal(np.where(listed, idx.cpu().numpy(), -1), np.where(listed, ridx, -1))
    # a compact row length truncates and keeps the true count
    small = max(1, int(rcnt.max()) - 3)
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    i2, c2 = vsa.vsa_mask_to_csr(dev(mask), lblock, shape, small, overflow=ovf, kv_valid=dev(val))
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), rcnt) and ovf.item() == 1
    keep = np.arange(small)[None, None, None, :] < np.minimum(rcnt, small)[..., None]
    assert np.array_equal(np.where(keep, i2.cpu().numpy(), -1), np.where(keep, ridx[..., :small], -1))


def test_mask_to_csr_overflow_flag(vsa):
    say("mask_to_csr overflow")
    rng = np.random.default_rng(5)
    mask = (rng.random((2, 3, 8, 16)) < 0.3).astype(np.uint8)
    mask[1, 2, 3, :] = 1  # a full row: 16 cells -> 32 tiles at kv_ratio 2
    ld = 20
    idx_ref, cnt_ref, ovf_ref = ofront.mask_to_csr(mask, (128, 64), (64, 32), ld)
    assert ovf_ref
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx, cnt = vsa.vsa_mask_to_csr(dev(mask), (128, 64), (64, 32), ld, overflow=ovf)
    torch.cuda.synchronize()
    assert np.array_equal(cnt.cpu().numpy(), cnt_ref)
    valid = np.arange(ld)[None, None, None, :] < np.minimum(cnt_ref, ld)[..., None]
    assert np.array_equal(np.where(valid, idx.cpu().numpy(), -1), np.where(valid, idx_ref, -1))
    assert ovf.item() == 1


WL_CASES = [
    # label, (lo, hi, n) or None for the native Q64 counts, ld, segment (None = whole list)
    ("native64 per head", None, 92, 512),
    ("native64 global", None, 92, None),
    ("random clamp", (-3, 100, 12345), 90, None),
    ("random clamp segmented", (-3, 100, 12345), 90, 823),
    ("single", (0, 5, 1), 5, None),
    ("ragged 65", (0, 3, 65), 3, 13),
    ("many", (0, 600, 100000), 600, 5000),
    ("wide bins", (0, 5000, 7777), 5000, None),
    ("wide bins segmented", (0, 5000, 7777), 5000, 7777 // 7),
    ("all equal", (7, 7, 3000), 7, 100),
]


@pytest.mark.parametrize("label,spec,ld,segment", WL_CASES, ids=[c[0] for c in WL_CASES])
def test_worklist_bit_exact(vsa, label, spec, ld, segment):
    say(f"worklist {label}")
    if spec is None:
        mask = W.NATIVE64.logical_mask()
        _, cnt, _ = ofront.mask_to_csr(mask, (64, 64), (64, 64), ld)
        cnt = cnt.reshape(-1)
    else:
        lo, hi, n = spec
        cnt = np.random.default_rng(n).integers(lo, hi + 1, size=n).astype(np.int32)
    seg = cnt.size if segment is None else segment
    ref = ofront.build_worklist(cnt, ld, segment=seg)
    got = vsa.vsa_build_worklist(dev(cnt), ld, segment=seg)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


# ------------------------------------------------------------ forward pass

def _run_fwd(vsa, q, k, v, idx, cnt, bq, bkv, scale, kv_valid=None):
    o, lse = vsa.vsa_attn_fwd(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=kv_valid)
    torch.cuda.synchronize()
    return o, lse


def test_tiny_workload_all_rows(vsa):
    wl = W.TINY
    say(f"forward {wl.name} (all rows)")
    q, k, v = wl.qkv()
    idx, cnt, _ = ofront.mask_to_csr(wl.logical_mask(), wl.logical_block, (64, 64), 16)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, 64, 64, wl.scale)
    o, lse = _run_fwd(vsa, dev(q), dev(k), dev(v), dev(idx), dev(cnt), 64, 64, wl.scale)
    B, S, H, D = q.shape
    rows = np.arange(B * H * S)
    check_rows(o, lse, rows, o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S, H, wl.name)


SHAPES = [(bq, bkv, d) for bq in (64, 128, 256) for bkv in (64, 128) for d in (64, 128)]


@pytest.mark.parametrize("bq,bkv,D", SHAPES, ids=[f"{a}x{b}_d{c}" for a, b, c in SHAPES])
def test_every_tile_shape_all_rows(vsa, bq, bkv, D):
    """Random shuffled CSR with empty and full rows, compact ld, B=2."""
    B, H, S = 2, 2, 1024
    say(f"forward shapes {bq}x{bkv} D={D}")
    q, k, v = W.qkv(B, S, H, D, seed=bq + bkv + D)
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=bq * 7 + bkv + D)
    cnt[0, 0, 0] = 0
    cnt[1, 1, nq - 1] = nkv
    idx[1, 1, nq - 1] = np.random.default_rng(1).permutation(nkv)
    ld = int(cnt.max())
    idx = np.ascontiguousarray(idx[..., :ld])
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale)
    o, lse = _run_fwd(vsa, dev(q), dev(k), dev(v), dev(idx), dev(cnt), bq, bkv, scale)
    rows = np.arange(B * H * S)
    check_rows(o, lse, rows, o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S, H,
               f"{bq}x{bkv} D={D}")


def _strided_views(q, k, v, layout):
    """q, k, v [B, S, H, D] (device) copied into the buffers of ``layout`` and
    returned as views of them: packed [B,S,3,H,D] projection, heads
    interleaved [B,S,H,3,D], q alone with k, v from a packed [B,S,2,H,D],
    [B,H,S,D] buffers seen as [B,S,H,D], k and v of head 0 broadcast over the
    heads (head stride 0), or each tensor in a token-padded buffer
    [B,S+64,H,D] at token 32."""
    B, S, H, D = q.shape
    if layout == "bhsd":
        return tuple(t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    if layout == "kv_broadcast":
        return q, k[:, :, :1].expand(B, S, H, D), v[:, :, :1].expand(B, S, H, D)
    if layout == "qkv_packed":
        buf = torch.stack((q, k, v), dim=2).contiguous()
        return buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
    if layout == "heads_interleaved":
        buf = torch.stack((q, k, v), dim=3).contiguous()
        return buf[:, :, :, 0], buf[:, :, :, 1], buf[:, :, :, 2]
    if layout == "kv_packed":
        buf = torch.stack((k, v), dim=2).contiguous()
        return q, buf[:, :, 0], buf[:, :, 1]
    out = []
    for t in (q, k, v):
        buf = torch.zeros((B, S + 64, H, D), dtype=t.dtype, device=t.device)
        buf[:, 32:32 + S] = t
        out.append(buf[:, 32:32 + S])
    return tuple(out)


STRIDED = [(bq, bkv, D, "qkv_packed") for bq, bkv, D in SHAPES] + \
          [(bq, bkv, D, "bhsd") for bq, bkv, D in SHAPES] + \
          [(256, 128, 128, lay) for lay in ("heads_interleaved", "kv_packed", "token_padded", "kv_broadcast")] + \
          [(64, 64, 64, lay) for lay in ("heads_interleaved", "kv_packed", "token_padded", "kv_broadcast")] + \
          [(128, 64, 128, "kv_broadcast")]


@pytest.mark.parametrize("bq,bkv,D,layout", STRIDED, ids=[f"{a}x{b}_d{c}_{l}" for a, b, c, l in STRIDED])
def test_strided_views_bitwise_equal_to_contiguous(vsa, bq, bkv, D, layout):
    """q, k, v read in place through their strides (vsa_attn_fwd_strided, the
    route vsa_attn_fwd takes for views) give the result of the contiguous
    call on copies of the same views bitwise, for every tile shape (splits
    included at these sizes); the packed 256x128 case and a broadcast case
    are also checked against the oracle on every row."""
    B, H, S = 2, 2, 1024
    say(f"strided views {layout} {bq}x{bkv} D={D}")
    q, k, v = W.qkv(B, S, H, D, seed=bq + bkv + D + 11)
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=bq * 5 + bkv + D + 11)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = dev(q), dev(k), dev(v)
    qs, ks, vs = _strided_views(qd, kd, vd, layout)
    assert not (qs.is_contiguous() and ks.is_contiguous() and vs.is_contiguous())
    qc, kc, vc = qs.contiguous(), ks.contiguous(), vs.contiguous()
    o1, l1 = _run_fwd(vsa, qc, kc, vc, dev(idx), dev(cnt), bq, bkv, scale)
    o2, l2 = _run_fwd(vsa, qs, ks, vs, dev(idx), dev(cnt), bq, bkv, scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{layout} {bq}x{bkv}: strided result differs"
    if (bq, bkv, D, layout) in ((256, 128, 128, "qkv_packed"), (128, 64, 128, "kv_broadcast")):
        q, k, v = qc.cpu(), kc.cpu(), vc.cpu()
        o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale)
        check_rows(o2, l2, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S,
                   H, f"strided {layout} {bq}x{bkv}")


@pytest.mark.parametrize("bq,bkv,D", SHAPES, ids=[f"{a}x{b}_d{c}" for a, b, c in SHAPES])
def test_partial_tiles_every_tile_shape_all_rows(vsa, bq, bkv, D):
    """Per-tile valid key counts (empty, partial, full tiles), including a row
    whose selected tiles hold no valid key."""
    B, H, S = 2, 2, 1024
    say(f"forward partial tiles {bq}x{bkv} D={D}")
    q, k, v = W.qkv(B, S, H, D, seed=bq + bkv + D + 5)
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 1, nkv, seed=bq * 7 + bkv + D + 5)
    val = W.ragged_block_sizes(nkv, bkv, seed=bq + 3 * bkv + D, p_full=0.4)
    val[:2] = 0
    val[2] = 1
    val[3] = bkv - 1
    cnt[1, 0, nq - 1] = 2  # only tiles without valid keys: an empty row
    idx[1, 0, nq - 1, :2] = [1, 0]
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=val)
    assert np.all(np.isneginf(lse_ref[1, 0, (nq - 1) * bq:]))
    o, lse = _run_fwd(vsa, dev(q), dev(k), dev(v), dev(idx), dev(cnt), bq, bkv, scale, kv_valid=dev(val))
    check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S, H,
               f"partial {bq}x{bkv} D={D}")


MANY_ITEMS = [(64, 64, 64), (64, 128, 128), (128, 64, 64), (128, 128, 128)]


@pytest.mark.parametrize("bq,bkv,D", MANY_ITEMS, ids=[f"{a}x{b}_d{c}" for a, b, c in MANY_ITEMS])
@pytest.mark.parametrize("partial", [False, True], ids=["full", "partial"])
def test_many_work_items_all_rows(vsa, bq, bkv, D, partial):
    """At least eight 64- or 128-row work items per compute unit: these run the
    independent-wave kernel (the small cases above run the multi-stream ones).
    Empty rows, short and long lists, partial tiles; every row."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = 2048
    B, H = 2, max(1, -(-8 * cus * bq // (2 * S)))
    nq, nkv = S // bq, S // bkv
    assert B * H * nq >= 8 * cus
    say(f"forward many items {bq}x{bkv} D={D} partial={partial}: B={B} H={H}")
    q, k, v = W.qkv(B, S, H, D, seed=bq + bkv + D + partial)
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv // 4, 0, nkv // 4, seed=bq * 3 + bkv + D)
    val = None
    if partial:
        val = W.ragged_block_sizes(nkv, bkv, seed=bq + bkv, p_full=0.4)
        val[:2] = [0, 1]
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=val)
    o, lse = _run_fwd(vsa, dev(q), dev(k), dev(v), dev(idx), dev(cnt), bq, bkv, scale,
                      kv_valid=None if val is None else dev(val))
    check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S, H,
               f"many items {bq}x{bkv} D={D} partial={partial}")


EXPAND_CASES = [(256, 128), (256, 64), (256, 256), (128, 32), (64, 64)]


@pytest.mark.parametrize("lkv,pkv", EXPAND_CASES, ids=[f"{a}->{b}" for a, b in EXPAND_CASES])
def test_expand_valid_bit_exact(vsa, lkv, pkv):
    say(f"expand_valid {lkv}->{pkv}")
    vbs = W.ragged_block_sizes(1000, lkv, seed=lkv + pkv)
    vbs[:3] = [0, lkv, 1]
    ref = ofront.expand_valid(vbs, lkv, pkv)
    got = vsa.vsa_expand_valid(dev(vbs), lkv, pkv)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_invalid_entries_are_skipped_and_counts_clamped(vsa):
    """Out-of-range tile indices are skipped; counts above ld use ld entries."""
    B, H, S, D, bq, bkv = 1, 2, 1024, 128, 128, 64
    say("forward invalid entries")
    q, k, v = W.qkv(B, S, H, D, seed=99)
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, 8, 3, 6, seed=98)
    idx[0, 0, 1, 1] = -5          # skipped
    idx[0, 1, 2, 0] = nkv         # skipped
    cnt[0, 1, 3] = 50             # clamped to ld = 8 (slots 6..7 hold -1: skipped)
    idx_clean = np.full_like(idx, -1)
    cnt_clean = np.zeros_like(cnt)
    for pos in np.ndindex(cnt.shape):
        ent = [t for t in idx[pos][:min(cnt[pos], 8)] if 0 <= t < nkv]
        idx_clean[pos][:len(ent)] = ent
        cnt_clean[pos] = len(ent)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx_clean, cnt_clean, bq, bkv, 1 / math.sqrt(D))
    o, lse = _run_fwd(vsa, dev(q), dev(k), dev(v), dev(idx), dev(cnt), bq, bkv, 1 / math.sqrt(D))
    check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1),
               S, H, "invalid entries")


UNSPLIT_CASES = [(bkv, D) for bkv in (64, 128) for D in (128, 64)]


@pytest.mark.parametrize("bkv,D", UNSPLIT_CASES, ids=[f"256x{a}_d{b}" for a, b in UNSPLIT_CASES])
def test_256_row_tiles_unsplit_all_rows(vsa, bkv, D):
    """256-row tiles through the work-list entry point (lists never split):
    lists of lengths 0, 1, 2, 3, all tiles and all but one, in shuffled
    order, with out-of-range entries that must be skipped and a work list in
    reverse order; every row against the oracle."""
    B, H, S = 2, 3, 4096
    nq, nkv = S // 256, S // bkv
    say(f"256-row tiles unsplit 256x{bkv} D={D}")
    q, k, v = W.qkv(B, S, H, D, seed=bkv + D + 300)
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=bkv * 5 + D)
    lens = [0, 1, 2, 3, nkv, nkv - 1, 5]
    for i, c in enumerate(lens):
        cnt[0, 0, i] = c
        idx[0, 0, i, :c] = np.random.default_rng(i).permutation(nkv)[:c]
    idx[1, 2, 3, 1] = -4          # skipped
    idx[1, 2, 4, 0] = nkv + 2     # skipped
    cnt[1, 2, 4] = max(cnt[1, 2, 4], 1)
    idx_clean = np.full_like(idx, -1)
    cnt_clean = np.zeros_like(cnt)
    for pos in np.ndindex(cnt.shape):
        ent = [t for t in idx[pos][:cnt[pos]] if 0 <= t < nkv]
        idx_clean[pos][:len(ent)] = ent
        cnt_clean[pos] = len(ent)
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx_clean, cnt_clean, 256, bkv, scale)
    work = torch.arange(B * H * nq, dtype=torch.int32, device="cuda").flip(0)
    o, lse = vsa.vsa_attn_fwd_worklist(dev(q), dev(k), dev(v), dev(idx), dev(cnt), 256, bkv, work, scale)
    torch.cuda.synchronize()
    check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S, H,
               f"256x{bkv} D={D} unsplit")


def test_worklist_subset_writes_only_listed_tiles(vsa):
    B, H, S, D, bq, bkv = 1, 2, 512, 64, 64, 64
    say("forward work-list subset")
    q, k, v = W.qkv(B, S, H, D, seed=5)
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 1, nkv, seed=6)
    work = np.array([3, 0, 9, 15], dtype=np.int32)  # flat (h*nq + p)
    o = torch.full((B, S, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, S), 7.0, dtype=torch.float32, device="cuda")
    vsa.vsa_attn_fwd_worklist(dev(q), dev(k), dev(v), dev(idx), dev(cnt), bq, bkv, dev(work), o=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 1 / math.sqrt(D))
    listed = np.zeros((H, nq), dtype=bool)
    listed.reshape(-1)[work] = True
    rows = [(h * S + p * bq + r) for h in range(H) for p in range(nq) if listed[h, p] for r in range(bq)]
    check_rows(o, lse, rows, o_ref.transpose(0, 2, 1, 3).reshape(-1, D)[rows], lse_ref.reshape(-1)[rows], S, H,
               "subset")
    on = o.float().cpu().numpy()
    ln = lse.cpu().numpy()
    for h in range(H):
        for p in range(nq):
            if not listed[h, p]:
                assert np.all(on[0, p * bq:(p + 1) * bq, h] == 7.0)
                assert np.all(ln[0, h, p * bq:(p + 1) * bq] == 7.0)


def test_deterministic_and_stream_aware(vsa):
    B, H, S, D, bq, bkv = 1, 3, 2048, 128, 128, 64
    say("forward determinism + side stream")
    q, k, v = (dev(t) for t in W.qkv(B, S, H, D, seed=3))
    idx, cnt = W.random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 20, seed=4)
    idx, cnt = dev(idx), dev(cnt)
    o1, l1 = _run_fwd(vsa, q, k, v, idx, cnt, bq, bkv, 0.09)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = vsa.vsa_attn_fwd(q, k, v, idx, cnt, bq, bkv, 0.09)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_concurrent_streams_every_row(vsa):
    """Two calls of different shapes enqueued back to back on two streams, no
    synchronisation between them: each call uses its own stream's work list
    and split workspace, so both outputs match the oracle on every row. Both
    launches split their lists (few work items), so the split counters and
    partial states of the two calls would collide if they shared buffers."""
    say("forward on two streams at once")
    cases = []
    for (B, H, S, D, bq, bkv, seed) in ((1, 1, 8192, 128, 256, 128, 61), (1, 2, 2048, 64, 64, 64, 62)):
        q, k, v = W.qkv(B, S, H, D, seed=seed)
        nq, nkv = S // bq, S // bkv
        idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 1, nkv, seed=seed + 1)
        scale = 1.0 / math.sqrt(D)
        o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
        cases.append(dict(q=q, k=k, v=v, idx=idx, cnt=cnt, qd=dev(q), kd=dev(k), vd=dev(v), idxd=dev(idx),
                          cntd=dev(cnt), o=o, lse=lse, bq=bq, bkv=bkv, scale=scale))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for c, s in zip(cases, streams):
            c["o"].fill_(7.0)
            c["lse"].fill_(7.0)
        torch.cuda.synchronize()
        for c, s in zip(cases, streams):
            vsa.vsa_attn_fwd(c["qd"], c["kd"], c["vd"], c["idxd"], c["cntd"], c["bq"], c["bkv"], c["scale"],
                             c["o"], c["lse"], stream=s)
        for s in streams:
            s.synchronize()
        for i, c in enumerate(cases):
            B, S, H, D = c["q"].shape
            o_ref, lse_ref = oracle.attn_full(c["q"], c["k"], c["v"], c["idx"], c["cnt"], c["bq"], c["bkv"],
                                              c["scale"])
            check_rows(c["o"], c["lse"], np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D),
                       lse_ref.reshape(-1), S, H, f"stream {i} call {rep}")


# ------------------------------------------------------------- split lists

@pytest.mark.parametrize("bq,bkv", [(256, 128), (64, 64)])
def test_split_lists_deterministic_and_equal_to_unsplit(vsa, bq, bkv):
    """256- and 64-row tiles with few work items run split lists
    (vsa_attn_fwd); two runs agree bitwise, and the unsplit kernel
    (vsa_attn_fwd_worklist) agrees within the tolerance; lists shorter than
    the number of parts leave some parts empty."""
    B, H, S, D = 1, 2, 2048, 128
    say("split lists: determinism and unsplit agreement")
    q, k, v = (dev(t) for t in W.qkv(B, S, H, D, seed=77))
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=78)
    cnt[0, 0, :4] = [0, 1, 2, 3]
    idx, cnt = dev(idx), dev(cnt)
    o1, l1 = _run_fwd(vsa, q, k, v, idx, cnt, bq, bkv, 0.09)
    o2, l2 = _run_fwd(vsa, q, k, v, idx, cnt, bq, bkv, 0.09)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    work = torch.arange(B * H * nq, dtype=torch.int32, device="cuda")
    o3, l3 = vsa.vsa_attn_fwd_worklist(q, k, v, idx, cnt, bq, bkv, work, 0.09)
    torch.cuda.synchronize()
    d = (o1.float() - o3.float()).abs()
    fin = torch.isfinite(l3)
    assert torch.equal(fin, torch.isfinite(l1))
    lrel = ((l1[fin] - l3[fin]).abs() / l3[fin].abs().clamp_min(1.0)).max().item()
    say(f"split vs unsplit: max|dO|={d.max().item():.3e} LSE rel={lrel:.3e}")
    assert d.max().item() <= O_MAX_ABS and lrel <= LSE_REL


def test_split_workspace_reuse_with_more_items(vsa):
    """A split launch with few items and large partial states, then one with
    more items whose counters reach into the first one's state bytes while
    its whole workspace still fits the buffer: the counters must read zero,
    so every row of the second launch is written and matches the oracle."""
    say("split workspace reuse")
    vsa.vsa_release()
    B, S, H, D = 1, 32768, 1, 128  # 128 items of 256 rows: split in two
    q, k, v = (dev(t) for t in W.qkv(B, S, H, D, seed=91))
    idx, cnt = W.random_csr(B, H, S // 256, S // 128, 2, 2, 2, seed=92)
    _run_fwd(vsa, q, k, v, dev(idx), dev(cnt), 256, 128, 0.09)
    B, S, H, D = 1, 16384, 2, 64  # 512 items of 64 rows: split in two
    q, k, v = W.qkv(B, S, H, D, seed=93)
    idx, cnt = W.random_csr(B, H, S // 64, S // 64, 3, 0, 3, seed=94)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, 64, 64, 0.125)
    for rep in range(2):
        o, lse = _run_fwd(vsa, dev(q), dev(k), dev(v), dev(idx), dev(cnt), 64, 64, 0.125)
        rows = np.arange(B * H * S)
        check_rows(o, lse, rows, o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S, H,
                   f"split reuse call {rep}")


# ------------------------------------------- Q64 pairing onto Q128 tiles

def _exact_expanded_q64(B, H, S, lblock, bkv, keep, seed):
    mask = np.stack([W.anchor_uniform_mask(H, S // lblock[0], S // lblock[1], keep, seed=seed + b) for b in range(B)])
    ld = keep * (lblock[1] // bkv)
    idx, cnt, _ = ofront.mask_to_csr(mask, lblock, (64, bkv), ld)
    return idx, cnt


PAIR_CASES = [
    ("vsa256 exact 64x64", W.VSA256, (64, 64), 52),
    ("native64", W.NATIVE64, (64, 64), 92),
]


@pytest.mark.parametrize("label,wl,shape,ld", PAIR_CASES, ids=[c[0] for c in PAIR_CASES])
def test_pair_q_tiles_bit_exact(vsa, label, wl, shape, ld):
    say(f"pair_q_tiles {label}")
    idx_ref, cnt_ref, _ = ofront.mask_to_csr(wl.logical_mask(), wl.logical_block, shape, ld)
    pidx_ref, pcnt_ref, unp_ref = ofront.pair_q_tiles(idx_ref, cnt_ref)
    pidx, pcnt, unp = vsa.vsa_pair_q_tiles(dev(idx_ref), dev(cnt_ref))
    torch.cuda.synchronize()
    assert int(unp.item()) == unp_ref
    assert np.array_equal(pcnt.cpu().numpy(), pcnt_ref)
    valid = np.arange(ld)[None, None, None, :] < np.minimum(pcnt_ref, ld)[..., None]
    assert np.array_equal(np.where(valid, pidx.cpu().numpy(), -1), np.where(valid, pidx_ref, -1))
    say(f"pair_q_tiles {label}: unpaired={unp_ref}")


def test_pair_q_tiles_planted_differences(vsa):
    """Pairs that differ in one entry, in order only, in count, or only past
    the stored prefix (ignored); counts above ld and negative counts."""
    say("pair_q_tiles planted differences")
    idx, cnt = _exact_expanded_q64(2, 3, 4096, (256, 256), 64, 5, seed=41)
    ld = idx.shape[-1]
    idx, cnt = idx.copy(), cnt.copy()
    idx[0, 0, 1, 0] = min(set(range(64)) - set(idx[0, 0, 0, :10].tolist()))
    idx[0, 1, 3, [0, 1]] = idx[0, 1, 3, [1, 0]]
    cnt[1, 2, 5] -= 1
    cnt[1, 0, 8] = cnt[1, 0, 9] = ld + 7          # both clamp to ld: the stored entries agree
    cnt[1, 1, 10] = cnt[1, 1, 11] = -3            # both empty
    pidx_ref, pcnt_ref, unp_ref = ofront.pair_q_tiles(idx, cnt)
    assert unp_ref == 3
    pidx, pcnt, unp = vsa.vsa_pair_q_tiles(dev(idx), dev(cnt))
    torch.cuda.synchronize()
    assert int(unp.item()) == unp_ref
    assert np.array_equal(pcnt.cpu().numpy(), pcnt_ref)
    valid = np.arange(ld)[None, None, None, :] < np.clip(pcnt_ref, 0, ld)[..., None]
    assert np.array_equal(np.where(valid, pidx.cpu().numpy(), -1), np.where(valid, pidx_ref, -1))


PAIRED_FWD = [(bkv, D, partial) for bkv in (64, 128) for D in (64, 128) for partial in (False, True)]


@pytest.mark.parametrize("bkv,D,partial", PAIRED_FWD, ids=[f"kv{a}_d{b}{'_partial' if c else ''}" for a, b, c in
                                                          PAIRED_FWD])
def test_paired_forward_all_rows(vsa, bkv, D, partial):
    """Exact-expanded Q64 lists run as 128-row tiles (bitwise the 128-row
    result), distinct lists as 64-row tiles (bitwise the 64-row result);
    both against the oracle on every row."""
    B, H, S = 2, 2, 2048
    q, k, v = W.qkv(B, S, H, D, seed=bkv + D + 71)
    qd, kd, vd = dev(q), dev(k), dev(v)
    scale = 1.0 / math.sqrt(D)
    val = None
    if partial:
        val = W.ragged_block_sizes(S // bkv, bkv, seed=bkv + D, p_full=0.4)
        val[:2] = [0, 1]
    vald = None if val is None else dev(val)
    pairable = _exact_expanded_q64(B, H, S, (256, 256), bkv, 3, seed=D + bkv)
    distinct = W.random_csr(B, H, S // 64, S // bkv, S // bkv, 0, S // bkv // 2, seed=D + bkv + 1)
    for label, (idx, cnt) in (("pairable", pairable), ("distinct", distinct)):
        idx = np.ascontiguousarray(idx[..., :max(1, int(cnt.max()))])
        say(f"paired forward {label} kv{bkv} D={D} partial={partial}")
        pidx, pcnt, unp = ofront.pair_q_tiles(idx, cnt)
        assert (unp == 0) == (label == "pairable")
        o, lse = vsa.vsa_attn_fwd_paired(qd, kd, vd, dev(idx), dev(cnt), bkv, scale, kv_valid=vald)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, 64, bkv, scale, kv_valid=val)
        check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1),
                   S, H, f"paired {label} kv{bkv} D={D}")
        # the schedule it must have run: the unsplit kernel over the paired
        # (128-row) or the input (64-row) lists, as the work-list entry runs it
        ridx, rcnt, rbq = (pidx, pcnt, 128) if label == "pairable" else (idx, cnt, 64)
        work = torch.arange(rcnt.size, dtype=torch.int32, device="cuda")
        o2, l2 = vsa.vsa_attn_fwd_worklist(qd, kd, vd, dev(ridx), dev(rcnt), rbq, bkv, work, scale, kv_valid=vald)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2), f"{label}: not the expected schedule's result"


def test_paired_forward_odd_tile_count_runs_native(vsa):
    B, H, S, D, bkv = 1, 2, 960, 64, 64
    say("paired forward with an odd number of 64-row tiles")
    q, k, v = W.qkv(B, S, H, D, seed=8)
    idx, cnt = W.random_csr(B, H, S // 64, S // bkv, S // bkv, 0, 6, seed=9)
    o, lse = vsa.vsa_attn_fwd_paired(dev(q), dev(k), dev(v), dev(idx), dev(cnt), bkv, 0.125)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, 64, bkv, 0.125)
    check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1), S, H,
               "paired odd nq")


COALESCED = [(bq, bkv, D, partial) for bq in (64, 128) for bkv in (64, 128) for D, partial in ((128, False), (64, True))]


@pytest.mark.parametrize("bq,bkv,D,partial", COALESCED,
                         ids=[f"q{a}_kv{b}_d{c}{'_partial' if p else ''}" for a, b, c, p in COALESCED])
def test_coalesced_forward_all_rows(vsa, bq, bkv, D, partial):
    """Lists expanded from 256-row logical blocks run as 256-row tiles, from
    128-row blocks as 128-row tiles, distinct lists natively: every row
    against the oracle, and bitwise equal to the schedule that must run (the
    unsplit kernel over the twice or once paired CSR, or over the input)."""
    B, H, S = 2, 2, 2048
    q, k, v = W.qkv(B, S, H, D, seed=bq + bkv + D + 91)
    qd, kd, vd = dev(q), dev(k), dev(v)
    scale = 1.0 / math.sqrt(D)
    val = None
    if partial:
        val = W.ragged_block_sizes(S // bkv, bkv, seed=bq + bkv + D, p_full=0.4)
        val[:2] = [0, 1]
    vald = None if val is None else dev(val)

    def expanded(lq, seed):
        mask = np.stack([W.anchor_uniform_mask(H, S // lq, S // 256, 3, seed=seed + b) for b in range(B)])
        idx, cnt, _ = ofront.mask_to_csr(mask, (lq, 256), (bq, bkv), 3 * (256 // bkv))
        return idx, cnt

    cases = [("q256", expanded(256, D + bkv), 256), ("q128", expanded(128, D + bkv + 3), 128),
             ("distinct", W.random_csr(B, H, S // bq, S // bkv, S // bkv, 0, S // bkv // 2, seed=D + bkv + bq), bq)]
    for label, (idx, cnt), rows in cases:
        idx = np.ascontiguousarray(idx[..., :max(1, int(cnt.max()))])
        # the schedule the device must choose, from the oracle's pairing
        ridx, rcnt, rbq = idx, cnt, bq
        while rbq < 256:
            pidx, pcnt, unp = ofront.pair_q_tiles(ridx, rcnt)
            if unp != 0:
                break
            ridx, rcnt, rbq = pidx, pcnt, rbq * 2
        assert rbq == (rows if rows >= bq else bq), f"{label}: unexpected pairing depth {rbq}"
        say(f"coalesced forward q{bq} {label} kv{bkv} D={D} partial={partial}: runs {rbq}-row tiles")
        o, lse = vsa.vsa_attn_fwd_coalesced(qd, kd, vd, dev(idx), dev(cnt), bq, bkv, scale, kv_valid=vald)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=val)
        check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1),
                   S, H, f"coalesced q{bq} {label} kv{bkv} D={D}")
        work = torch.arange(rcnt.size, dtype=torch.int32, device="cuda")
        o2, l2 = vsa.vsa_attn_fwd_worklist(qd, kd, vd, dev(np.ascontiguousarray(ridx)), dev(rcnt), rbq, bkv, work,
                                           scale, kv_valid=vald)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2), f"{label}: not the {rbq}-row schedule's result"


def test_coalesced_forward_without_256_row_tiles(vsa):
    """seqlen a multiple of 128 but not of 256: 64-row input falls back to the
    64 -> 128 pairing, 128-row input to vsa_attn_fwd; every row against the
    oracle and bitwise equal to those entry points."""
    B, H, S, D, bkv = 1, 2, 1152, 64, 64
    say("coalesced forward, seqlen 1152")
    q, k, v = W.qkv(B, S, H, D, seed=17)
    qd, kd, vd = dev(q), dev(k), dev(v)
    for bq in (64, 128):
        idx, cnt = W.random_csr(B, H, S // bq, S // bkv, 6, 0, 6, seed=18 + bq)
        o, lse = vsa.vsa_attn_fwd_coalesced(qd, kd, vd, dev(idx), dev(cnt), bq, bkv, 0.125)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, bq, bkv, 0.125)
        check_rows(o, lse, np.arange(B * H * S), o_ref.transpose(0, 2, 1, 3).reshape(-1, D), lse_ref.reshape(-1),
                   S, H, f"coalesced q{bq} seqlen {S}")
        if bq == 64:
            o2, l2 = vsa.vsa_attn_fwd_paired(qd, kd, vd, dev(idx), dev(cnt), bkv, 0.125)
        else:
            o2, l2 = vsa.vsa_attn_fwd(qd, kd, vd, dev(idx), dev(cnt), bq, bkv, 0.125)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_tensors_past_2gib_sampled(vsa):
    """B=12, S=32k, H=24, D=128: Q, K, V and O are 2.4 GB each, so the rows of
    the last batches sit past 2^31 bytes. Sampled rows of the first and last
    batch against the oracle (inputs drawn on the device with a seeded
    generator and copied back for the oracle)."""
    B, S, H, D, bq, bkv = 12, 32768, 24, 128, 256, 128
    say("forward past 2 GiB: generating inputs")
    g = torch.Generator(device="cuda").manual_seed(2024)

    def draw():
        x = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
        for b in range(B):  # one batch at a time keeps the fp32 temporary small
            x[b] = torch.randn((S, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        return x

    q, k, v = draw(), draw(), draw()
    assert q.numel() * 2 > 2 ** 31
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, 12, 1, 12, seed=2025)
    scale = 1.0 / math.sqrt(D)
    say("forward past 2 GiB: kernel")
    o, lse = _run_fwd(vsa, q, k, v, dev(idx), dev(cnt), bq, bkv, scale)
    rows = [r for r in sample_rows(B, H, S, bq, 1, seed=7) if r // (S * H) in (0, B - 1)]
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    o_ref, lse_ref = oracle.attn_rows(qc, kc, vc, idx, cnt, bq, bkv, scale, rows)
    check_rows(o, lse, rows, o_ref, lse_ref, S, H, "past 2 GiB")
    del q, k, v, o, lse, qc, kc, vc
    torch.cuda.empty_cache()
