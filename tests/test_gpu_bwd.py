"""GPU parity of the backward pass (dQ, dK, dV) and the Q-direction CSR
against the CPU oracle, through the C ABI.

The oracle recomputes the forward from q, k, v and the mask; the GPU
backward uses the GPU forward's O and LSE, as a caller would. Tolerances
(bf16 gradients compared after conversion to fp32, against fp32 oracle
gradients): max |d| <= 2e-2 * max(1, max |ref|) and mean |d| <= 2e-3 *
max(1, mean |ref|) per tensor -- the forward's bounds scaled to the
gradient's magnitude: bf16 rounding of the output (2^-9 relative) and of P
and dS inside the MFMA products (2^-9 relative per term, averaging over the
sums) keep the error well inside them. Integer outputs are bit-exact.
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

G_MAX = 2e-2
G_MEAN = 2e-3


def say(msg):
    line = f"[gpu-bwd] {msg}"
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


def check(name, got, ref, label):
    d = np.abs(got - ref)
    mx, mean = float(d.max()), float(d.mean())
    rmax, rmean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    say(f"{label} {name}: max|d|={mx:.3e} (ref max {rmax:.3e}) mean|d|={mean:.3e} (ref mean {rmean:.3e})")
    assert np.isfinite(got).all(), f"{label} {name}: non-finite"
    assert mx <= G_MAX * max(1.0, rmax), f"{label} {name}: max |d| {mx}"
    assert mean <= G_MEAN * max(1.0, rmean), f"{label} {name}: mean |d| {mean}"


TRANSPOSE_CASES = [
    ("random", None),
    ("vsa256 256x128", (W.VSA256, (256, 128), 26)),
    ("native64", (W.NATIVE64, (64, 64), 92)),
]


@pytest.mark.parametrize("label,spec", TRANSPOSE_CASES, ids=[c[0] for c in TRANSPOSE_CASES])
def test_csr_transpose_bit_exact(vsa, label, spec):
    say(f"csr_transpose {label}")
    if spec is None:
        B, H, NQ, NKV = 2, 3, 40, 24
        idx, cnt = W.random_csr(B, H, NQ, NKV, NKV, 0, NKV, seed=17)
        cnt[0, 0, 0] = 0
        idx[1, 2, 3, 0] = -4  # out-of-range entry: ignored
        idx[1, 2, 3, 1] = NKV + 3
    else:
        wl, shape, ld = spec
        idx, cnt, _ = ofront.mask_to_csr(wl.logical_mask(), wl.logical_block, shape, ld)
        NQ, NKV = idx.shape[2], wl.seqlen // shape[1]
    clean_idx = idx.copy()
    # the oracle takes valid rows only: drop out-of-range entries (the kernel ignores them)
    clean_cnt = cnt.copy()
    for pos in np.ndindex(cnt.shape):
        ent = [t for t in idx[pos][:cnt[pos]] if 0 <= t < NKV]
        clean_idx[pos][:len(ent)] = ent
        clean_cnt[pos] = len(ent)
    q_ld = NQ
    ref_idx, ref_cnt, ref_ovf = ofront.transpose_csr(clean_idx, clean_cnt, NKV, q_ld)
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    q_idx, q_cnt = vsa.vsa_csr_transpose(dev(idx), dev(cnt), NKV, q_ld, overflow=ovf)
    torch.cuda.synchronize()
    assert np.array_equal(q_cnt.cpu().numpy(), ref_cnt)
    valid = np.arange(q_ld)[None, None, None, :] < ref_cnt[..., None]
    assert np.array_equal(np.where(valid, q_idx.cpu().numpy(), -1), np.where(valid, ref_idx, -1))
    assert bool(ovf.item()) == ref_ovf
    # compact row length: counts stay true, overflow is flagged
    small = max(1, int(ref_cnt.max()) - 1)
    ovf.zero_()
    _, c2 = vsa.vsa_csr_transpose(dev(idx), dev(cnt), NKV, small, overflow=ovf)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), ref_cnt) and ovf.item() == 1


def _run_bwd(vsa, q, k, v, do, idx, cnt, bq, bkv, scale, kv_valid=None):
    B, S, H, D = q.shape
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    idxd, cntd = dev(idx), dev(cnt)
    vd_valid = None if kv_valid is None else dev(kv_valid)
    o, lse = vsa.vsa_attn_fwd(qd, kd, vd, idxd, cntd, bq, bkv, scale, kv_valid=vd_valid)
    nkv = S // bkv
    q_idx, q_cnt = vsa.vsa_csr_transpose(idxd, cntd, nkv, S // bq)
    dq, dk, dv = vsa.vsa_attn_bwd(qd, kd, vd, o, lse, dod, idxd, cntd, q_idx, q_cnt, bq, bkv, scale,
                                  kv_valid=vd_valid)
    torch.cuda.synchronize()
    return dq, dk, dv


BWD_SHAPES = [(bq, bkv, d) for bq in (64, 128, 256) for bkv in (64, 128) for d in (64, 128)]


@pytest.fixture
def max_splits(vsa, request):
    """Cap on split lists for the test (restored afterwards)."""
    prev = vsa.vsa_set_max_splits(request.param)
    yield request.param
    vsa.vsa_set_max_splits(prev)


@pytest.mark.parametrize("bq,bkv,D", BWD_SHAPES, ids=[f"{a}x{b}_d{c}" for a, b, c in BWD_SHAPES])
@pytest.mark.parametrize("partial", [False, True], ids=["full", "partial"])
@pytest.mark.parametrize("max_splits", [4, 1], ids=["split", "unsplit"], indirect=True)
def test_backward_every_tile_shape_all_rows(vsa, bq, bkv, D, partial, max_splits):
    """At this size every list is split (four parts) unless max_splits is 1."""
    B, H, S = 1, 2, 768
    label = f"{bq}x{bkv} D={D} {'partial' if partial else 'full'} max_splits={max_splits}"
    say(f"backward {label}")
    q, k, v = W.qkv(B, S, H, D, seed=bq + bkv + D + 100)
    do = W.qkv(B, S, H, D, seed=bq + bkv + D + 101)[0]
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=bq * 3 + bkv + D)
    cnt[0, 0, 0] = 0  # an empty query tile
    val = None
    if partial:
        val = W.ragged_block_sizes(nkv, bkv, seed=bq + bkv + D, p_full=0.4)
        val[0] = 0
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = _run_bwd(vsa, q, k, v, do, idx, cnt, bq, bkv, scale, val)
    rq, rk, rv = oracle.bwd_full(q, k, v, do, idx, cnt, bq, bkv, scale, kv_valid=val)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check(name, got.float().cpu().numpy(), ref, label)


@pytest.mark.parametrize("max_splits", [4, 1], ids=["split", "unsplit"], indirect=True)
def test_backward_is_deterministic(vsa, max_splits):
    """Two runs agree bit for bit, with split lists (the last part to finish
    sums all parts in part order) and without."""
    B, H, S, D, bq, bkv = 1, 2, 1024, 128, 128, 64
    say(f"backward determinism max_splits={max_splits}")
    q, k, v = W.qkv(B, S, H, D, seed=7)
    do = W.qkv(B, S, H, D, seed=8)[0]
    idx, cnt = W.random_csr(B, H, S // bq, S // bkv, S // bkv, 1, 12, seed=9)
    a = _run_bwd(vsa, q, k, v, do, idx, cnt, bq, bkv, 0.09)
    b = _run_bwd(vsa, q, k, v, do, idx, cnt, bq, bkv, 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_dense_backward_split_lists_every_row(vsa):
    """Dense S=4k at 128x128 (256 query and 256 KV tiles: split in two on a
    256-CU GPU): dQ, dK and dV of every row against the oracle."""
    wl = W.DENSE
    say("dense backward 128x128: inputs")
    q, k, v = wl.qkv()
    do = W.qkv(wl.batch, wl.seqlen, wl.heads, wl.head_dim, seed=4243)[0]
    idx, cnt, _ = ofront.mask_to_csr(wl.logical_mask(), wl.logical_block, (128, 128), 32)
    dq, dk, dv = _run_bwd(vsa, q, k, v, do, idx, cnt, 128, 128, wl.scale)
    say("dense backward 128x128: oracle, every row")
    rq, rk, rv = oracle.bwd_full(q, k, v, do, idx, cnt, 128, 128, wl.scale)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check(name, got.float().cpu().numpy(), ref, "dense split every row")


FULL_SIZE = [
    # label, workload, tile, idx_ld, heads compared on every row
    ("vsa256 256x128", W.VSA256, (256, 128), 26, (0, 23)),
    ("vsa256 64x64", W.VSA256_FINE, (64, 64), 52, (7,)),
    ("native64 64x64", W.NATIVE64, (64, 64), 92, (16,)),
    ("vsa256 d64 256x128", W.VSA256_D64, (256, 128), 26, (40,)),
]


@pytest.mark.parametrize("label,wl,tile,ld,heads", FULL_SIZE, ids=[c[0] for c in FULL_SIZE])
def test_backward_full_size_whole_heads(vsa, label, wl, tile, ld, heads):
    """Full-size workloads (B1 S32768, H24 at D128, H48 at D64): the GPU runs every head; dQ,
    dK and dV of whole heads (every one of their 32768 query and key rows)
    are compared with the oracle run on those heads alone (heads are
    independent, so this is the same computation)."""
    say(f"backward {label}: inputs")
    q, k, v = wl.qkv()
    do = W.qkv(wl.batch, wl.seqlen, wl.heads, wl.head_dim, seed=4242)[0]
    idx, cnt, _ = ofront.mask_to_csr(wl.logical_mask(), wl.logical_block, tile, ld)
    say(f"backward {label}: kernels")
    dq, dk, dv = _run_bwd(vsa, q, k, v, do, idx, cnt, tile[0], tile[1], wl.scale)
    for h in heads:
        say(f"backward {label}: oracle, head {h}, every row")
        sl = [t[:, :, h:h + 1].contiguous() for t in (q, k, v, do)]
        rq, rk, rv = oracle.bwd_full(*sl, idx[:, h:h + 1], cnt[:, h:h + 1], tile[0], tile[1], wl.scale)
        for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            check(name, got[:, :, h:h + 1].float().cpu().numpy(), ref, f"{label} head {h} every row")
    del dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tile", [(256, 128), (64, 64)], ids=["256x128", "64x64"])
def test_backward_with_empty_tiles_dropped(vsa, tile):
    """Ragged KV blocks with tiles left out of the lists by the front-end:
    dQ, dK, dV of every row against the oracle (which lists every selected
    tile; keys of a dropped tile get zero gradients)."""
    B, H, S, D = 1, 2, 2048, 128
    say(f"backward, empty tiles dropped, {tile}")
    q, k, v = W.qkv(B, S, H, D, seed=510 + tile[0])
    do = W.qkv(B, S, H, D, seed=511 + tile[0])[0]
    mask = W.anchor_uniform_mask(H, S // 256, S // 256, 4, seed=512)[None]
    vbs = W.ragged_block_sizes(S // 256, 256, seed=513)
    vbs[:2] = [0, 100]
    val = ofront.expand_valid(vbs, 256, tile[1])
    ld = 4 * (256 // tile[1])
    idx, cnt, _ = ofront.mask_to_csr(mask, (256, 256), tile, ld)
    didx, dcnt = vsa.vsa_mask_to_csr(dev(mask), (256, 256), tile, ld, kv_valid=dev(val))
    torch.cuda.synchronize()
    assert int(dcnt.sum()) < int(cnt.sum())
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = _run_bwd(vsa, q, k, v, do, didx.cpu().numpy(), dcnt.cpu().numpy(), tile[0], tile[1], scale, val)
    rq, rk, rv = oracle.bwd_full(q, k, v, do, idx, cnt, tile[0], tile[1], scale, kv_valid=val)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check(name, got.float().cpu().numpy(), ref, f"dropped {tile}")


@pytest.mark.parametrize("bq,bkv,D", [(256, 128, 64), (128, 64, 64), (64, 64, 64), (256, 128, 128), (128, 128, 128),
                                      (64, 128, 128)])
def test_maximum_list_stride_and_empty_head(vsa, bq, bkv, D):
    """idx_ld = q_ld = 8191 (the largest accepted; the kernels stage whole
    rows, and the backward then needs more than 64 KB of LDS; at D=128 the
    256-row forward fills the whole 160 KB of a compute unit's LDS), with
    every row of head 1 empty: forward and backward against the oracle on all
    rows."""
    B, H, S = 1, 2, 1024
    say(f"maximum list stride {bq}x{bkv} D={D}")
    q, k, v = W.qkv(B, S, H, D, seed=bq + bkv + 3)
    do = W.qkv(B, S, H, D, seed=bq + bkv + 4)[0]
    nq, nkv = S // bq, S // bkv
    idx_c, cnt = W.random_csr(B, H, nq, nkv, nkv, 1, nkv, seed=bq + bkv + 5)
    cnt[0, 1, :] = 0
    LD = 8191
    idx = np.full((B, H, nq, LD), -1, dtype=np.int32)
    idx[..., :nkv] = idx_c
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx_c, cnt, bq, bkv, scale)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    idxd, cntd = dev(idx), dev(cnt)
    o, lse = vsa.vsa_attn_fwd(qd, kd, vd, idxd, cntd, bq, bkv, scale)
    torch.cuda.synchronize()
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.all(og[0, :, 1] == 0.0) and np.all(np.isneginf(lg[0, 1]))
    d = np.abs(og - o_ref)  # both [B, S, H, D]
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lg))
    assert (np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))).max() <= 1e-3
    q_idx, q_cnt = vsa.vsa_csr_transpose(idxd, cntd, nkv, LD)
    dq, dk, dv = vsa.vsa_attn_bwd(qd, kd, vd, o, lse, dod, idxd, cntd, q_idx, q_cnt, bq, bkv, scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd_full(q, k, v, do, idx_c, cnt, bq, bkv, scale)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check(name, got.float().cpu().numpy(), ref, f"max stride {bq}x{bkv} D={D}")
        assert np.all(got.float().cpu().numpy()[0, :, 1] == 0.0)


def test_backward_tensors_past_2gib_sampled(vsa):
    """B=12, S=32k, H=24, D=128 (Q, K, V, dO and the gradients 2.4 GB each):
    sampled dQ and dK/dV rows of the last batch, past 2^31 bytes, against
    the oracle (inputs drawn on the device with a seeded generator)."""
    B, S, H, D, bq, bkv = 12, 32768, 24, 128, 256, 128
    say("backward past 2 GiB: inputs")
    g = torch.Generator(device="cuda").manual_seed(4048)

    def draw():
        x = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            x[b] = torch.randn((S, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        return x

    q, k, v, do = draw(), draw(), draw(), draw()
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, 12, 1, 12, seed=4049)
    scale = 1.0 / math.sqrt(D)
    idxd, cntd = dev(idx), dev(cnt)
    say("backward past 2 GiB: kernels")
    o, lse = vsa.vsa_attn_fwd(q, k, v, idxd, cntd, bq, bkv, scale)
    q_idx, q_cnt = vsa.vsa_csr_transpose(idxd, cntd, nkv, nq)
    dq, dk, dv = vsa.vsa_attn_bwd(q, k, v, o, lse, do, idxd, cntd, q_idx, q_cnt, bq, bkv, scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    b = B - 1
    qrows = np.array([(b * H + h) * S + r for h in (0, 23) for r in rng.integers(0, S, size=16)], dtype=np.int64)
    krows = np.array([(b * H + h) * S + r for h in (0, 23) for r in rng.integers(0, S, size=3)], dtype=np.int64)
    qc, kc, vc, doc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    say("backward past 2 GiB: oracle rows")
    rq = oracle.bwd_dq_rows(qc, kc, vc, doc, idx, cnt, bq, bkv, scale, qrows)
    rk, rv = oracle.bwd_dkv_rows(qc, kc, vc, doc, idx, cnt, bq, bkv, scale, krows)

    def pick(t, rows):
        bh, i = rows // S, rows % S
        return t[torch.as_tensor(bh // H), torch.as_tensor(i), torch.as_tensor(bh % H)].float().cpu().numpy()

    check("dQ", pick(dq, qrows), rq, "past 2 GiB")
    check("dK", pick(dk, krows), rk, "past 2 GiB")
    check("dV", pick(dv, krows), rv, "past 2 GiB")
    del q, k, v, do, o, lse, dq, dk, dv, qc, kc, vc, doc
    torch.cuda.empty_cache()


def _views(t, layout):
    """A [B, S, H, D] device tensor's values as a strided view: sliced from a
    packed [B, S, 3, H, D] buffer, from a [B, H, S, D] buffer, or head 0
    broadcast over the heads (head stride 0)."""
    B, S, H, D = t.shape
    if layout == "packed":
        buf = torch.zeros((B, S, 3, H, D), dtype=t.dtype, device=t.device)
        buf[:, :, 1] = t
        return buf[:, :, 1]
    if layout == "bhsd":
        return t.transpose(1, 2).contiguous().transpose(1, 2)
    assert layout == "broadcast"
    return t[:, :, :1].expand(B, S, H, D)


STRIDED_BWD = [(256, 128, 128, "packed", "packed", "bhsd", False), (128, 64, 64, "bhsd", "bhsd", "packed", False),
               (64, 64, 128, "packed", "broadcast", "bhsd", False), (256, 64, 64, "bhsd", "broadcast", "packed", False),
               (128, 128, 128, "packed", "packed", "packed", False), (256, 128, 64, "packed", "bhsd", "bhsd", True),
               (64, 64, 64, "bhsd", "packed", "packed", True)]


@pytest.mark.parametrize("bq,bkv,D,qlay,kvlay,dolay,partial", STRIDED_BWD,
                         ids=[f"{a}x{b}_d{c}_{q}_{kv}_{d}{'_partial' if pt else ''}"
                              for a, b, c, q, kv, d, pt in STRIDED_BWD])
@pytest.mark.parametrize("max_splits", [4, 1], ids=["split", "unsplit"], indirect=True)
def test_strided_backward_bitwise_equal_to_contiguous(vsa, bq, bkv, D, qlay, kvlay, dolay, partial, max_splits):
    """q, k, v and dout read in place through their strides
    (vsa_attn_bwd_strided, the route vsa_attn_bwd takes for views) give the
    gradients of the contiguous call on copies of the same values bitwise,
    with full and partial tiles; some cases are also checked against the
    oracle."""
    B, H, S = 2, 2, 768
    say(f"strided backward {bq}x{bkv} D={D} q:{qlay} kv:{kvlay} dout:{dolay} partial={partial} "
        f"max_splits={max_splits}")
    q, k, v = (dev(t) for t in W.qkv(B, S, H, D, seed=bq + bkv + D + 300))
    do = dev(W.qkv(B, S, H, D, seed=bq + bkv + D + 301)[0])
    qs, ks, vs, dos = _views(q, qlay), _views(k, kvlay), _views(v, kvlay), _views(do, dolay)
    qc, kc, vc, doc = qs.contiguous(), ks.contiguous(), vs.contiguous(), dos.contiguous()
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=bq * 9 + bkv + D)
    idxd, cntd = dev(idx), dev(cnt)
    val = W.ragged_block_sizes(nkv, bkv, seed=bq + bkv + D + 7, p_full=0.4) if partial else None
    vd = None if val is None else dev(val)
    scale = 1.0 / math.sqrt(D)
    o, lse = vsa.vsa_attn_fwd(qc, kc, vc, idxd, cntd, bq, bkv, scale, kv_valid=vd)
    q_idx, q_cnt = vsa.vsa_csr_transpose(idxd, cntd, nkv, nq)
    ref = vsa.vsa_attn_bwd(qc, kc, vc, o, lse, doc, idxd, cntd, q_idx, q_cnt, bq, bkv, scale, kv_valid=vd)
    got = vsa.vsa_attn_bwd(qs, ks, vs, o, lse, dos, idxd, cntd, q_idx, q_cnt, bq, bkv, scale, kv_valid=vd)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"strided {name} differs from the contiguous call"
    if max_splits == 4 and (partial or (qlay, kvlay) in (("packed", "packed"), ("packed", "broadcast"))):
        rq, rk, rv = oracle.bwd_full(qc.cpu(), kc.cpu(), vc.cpu(), doc.cpu(), idx, cnt, bq, bkv, scale, kv_valid=val)
        for name, g, r in (("dQ", got[0], rq), ("dK", got[1], rk), ("dV", got[2], rv)):
            check(name, g.float().cpu().numpy(), r, f"strided {bq}x{bkv}")
