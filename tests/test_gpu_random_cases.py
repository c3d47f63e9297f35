"""GPU parity on seeded random problems: every forward entry point, and the
backward, against the CPU oracle on every row.

Each case draws its sizes (batch, heads, sequence length, head_dim), its tile
shape, its lists (density, empty and full rows, shuffled order), whether KV
tiles are partial (ragged valid key counts), the softmax scale and the entry
point (vsa_attn_fwd, the work-list kernel, strided q/k/v views, the no-alloc
entry, the paired and coalesced entries where the tile shape allows), so that
combinations no hand-written case names still meet the oracle. The backward
cases draw the same way and run the transposed lists and vsa_attn_bwd on the
GPU forward's O and LSE (on strided views of packed buffers where the case draws
the strided entry). Tolerances as in test_gpu_parity.py and test_gpu_bwd.py.
"""

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
N_CASES = 400
N_BWD_CASES = 120
G_MAX = 2e-2
G_MEAN = 2e-3


def say(msg):
    line = f"[gpu-random] {msg}"
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


def draw_case(i):
    """Sizes, tiles, lists and entry point of case i (a pure function of i)."""
    rng = np.random.default_rng(1000 + i)
    D = int(rng.choice([64, 128]))
    bq = int(rng.choice([64, 128, 256]))
    bkv = int(rng.choice([64, 128]))
    S = 256 * int(rng.integers(1, 9))          # 256 .. 2048
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 6))
    nq, nkv = S // bq, S // bkv
    lo = int(rng.integers(0, nkv + 1))
    hi = int(rng.integers(lo, nkv + 1))
    partial = bool(rng.random() < 0.3)
    scale = float(rng.uniform(0.5, 2.0) / math.sqrt(D))
    entries = ["fwd", "worklist", "strided", "noalloc"]
    if bq in (64, 128):
        entries.append("coalesced")
    if bq == 64:
        entries.append("paired")
    entry = str(rng.choice(entries))
    return dict(D=D, bq=bq, bkv=bkv, S=S, B=B, H=H, nq=nq, nkv=nkv, lo=lo, hi=hi, partial=partial, scale=scale,
                entry=entry, seed=int(rng.integers(1 << 30)))


def run_entry(vsa, c, q, k, v, idx, cnt, valid):
    bq, bkv, scale, entry = c["bq"], c["bkv"], c["scale"], c["entry"]
    if entry == "fwd":
        return vsa.vsa_attn_fwd(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=valid)
    if entry == "worklist":
        work = vsa.vsa_build_worklist(cnt, idx.shape[3])
        return vsa.vsa_attn_fwd_worklist(q, k, v, idx, cnt, bq, bkv, work, scale, kv_valid=valid)
    if entry == "strided":
        buf = torch.stack((q, k, v), dim=2).contiguous()  # packed [B, S, 3, H, D]
        return vsa.vsa_attn_fwd(buf[:, :, 0], buf[:, :, 1], buf[:, :, 2], idx, cnt, bq, bkv, scale, kv_valid=valid)
    if entry == "noalloc":
        return vsa.vsa_attn_fwd_noalloc(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=valid)
    if entry == "coalesced":
        return vsa.vsa_attn_fwd_coalesced(q, k, v, idx, cnt, bq, bkv, scale, kv_valid=valid)
    assert entry == "paired"
    return vsa.vsa_attn_fwd_paired(q, k, v, idx, cnt, bkv, scale, kv_valid=valid)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_every_row(vsa, i):
    c = draw_case(i)
    B, H, S, D, nq, nkv = c["B"], c["H"], c["S"], c["D"], c["nq"], c["nkv"]
    say(f"case {i}: B{B} H{H} S{S} D{D} {c['bq']}x{c['bkv']} counts {c['lo']}..{c['hi']} "
        f"partial={c['partial']} entry={c['entry']}")
    q, k, v = W.qkv(B, S, H, D, seed=c["seed"])
    idx, cnt = W.random_csr(B, H, nq, nkv, max(c["hi"], 1), c["lo"], c["hi"], seed=c["seed"] + 1)
    valid = None
    if c["partial"]:
        valid = W.ragged_block_sizes(nkv, c["bkv"], seed=c["seed"] + 2, p_full=0.3)
    o_ref, lse_ref = oracle.attn_full(q, k, v, idx, cnt, c["bq"], c["bkv"], c["scale"], kv_valid=valid)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")  # noqa: E731
    o, lse = run_entry(vsa, c, q.to("cuda"), k.to("cuda"), v.to("cuda"), dev(idx), dev(cnt),
                       None if valid is None else dev(valid))
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lg)), f"case {i}: LSE finiteness differs"
    assert np.all(og.transpose(0, 2, 1, 3)[~fin] == 0.0), f"case {i}: rows without keys must have O=0"
    d = np.abs(og - o_ref)
    assert d.max() <= O_MAX_ABS and d.mean() <= O_MEAN_ABS, f"case {i}: max |dO| {d.max()} mean {d.mean()}"
    if fin.any():
        rel = np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        assert rel.max() <= LSE_REL, f"case {i}: LSE rel {rel.max()}"


@pytest.mark.parametrize("i", range(N_BWD_CASES))
def test_random_backward_case_every_row(vsa, i):
    c = draw_case(5000 + i)
    B, H, S, D, nq, nkv, bq, bkv = c["B"], c["H"], c["S"], c["D"], c["nq"], c["nkv"], c["bq"], c["bkv"]
    say(f"backward case {i}: B{B} H{H} S{S} D{D} {bq}x{bkv} counts {c['lo']}..{c['hi']} partial={c['partial']}")
    q, k, v = W.qkv(B, S, H, D, seed=c["seed"])
    do = W.qkv(B, S, H, D, seed=c["seed"] + 3)[0]
    idx, cnt = W.random_csr(B, H, nq, nkv, max(c["hi"], 1), c["lo"], c["hi"], seed=c["seed"] + 1)
    valid = None
    if c["partial"]:
        valid = W.ragged_block_sizes(nkv, bkv, seed=c["seed"] + 2, p_full=0.3)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")  # noqa: E731
    qd, kd, vd, dod = q.to("cuda"), k.to("cuda"), v.to("cuda"), do.to("cuda")
    if c["entry"] == "strided":
        # q, k, v as slices of a packed [B, S, 3, H, D] buffer and dO as one of a [B, S, 2, H, D]
        # buffer: both passes read them in place through their strides
        buf = torch.stack((qd, kd, vd), dim=2).contiguous()
        qd, kd, vd = buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
        dod = torch.stack((dod, torch.zeros_like(dod)), dim=2).contiguous()[:, :, 0]
    idxd, cntd = dev(idx), dev(cnt)
    vv = None if valid is None else dev(valid)
    o, lse = vsa.vsa_attn_fwd(qd, kd, vd, idxd, cntd, bq, bkv, c["scale"], kv_valid=vv)
    q_idx, q_cnt = vsa.vsa_csr_transpose(idxd, cntd, nkv, nq)
    dq, dk, dv = vsa.vsa_attn_bwd(qd, kd, vd, o, lse, dod, idxd, cntd, q_idx, q_cnt, bq, bkv, c["scale"],
                                  kv_valid=vv)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd_full(q, k, v, do, idx, cnt, bq, bkv, c["scale"], kv_valid=valid)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        g = got.float().cpu().numpy()
        d = np.abs(g - ref)
        assert np.isfinite(g).all(), f"backward case {i} {name}: non-finite"
        assert d.max() <= G_MAX * max(1.0, float(np.abs(ref).max())), f"backward case {i} {name}: max |d| {d.max()}"
        assert d.mean() <= G_MEAN * max(1.0, float(np.abs(ref).mean())), \
            f"backward case {i} {name}: mean |d| {d.mean()}"
