"""vsa_attn_fwd_noalloc captured in a HIP graph (the use it exists for):
the graph is replayed several times, with eager work between the replays
that rewrites the library's fixed scratch array (another no-alloc call on a
different problem) and its per-stream buffers (vsa_attn_fwd), and every
replay must reproduce the eager no-alloc result bit for bit. The cases use
split lists, whose per-item counters must be back at zero when each replay
starts."""

import math

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-graph] {msg}", flush=True)


@pytest.fixture(scope="module")
def vsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flashattention_amd as m

    m.load_library()
    return m


def _problem(B, H, S, D, bq, bkv, seed):
    q, k, v = (t.to("cuda") for t in W.qkv(B, S, H, D, seed=seed))
    nq, nkv = S // bq, S // bkv
    idx, cnt = W.random_csr(B, H, nq, nkv, nkv, 0, nkv, seed=seed + 1)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")  # noqa: E731
    return dict(q=q, k=k, v=v, idx=dev(idx), cnt=dev(cnt), bq=bq, bkv=bkv, scale=1.0 / math.sqrt(D),
                o=torch.empty_like(q), lse=torch.empty((B, H, S), dtype=torch.float32, device="cuda"))


def _noalloc(vsa, p, o=None, lse=None):
    return vsa.vsa_attn_fwd_noalloc(p["q"], p["k"], p["v"], p["idx"], p["cnt"], p["bq"], p["bkv"], p["scale"],
                                    p["o"] if o is None else o, p["lse"] if lse is None else lse)


# (B, H, S, D, bq, bkv): few query tiles, so lists are split over workgroups
CASES = [(1, 2, 2048, 128, 256, 128), (2, 3, 2048, 64, 64, 64), (1, 1, 4096, 128, 128, 64)]


@pytest.mark.parametrize("B,H,S,D,bq,bkv", CASES, ids=[f"{c[4]}x{c[5]}_d{c[3]}" for c in CASES])
def test_noalloc_forward_replays_in_a_hip_graph(vsa, B, H, S, D, bq, bkv):
    say(f"graph capture {bq}x{bkv} D={D}")
    p = _problem(B, H, S, D, bq, bkv, seed=bq + bkv + D)
    other = _problem(2, 2, 1024, D, bq, bkv, seed=bq + bkv + D + 7)   # rewrites the scratch array
    third = _problem(1, 2, 1024, D, bq, bkv, seed=bq + bkv + D + 9)   # goes through vsa_attn_fwd
    # eager reference (this also takes the scratch array's address and clears its counters outside capture)
    _noalloc(vsa, p)
    torch.cuda.synchronize()
    o_ref, lse_ref = p["o"].clone(), p["lse"].clone()

    o_g, lse_g = torch.empty_like(p["o"]), torch.empty_like(p["lse"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc(vsa, p, o_g, lse_g)
    for r in range(4):
        o_g.fill_(0)
        lse_g.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(lse_g, lse_ref), f"replay {r} differs from the eager call"
        # eager work between replays
        _noalloc(vsa, other)
        vsa.vsa_attn_fwd(third["q"], third["k"], third["v"], third["idx"], third["cnt"], bq, bkv, third["scale"],
                         third["o"], third["lse"])
        torch.cuda.synchronize()
    say(f"graph capture {bq}x{bkv} D={D}: 4 replays bitwise equal to the eager call")
