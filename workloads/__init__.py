"""Seeded synthetic inputs for block-sparse attention: Q/K/V and block masks.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark. It holds only input recipes (random draws and the mask sampler);
none of the attention arithmetic, the mask expansion, the CSR build or the
work-list ordering lives here.

Recipes follow the FastVideo "[perf] Add fine-grained FA4 VSA kernels" page,
file ``benchmarks/bench_vsa_blackwell.py``:

* Q/K/V are i.i.d. standard normal values rounded to bf16, one draw per tensor
  in the order q, k, v (section ``main``, the per-sequence-length draw). The
  page draws on the CUDA device; here the draw is on a CPU generator so the
  values do not depend on the GPU vendor's RNG stream.
* A logical block mask keeps, in every Q-block row, the "diagonal anchor"
  KV block floor(q*NKV/NQ) plus ``keep-1`` further blocks chosen uniformly
  without replacement (what the page's ``make_logical_mask`` selects; drawn
  here with numpy's ``Generator.choice``, one call per row).
* The mask seed is ``seed + seq_len + int(keep_fraction*1000)``, plus
  ``q_block*1_000_003 + kv_block*9_176`` when a shape is sampled natively
  rather than expanded from a 256x256 base (section ``main``).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DEFAULT_SEED = 42


def qkv(batch: int, seqlen: int, heads: int, head_dim: int, seed: int = DEFAULT_SEED):
    """Return bf16 CPU tensors q, k, v of shape [B, S, H, D], i.i.d. N(0,1)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    out = []
    for _ in range(3):
        t = torch.randn(batch, seqlen, heads, head_dim, dtype=torch.float32, generator=g)
        out.append(t.to(torch.bfloat16))
    return tuple(out)


def _anchor_plus_uniform(rng: np.random.Generator, nq: int, nkv: int, counts: np.ndarray) -> np.ndarray:
    """Rows of a logical block mask, one per entry of ``counts`` [H, NQ].

    Row (h, r) keeps its diagonal anchor block a = floor(r*NKV/NQ) and
    counts[h, r] - 1 further blocks drawn uniformly without replacement from
    the NKV - 1 blocks other than a (one ``Generator.choice`` per row, rows in
    (h, r) order).
    """
    heads = counts.shape[0]
    m = np.zeros((heads, nq, nkv), dtype=np.uint8)
    for h in range(heads):
        for r in range(nq):
            a = (r * nkv) // nq
            picks = rng.choice(nkv - 1, size=int(counts[h, r]) - 1, replace=False)
            picks = picks + (picks >= a)  # positions 0..NKV-2 of the non-anchor blocks
            m[h, r, a] = 1
            m[h, r, picks] = 1
    return m


def anchor_uniform_mask(heads: int, nq: int, nkv: int, keep: int, seed: int) -> np.ndarray:
    """[H, NQ, NKV] uint8 mask: every row keeps ``keep`` blocks, its diagonal
    anchor and keep-1 others chosen uniformly without replacement (the
    selection the FastVideo page's ``make_logical_mask`` describes: anchor
    always kept, the rest a uniform draw)."""
    if keep < 1 or keep > nkv:
        raise ValueError(f"cannot keep {keep} blocks in a row of {nkv}")
    rng = np.random.default_rng(seed)
    return _anchor_plus_uniform(rng, nq, nkv, np.full((heads, nq), keep, dtype=np.int64))


def anchor_count_mask(heads: int, nq: int, nkv: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """[H, NQ, NKV] uint8 mask whose per-row kept count is U{lo..hi}.

    The count of every (head, Q-block) row is drawn independently and
    uniformly from the integers lo..hi inclusive (one draw of all counts
    first); the row then keeps its diagonal anchor plus count-1 further
    blocks chosen uniformly without replacement, as in anchor_uniform_mask.
    """
    if not 1 <= lo <= hi <= nkv:
        raise ValueError(f"row counts {lo}..{hi} do not fit rows of {nkv} blocks")
    rng = np.random.default_rng(seed)
    counts = rng.integers(lo, hi + 1, size=(heads, nq))
    return _anchor_plus_uniform(rng, nq, nkv, counts)


def mask_seed(seed: int, seqlen: int, keep_fraction: float, native_shape=None) -> int:
    """Mask seed rule of the FastVideo benchmark (section ``main``)."""
    s = seed + seqlen + int(keep_fraction * 1000)
    if native_shape is not None:
        qb, kb = native_shape
        s += qb * 1_000_003 + kb * 9_176
    return s


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem: sizes, the logical mask grid and physical tiles.

    ``logical_block`` is the (Q, KV) token size of one logical mask cell;
    ``physical`` lists the (block_q, block_kv) tile shapes the forward pass
    runs this mask at (each must divide the logical block).
    """

    name: str
    batch: int
    heads: int
    seqlen: int
    head_dim: int
    logical_block: tuple
    physical: tuple
    mask_kind: str            # "topk", "dense" or "count"
    keep: int = 0             # for "topk"
    count_range: tuple = (0, 0)  # for "count"
    keep_fraction: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def nq_logical(self) -> int:
        return self.seqlen // self.logical_block[0]

    @property
    def nkv_logical(self) -> int:
        return self.seqlen // self.logical_block[1]

    def mask_seed(self, seed: int = DEFAULT_SEED) -> int:
        native = None if self.logical_block == (256, 256) else self.logical_block
        return mask_seed(seed, self.seqlen, self.keep_fraction, native)

    def logical_mask(self, seed: int = DEFAULT_SEED) -> np.ndarray:
        """[B, H, NQ_l, NKV_l] uint8 logical mask (same pattern for every b)."""
        nq, nkv = self.nq_logical, self.nkv_logical
        if self.mask_kind == "dense":
            m = np.ones((self.heads, nq, nkv), dtype=np.uint8)
        elif self.mask_kind == "topk":
            m = anchor_uniform_mask(self.heads, nq, nkv, self.keep, self.mask_seed(seed))
        elif self.mask_kind == "count":
            lo, hi = self.count_range
            m = anchor_count_mask(self.heads, nq, nkv, lo, hi, self.mask_seed(seed))
        else:
            raise ValueError(self.mask_kind)
        return np.ascontiguousarray(np.broadcast_to(m[None], (self.batch,) + m.shape))

    def qkv(self, seed: int = DEFAULT_SEED):
        return qkv(self.batch, self.seqlen, self.heads, self.head_dim, seed)


# The workloads of the block-sparse forward (tiny, dense, VSA-256 on its own
# tiles and on finer tiles, native Q64/KV64 with skewed counts), and the
# VSA-256 mask at head_dim 64 with twice the heads (the flops of VSA-256),
# a parity and throughput case for the head_dim-64 kernels.
TINY = Workload("tiny_64x64_b1h2s1024d64", 1, 2, 1024, 64, (64, 64), ((64, 64),),
                "topk", keep=8, keep_fraction=0.5)
DENSE = Workload("dense_b1h8s4096d128", 1, 8, 4096, 128, (256, 256), ((128, 128), (256, 128)),
                 "dense", keep_fraction=1.0)
VSA256 = Workload("vsa256_b1h24s32768d128_keep13", 1, 24, 32768, 128, (256, 256),
                  ((256, 128),), "topk", keep=13, keep_fraction=0.1)
VSA256_FINE = Workload("vsa256_fine_b1h24s32768d128_keep13", 1, 24, 32768, 128, (256, 256),
                       ((128, 64), (64, 64)), "topk", keep=13, keep_fraction=0.1)
NATIVE64 = Workload("native64_b1h24s32768d128_cnt10to92", 1, 24, 32768, 128, (64, 64),
                    ((64, 64),), "count", count_range=(10, 92), keep_fraction=0.1)

VSA256_D64 = Workload("vsa256_b1h48s32768d64_keep13", 1, 48, 32768, 64, (256, 256),
                      ((256, 128), (128, 64), (64, 64)), "topk", keep=13, keep_fraction=0.1)

WORKLOADS = {w.name: w for w in (TINY, DENSE, VSA256, VSA256_FINE, NATIVE64, VSA256_D64)}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """View a contiguous bf16 CPU tensor as a numpy uint16 array of raw bits."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def random_csr(batch, heads, nq, nkv, ld, count_lo, count_hi, seed, shuffle=True):
    """Random block CSR (idx [B,H,NQ,ld] int32, cnt [B,H,NQ] int32) for tests.

    Row counts are U{count_lo..count_hi}; each row holds distinct tile
    indices, in random order when ``shuffle``; unused slots hold -1.
    """
    rng = np.random.default_rng(seed)
    cnt = rng.integers(count_lo, count_hi + 1, size=(batch, heads, nq)).astype(np.int32)
    idx = np.full((batch, heads, nq, ld), -1, dtype=np.int32)
    for b in range(batch):
        for h in range(heads):
            for p in range(nq):
                c = int(cnt[b, h, p])
                sel = rng.choice(nkv, size=c, replace=False)
                if not shuffle:
                    sel = np.sort(sel)
                idx[b, h, p, :c] = sel
    return idx, cnt


def ragged_block_sizes(n_blocks: int, block: int, seed: int, lo: int = 0, p_full: float = 0.3) -> np.ndarray:
    """Valid token counts per KV block for partial-tile inputs: int32 [n_blocks],
    each uniform in [lo, block], a fraction p_full of them exactly full. Video
    latents whose tiles do not divide the frame give such ragged blocks."""
    rng = np.random.default_rng(seed)
    v = rng.integers(lo, block + 1, size=n_blocks).astype(np.int32)
    v[rng.random(n_blocks) < p_full] = block
    return v
