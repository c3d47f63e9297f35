"""Mask front-end oracle (numpy) -- TEST INFRASTRUCTURE.

Two integer steps precede the attention kernel:

``mask_to_csr``: exact expansion of a logical block mask to a finer physical
tile shape, then the per-Q-tile list of selected KV tiles. It follows the
FastVideo page (benchmarks/bench_vsa_blackwell.py): ``expand_exact256_mask``
repeats every mask row 256/q_block times along Q and every column
256/kv_block times along KV, which leaves the selected token pairs unchanged;
``arm_fa4`` then lists, per physical Q tile, the ascending physical KV tile
indices of the expanded mask (``arange(nkv).masked_select(mask)``) together
with their count.

``expand_valid``: per-tile valid key counts (partial tiles) at the physical
KV tile size, from the logical blocks' valid token counts (the variable block
sizes ``vbs`` of the FastVideo page's VSA wrapper): a logical block of LKV
positions holding vbs valid tokens first, then padding, splits into LKV/PKV
physical tiles holding clamp(vbs - r*PKV, 0, PKV) valid tokens each.

``transpose_csr``: the Q-direction lists the backward pass walks (page
"block_sparsity.py" of the FastVideo page's FA4 files: the backward expects
per-KV-tile lists of the Q tiles that select it, "transposed from forward"):
for KV tile n, the ascending Q tile indices m whose forward row lists n.

``pair_q_tiles``: the pairing of adjacent 64-row query tiles onto 128-row
tiles (FastVideo page, README of the fine-grained VSA kernels and the
benchmark notes: at the Q256 API boundary the Q64 children of a logical row
have identical KV lists and are "safely paired" onto the physical Q128/KV64
schedule; arbitrary Q64 lists keep the native Q64 kernel). Query tiles 2p and
2p+1 pair when their counts are equal and their stored lists are equal entry
by entry, in order; the paired row p holds row 2p's list. The pairing is used
only when every pair of the CSR pairs.

``build_worklist``: the order in which Q tiles are processed. Items
(b, h, p) are encoded as their flat index into kv_block_cnt. Within each
segment of ``segment`` consecutive items (one segment per batch and head when
segment = nq) they are sorted by count, largest first, ties kept in
ascending flat order (a stable sort), so that long rows start first (the
work-list idea of the page "BlackwellMultiHeadLatentAttentionForwardFP8": a
grid walking a device list of work tiles instead of a plain grid); segments
keep their order.
"""

from __future__ import annotations

import numpy as np


def mask_to_csr(logical_mask, logical_block, physical_block, ld, fill=-1, kv_valid=None):
    """Expand a logical mask and list its selected KV tiles per Q tile.

    logical_mask: [B, H, NQ_l, NKV_l], nonzero = selected.
    logical_block = (LQ, LKV) tokens per logical cell; physical_block =
    (PQ, PKV) with LQ % PQ == 0 and LKV % PKV == 0.
    Returns (idx [B, H, NQ_p, ld] int32, cnt [B, H, NQ_p] int32, overflow).
    cnt is the true count; a row with cnt > ld keeps only its first ld
    entries and sets ``overflow``. Slots past a row's count hold ``fill``.
    kv_valid [NKV_p] (optional): valid keys per physical KV tile; a tile
    with none holds no selectable key, so it is not listed.
    """
    m = np.asarray(logical_mask) != 0
    lq, lkv = logical_block
    pq, pkv = physical_block
    if lq % pq or lkv % pkv:
        raise ValueError("physical tile sizes must divide the logical block sizes")
    phys = np.repeat(np.repeat(m, lq // pq, axis=2), lkv // pkv, axis=3)
    if kv_valid is not None:
        has_key = np.asarray(kv_valid).reshape(-1) > 0
        if has_key.size != phys.shape[3]:
            raise ValueError("kv_valid must hold one count per physical KV tile")
        phys = phys & has_key[None, None, None, :]
    B, H, NQ, NKV = phys.shape
    idx = np.full((B, H, NQ, ld), fill, dtype=np.int32)
    cnt = np.zeros((B, H, NQ), dtype=np.int32)
    overflow = False
    cols = np.arange(NKV, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for p in range(NQ):
                sel = cols[phys[b, h, p]]
                cnt[b, h, p] = sel.size
                n = min(sel.size, ld)
                idx[b, h, p, :n] = sel[:n]
                overflow |= sel.size > ld
    return idx, cnt, bool(overflow)


def build_worklist(kv_block_cnt, ld, segment=None):
    """Flat (b, h, p) indices; within each segment sorted by clamp(cnt, 0, ld)
    descending, stable. segment defaults to the whole list."""
    c = np.clip(np.asarray(kv_block_cnt, dtype=np.int64).reshape(-1), 0, ld)
    n = c.size
    segment = n if segment is None else segment
    if n and n % segment:
        raise ValueError("segment must divide the number of items")
    out = np.empty(n, dtype=np.int32)
    for s0 in range(0, n, segment):
        out[s0:s0 + segment] = s0 + np.argsort(-c[s0:s0 + segment], kind="stable")
    return out


def expand_valid(vbs, logical_kv, physical_kv):
    """Valid key tokens per physical KV tile [NKV_l * LKV/PKV] from the valid
    tokens per logical KV block vbs [NKV_l] (each in [0, LKV])."""
    v = np.asarray(vbs, dtype=np.int64)
    if logical_kv % physical_kv:
        raise ValueError("physical tile size must divide the logical block size")
    if np.any(v < 0) or np.any(v > logical_kv):
        raise ValueError("valid counts must lie in [0, logical block size]")
    e = logical_kv // physical_kv
    out = np.empty((v.size, e), dtype=np.int32)
    for r in range(e):
        out[:, r] = np.clip(v - r * physical_kv, 0, physical_kv)
    return out.reshape(-1)


def transpose_csr(kv_block_idx, kv_block_cnt, nkv, ld_q, fill=-1):
    """Q-direction block CSR from a KV-direction one.

    kv_block_idx [B, H, NQ, ld], kv_block_cnt [B, H, NQ] (entries [0, cnt) of
    a row are distinct KV tiles in [0, nkv)). Returns (q_block_idx [B, H, nkv,
    ld_q] int32, q_block_cnt [B, H, nkv] int32, overflow): row n lists, in
    ascending order, the Q tiles m whose row holds n; slots past the count
    hold ``fill``; a count above ld_q keeps the first ld_q entries and sets
    overflow.
    """
    idx = np.asarray(kv_block_idx)
    cnt = np.asarray(kv_block_cnt)
    B, H, NQ, _ = idx.shape
    q_idx = np.full((B, H, nkv, ld_q), fill, dtype=np.int32)
    q_cnt = np.zeros((B, H, nkv), dtype=np.int32)
    overflow = False
    for b in range(B):
        for h in range(H):
            sel = np.zeros((nkv, NQ), dtype=bool)
            for m in range(NQ):
                for t in idx[b, h, m, :cnt[b, h, m]]:
                    sel[t, m] = True
            for n in range(nkv):
                ms = np.nonzero(sel[n])[0].astype(np.int32)
                q_cnt[b, h, n] = ms.size
                k = min(ms.size, ld_q)
                q_idx[b, h, n, :k] = ms[:k]
                overflow |= ms.size > ld_q
    return q_idx, q_cnt, bool(overflow)


def pair_q_tiles(kv_block_idx, kv_block_cnt, fill=-1):
    """Pair query tiles (2p, 2p+1) of a block CSR onto tiles twice as tall.

    kv_block_idx [B, H, NQ, ld], kv_block_cnt [B, H, NQ], NQ even. Returns
    (idx [B, H, NQ/2, ld] int32, cnt [B, H, NQ/2] int32, unpaired): row p
    holds the count of row 2p and its first min(count, ld) entries (slots past
    them hold ``fill``); ``unpaired`` counts the pairs whose two rows differ
    in count or in any of those entries.
    """
    idx = np.asarray(kv_block_idx)
    cnt = np.asarray(kv_block_cnt)
    B, H, NQ, ld = idx.shape
    if NQ % 2:
        raise ValueError("the number of query tiles must be even")
    out_idx = np.full((B, H, NQ // 2, ld), fill, dtype=np.int32)
    out_cnt = np.zeros((B, H, NQ // 2), dtype=np.int32)
    unpaired = 0
    for b in range(B):
        for h in range(H):
            for p in range(NQ // 2):
                c0, c1 = int(cnt[b, h, 2 * p]), int(cnt[b, h, 2 * p + 1])
                n = max(0, min(c0, ld))
                top = idx[b, h, 2 * p, :n]
                out_idx[b, h, p, :n] = top
                out_cnt[b, h, p] = c0
                same = c0 == c1 and np.array_equal(top, idx[b, h, 2 * p + 1, :n])
                unpaired += 0 if same else 1
    return out_idx, out_cnt, unpaired
