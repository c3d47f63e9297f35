"""Pins for the mask front-end oracle (exact expansion + CSR, work list)."""

import numpy as np
import pytest

from oracle import frontend
from workloads import anchor_count_mask, anchor_uniform_mask


def _selected_by_logical(mask, lblock, S):
    """Brute force over tokens: pairs (i, j) the logical mask selects."""
    B, H, _, _ = mask.shape
    i = np.arange(S)
    return mask[:, :, i[:, None] // lblock[0], i[None, :] // lblock[1]] != 0  # [B,H,S,S]


def _selected_by_csr(idx, cnt, pblock, S):
    B, H, NQ, _ = idx.shape
    out = np.zeros((B, H, S, S), dtype=bool)
    for b in range(B):
        for h in range(H):
            for p in range(NQ):
                for t in idx[b, h, p, :cnt[b, h, p]]:
                    out[b, h, p * pblock[0]:(p + 1) * pblock[0], t * pblock[1]:(t + 1) * pblock[1]] = True
    return out


@pytest.mark.parametrize("lblock,pblock", [((256, 256), (256, 128)), ((256, 256), (128, 64)),
                                           ((256, 256), (64, 64)), ((256, 256), (256, 256)),
                                           ((64, 64), (64, 64)), ((128, 64), (32, 16))])
def test_csr_selects_exactly_the_logical_token_pairs(lblock, pblock):
    S = 1024
    rng = np.random.default_rng(lblock[0] + pblock[1])
    mask = (rng.random((2, 2, S // lblock[0], S // lblock[1])) < 0.4).astype(np.uint8)
    ld = S // pblock[1]
    idx, cnt, ovf = frontend.mask_to_csr(mask, lblock, pblock, ld)
    assert not ovf
    assert idx.shape == (2, 2, S // pblock[0], ld) and cnt.shape == (2, 2, S // pblock[0])
    assert np.array_equal(_selected_by_csr(idx, cnt, pblock, S), _selected_by_logical(mask, lblock, S))
    # rows list distinct tiles in ascending order; unused slots hold the fill
    for pos in np.ndindex(cnt.shape):
        row = idx[pos][:cnt[pos]]
        assert np.all(np.diff(row) > 0)
        assert np.all(idx[pos][cnt[pos]:] == -1)
    # counts scale by the KV expansion factor
    e = lblock[1] // pblock[1]
    assert np.all(cnt % e == 0)


@pytest.mark.parametrize("lblock,pblock", [((256, 256), (256, 128)), ((256, 256), (128, 64)),
                                           ((256, 256), (64, 64)), ((128, 64), (32, 16))])
def test_csr_with_valid_counts_selects_exactly_the_valid_token_pairs(lblock, pblock):
    """With valid keys per physical tile, the listed tiles' valid keys are
    exactly the logical mask's pairs restricted to valid key tokens, and no
    listed tile is empty (the tiles left out held no valid key)."""
    S = 1024
    rng = np.random.default_rng(lblock[1] + pblock[0])
    mask = (rng.random((2, 2, S // lblock[0], S // lblock[1])) < 0.5).astype(np.uint8)
    vbs = rng.integers(0, lblock[1] + 1, size=S // lblock[1])
    vbs[:2] = [0, lblock[1]]
    val = frontend.expand_valid(vbs, lblock[1], pblock[1])
    ld = S // pblock[1]
    idx, cnt, ovf = frontend.mask_to_csr(mask, lblock, pblock, ld, kv_valid=val)
    assert not ovf
    key_exists = np.concatenate([np.arange(lblock[1]) < n for n in vbs])  # per key token
    want = _selected_by_logical(mask, lblock, S) & key_exists[None, None, None, :]
    got = _selected_by_csr(idx, cnt, pblock, S) & key_exists[None, None, None, :]
    assert np.array_equal(got, want)
    for pos in np.ndindex(cnt.shape):
        row = idx[pos][:cnt[pos]]
        assert np.all(val[row] > 0) and np.all(np.diff(row) > 0)
    # without valid counts the same rows list at least as many tiles
    _, cnt_all, _ = frontend.mask_to_csr(mask, lblock, pblock, ld)
    assert np.all(cnt <= cnt_all) and cnt.sum() < cnt_all.sum()


def test_overflow_truncates_and_flags():
    mask = np.ones((1, 1, 2, 8), dtype=np.uint8)
    idx, cnt, ovf = frontend.mask_to_csr(mask, (64, 64), (64, 32), ld=10)
    assert ovf and np.all(cnt == 16)
    assert np.array_equal(idx[0, 0, 0], np.arange(10))


def test_coarser_physical_tile_rejected():
    with pytest.raises(ValueError):
        frontend.mask_to_csr(np.ones((1, 1, 4, 4), np.uint8), (64, 64), (128, 64), 4)


def test_worklist_is_a_stable_descending_count_order():
    rng = np.random.default_rng(3)
    cnt = rng.integers(0, 20, size=(2, 3, 50)).astype(np.int32)
    cnt[0, 0, 5] = 99  # beyond ld: clamped to ld for ordering
    ld = 25
    w = frontend.build_worklist(cnt, ld)
    flat = np.clip(cnt.reshape(-1), 0, ld)
    assert sorted(w.tolist()) == list(range(flat.size))
    keys = flat[w]
    assert np.all(np.diff(keys) <= 0)
    for a, b in zip(w[:-1], w[1:]):
        if flat[a] == flat[b]:
            assert a < b
    # same order as an explicit comparison sort on (-count, index)
    assert w.tolist() == sorted(range(flat.size), key=lambda i: (-flat[i], i))


def test_segmented_worklist_sorts_within_segments_only():
    rng = np.random.default_rng(4)
    cnt = rng.integers(0, 12, size=(2, 3, 40)).astype(np.int32)
    ld = 10
    seg = 40
    w = frontend.build_worklist(cnt, ld, segment=seg)
    flat = np.clip(cnt.reshape(-1), 0, ld)
    assert sorted(w.tolist()) == list(range(flat.size))
    for s0 in range(0, flat.size, seg):
        part = w[s0:s0 + seg]
        assert np.all((part >= s0) & (part < s0 + seg))  # items stay in their segment
        assert part.tolist() == sorted(range(s0, s0 + seg), key=lambda i: (-flat[i], i))
    # one segment = the global order; segment must divide the item count
    assert np.array_equal(frontend.build_worklist(cnt, ld, segment=flat.size), frontend.build_worklist(cnt, ld))
    with pytest.raises(ValueError):
        frontend.build_worklist(cnt, ld, segment=7)


def test_page_mask_generator_invariants():
    m = anchor_uniform_mask(3, 16, 16, 8, seed=1566)
    assert m.shape == (3, 16, 16)
    assert np.all(m.sum(-1) == 8)
    rows = np.arange(16)
    assert np.all(m[:, rows, rows] == 1)  # anchor floor(q*nkv/nq) = q on a square grid
    m2 = anchor_uniform_mask(3, 16, 16, 8, seed=1566)
    assert np.array_equal(m, m2)
    # rectangular grid anchor
    m3 = anchor_uniform_mask(2, 8, 32, 3, seed=5)
    assert np.all(m3[:, np.arange(8), np.arange(8) * 4] == 1)
    assert np.all(m3.sum(-1) == 3)
    # keep = nkv selects every block; keep = 1 only the anchor
    assert np.all(anchor_uniform_mask(1, 4, 4, 4, seed=0) == 1)
    assert np.array_equal(anchor_uniform_mask(1, 4, 4, 1, seed=0)[0], np.eye(4, dtype=np.uint8))
    with pytest.raises(ValueError):
        anchor_uniform_mask(1, 4, 4, 5, seed=0)


def test_mask_generator_is_uniform_off_the_anchor():
    """Off the anchor every block is kept with probability (keep-1)/(NKV-1),
    and pairs of blocks are kept together with the without-replacement
    probability (keep-1)(keep-2)/((NKV-1)(NKV-2)), not the independent one."""
    H, NQ, NKV, keep = 64, 64, 16, 5
    m = anchor_uniform_mask(H, NQ, NKV, keep, seed=7).astype(np.float64)
    anchor = (np.arange(NQ) * NKV) // NQ
    off = np.ones((NQ, NKV), dtype=bool)
    off[np.arange(NQ), anchor] = False
    n = H * NQ
    p1 = (keep - 1) / (NKV - 1)
    overall = m[:, off].mean()
    assert abs(overall - p1) < 4 * np.sqrt(p1 * (1 - p1) / (n * (NKV - 1)))
    # per-column frequency, pooled over rows: no block favoured
    col = np.array([m[:, off[:, j], j].mean() for j in range(NKV)])
    sd = np.sqrt(p1 * (1 - p1) / (H * off.sum(0)))
    assert np.all(np.abs(col - p1) < 5 * sd)
    # joint frequency of two fixed non-anchor blocks in rows where both are off-anchor
    both = off[:, 1] & off[:, 2]
    joint = (m[:, both, 1] * m[:, both, 2]).mean()
    p2 = (keep - 1) * (keep - 2) / ((NKV - 1) * (NKV - 2))
    assert abs(joint - p2) < 5 * np.sqrt(p2 * (1 - p2) / (H * both.sum()))


def test_count_mask_generator_invariants():
    m = anchor_count_mask(4, 512, 512, 10, 92, seed=9)
    c = m.sum(-1)
    assert c.min() >= 10 and c.max() <= 92
    assert abs(c.mean() - 51) < 1.0
    # every count in 10..92 occurs, none outside
    assert set(np.unique(c).tolist()) == set(range(10, 93))
    rows = np.arange(512)
    assert np.all(m[:, rows, rows] == 1)


def test_expand_valid_matches_token_level_definition():
    """Token r of logical block T exists iff r < vbs[T]; the physical tiles must
    hold exactly those tokens as their valid prefixes."""
    rng = np.random.default_rng(8)
    for lkv, pkv in ((256, 128), (256, 64), (256, 256), (128, 32)):
        vbs = rng.integers(0, lkv + 1, size=9)
        vbs[0], vbs[1] = 0, lkv
        val = frontend.expand_valid(vbs, lkv, pkv)
        assert val.shape == (9 * lkv // pkv,) and val.dtype == np.int32
        exists = np.concatenate([np.arange(lkv) < n for n in vbs])           # logical, per token
        tiles = np.concatenate([np.arange(pkv) < n for n in val])            # physical prefixes
        assert np.array_equal(exists, tiles)
    with pytest.raises(ValueError):
        frontend.expand_valid([257], 256, 64)
    with pytest.raises(ValueError):
        frontend.expand_valid([10], 256, 96)


def test_transpose_csr_lists_exactly_the_selecting_query_tiles():
    from workloads import random_csr

    for B, H, NQ, NKV, seed in ((2, 3, 12, 20, 1), (1, 2, 64, 32, 2)):
        idx, cnt = random_csr(B, H, NQ, NKV, NKV, 0, NKV, seed=seed)
        ld_q = NQ
        q_idx, q_cnt, ovf = frontend.transpose_csr(idx, cnt, NKV, ld_q)
        assert not ovf and q_idx.shape == (B, H, NKV, ld_q) and q_cnt.shape == (B, H, NKV)
        fwd_pairs = {(b, h, m, int(t)) for b in range(B) for h in range(H) for m in range(NQ)
                     for t in idx[b, h, m, :cnt[b, h, m]]}
        bwd_pairs = {(b, h, int(m), n) for b in range(B) for h in range(H) for n in range(NKV)
                     for m in q_idx[b, h, n, :q_cnt[b, h, n]]}
        assert fwd_pairs == bwd_pairs
        for pos in np.ndindex(q_cnt.shape):
            row = q_idx[pos][:q_cnt[pos]]
            assert np.all(np.diff(row) > 0) and np.all(q_idx[pos][q_cnt[pos]:] == -1)
        assert q_cnt.sum() == cnt.sum()
        # compact ld_q: truncation flags overflow
        small = max(1, int(q_cnt.max()) - 1)
        _, c2, ovf2 = frontend.transpose_csr(idx, cnt, NKV, small)
        assert ovf2 and np.array_equal(c2, q_cnt)


@pytest.mark.parametrize("lblock,pkv", [((256, 256), 64), ((128, 64), 64), ((256, 256), 128)])
def test_pairing_of_exact_expanded_q64_rows_gives_the_q128_csr(lblock, pkv):
    """Exact expansion of a logical mask with LQ >= 128 gives Q64 rows whose
    pairs always agree; the paired CSR is then the expansion at Q128 itself,
    and it selects the same token pairs as the Q64 CSR."""
    S = 1024
    nql, nkvl = S // lblock[0], S // lblock[1]
    mask = anchor_uniform_mask(3, nql, nkvl, max(1, nkvl // 3), seed=17)[None]
    ld = nkvl * (lblock[1] // pkv)
    idx64, cnt64, _ = frontend.mask_to_csr(mask, lblock, (64, pkv), ld)
    idx128, cnt128, _ = frontend.mask_to_csr(mask, lblock, (128, pkv), ld)
    pidx, pcnt, unpaired = frontend.pair_q_tiles(idx64, cnt64)
    assert unpaired == 0
    assert np.array_equal(pidx, idx128) and np.array_equal(pcnt, cnt128)
    assert np.array_equal(_selected_by_csr(pidx, pcnt, (128, pkv), S), _selected_by_csr(idx64, cnt64, (64, pkv), S))


def test_pairing_counts_each_kind_of_differing_pair():
    """Starting from a fully paired CSR, each planted difference (one entry
    changed, two entries swapped, a count changed, a difference only past the
    stored prefix) is counted exactly when it changes the stored list."""
    mask = anchor_uniform_mask(2, 4, 16, 5, seed=3)[None]
    idx, cnt, _ = frontend.mask_to_csr(mask, (256, 64), (64, 64), 16)
    assert frontend.pair_q_tiles(idx, cnt)[2] == 0
    idx, cnt = idx.copy(), cnt.copy()
    assert np.all(cnt == 5)
    idx[0, 0, 1, 0] = min(set(range(16)) - set(idx[0, 0, 0, :5].tolist()))  # another tile
    idx[0, 1, 3, [0, 1]] = idx[0, 1, 3, [1, 0]]   # same set, another order: not paired
    cnt[0, 1, 5] -= 1                              # shorter list
    idx[0, 0, 7, 10] = 3                           # past the count: ignored
    _, _, unpaired = frontend.pair_q_tiles(idx, cnt)
    assert unpaired == 3
    pidx, pcnt, _ = frontend.pair_q_tiles(idx, cnt)
    assert pcnt[0, 1, 2] == cnt[0, 1, 4] and np.array_equal(pidx[0, 1, 1, :5], idx[0, 1, 2, :5])


def test_pairing_of_natively_sampled_q64_rows_is_refused():
    mask = anchor_count_mask(2, 32, 32, 3, 12, seed=5)[None]
    idx, cnt, _ = frontend.mask_to_csr(mask, (64, 64), (64, 64), 32)
    assert frontend.pair_q_tiles(idx, cnt)[2] > 0
    with pytest.raises(ValueError):
        frontend.pair_q_tiles(idx[:, :, :3], cnt[:, :, :3])
