"""Pins for the oracle's candidate-block selection (level one of the two-level top-k) and
level two's mask.

Definition (DeepSeek-V4.1-Flash-NVFP4 model.py, select_candidate_blocks and
Indexer.forward): block score = max over the block's positions (-inf padding), the block
with the query's newest visible row pinned to +inf, the min(topk_blocks, n_blocks) best
blocks kept unless their score is -inf; level two masks every other position to -inf
before its own top-k.

Pins (hand-derived sets, invariants and identities; none re-runs the oracle's steps):
* a hand-ranked case: known block maxima, the newest block pinned although it is not
  among the best;
* every visible block is kept when there are at most topk_blocks of them;
* blocks a query cannot see are never kept; a query that sees nothing keeps nothing;
* equal block scores keep the lower blocks (the tie reading), the pinned block always;
* a strictly increasing map of the scores, and a permutation of whole older blocks, map
  the kept set as they should;
* level two with every visible row kept is the ordinary top-k.
"""
import numpy as np
import pytest


def _row(T, fill=-5.0):
    return np.full((1, 1, T), fill, dtype=np.float64)


def test_hand_ranked_blocks(orc):
    # 8 blocks of 8; block maxima chosen by hand, every other entry lower
    maxima = [5.0, 1.0, 7.0, 3.0, 8.0, 2.0, 6.0, 4.0]
    s = _row(64)
    for j, m in enumerate(maxima):
        s[0, 0, 8 * j + (j * 3) % 8] = m
    # decode at end_pos = 128, ratio 2: 64 visible rows, newest block 7 (max 4) pinned
    got = orc.candidate_blocks(s, start_pos=127, ratio=2, topk_blocks=4, block_size=8)
    # pinned 7, then the three best others: blocks 4 (8), 2 (7), 6 (6)
    assert got.tolist() == [[[2, 4, 6, 7]]]
    got = orc.candidate_blocks(s, start_pos=127, ratio=2, topk_blocks=1, block_size=8)
    assert got.tolist() == [[[7]]]


def test_all_visible_blocks_kept_when_few(orc):
    rng = np.random.default_rng(0)
    s = rng.standard_normal((2, 1, 61))          # 61 rows: the last block holds 5
    got = orc.candidate_blocks(s, start_pos=60, ratio=1, topk_blocks=8, block_size=8)
    assert got.shape == (2, 1, 8)
    assert (got == np.arange(8)).all()
    got = orc.candidate_blocks(s, start_pos=60, ratio=1, topk_blocks=20, block_size=8)
    assert got.shape == (2, 1, 8) and (got == np.arange(8)).all()


def test_prefill_visibility_and_empty_query(orc):
    # prefill from 0, ratio 2, 16 queries: query i sees (i+1)//2 rows, the rest are -inf
    S, r, bs = 16, 2, 2
    T = S // r
    rng = np.random.default_rng(1)
    s = rng.standard_normal((1, S, T))
    for i in range(S):
        s[0, i, (i + 1) // r:] = -np.inf
    got = orc.candidate_blocks(s, start_pos=0, ratio=r, topk_blocks=2, block_size=bs)
    assert got.shape == (1, S, 2)
    for i in range(S):
        nvis = (i + 1) // r
        kept = [j for j in got[0, i] if j >= 0]
        nb_vis = (nvis + bs - 1) // bs
        assert len(kept) == min(2, nb_vis), (i, kept)
        assert all(j < nb_vis for j in kept)
        if nvis:
            assert (nvis - 1) // bs in kept        # the newest block is pinned
    assert got[0, 0].tolist() == [-1, -1]          # query 0 sees nothing


def test_ties_keep_lower_blocks_and_the_pinned_one(orc):
    s = np.zeros((1, 1, 80))                       # 10 blocks, all equal
    got = orc.candidate_blocks(s, start_pos=79, ratio=1, topk_blocks=4, block_size=8)
    assert got.tolist() == [[[0, 1, 2, 9]]]


def test_monotone_map_and_block_permutation(orc):
    rng = np.random.default_rng(2)
    T, bs, kb = 96, 8, 5
    s = rng.standard_normal((1, 1, T))
    base = orc.candidate_blocks(s, start_pos=T - 1, ratio=1, topk_blocks=kb, block_size=bs)
    mapped = orc.candidate_blocks(np.exp(3 * s) + 7, start_pos=T - 1, ratio=1, topk_blocks=kb,
                                  block_size=bs)
    assert np.array_equal(base, mapped)
    # permute the older blocks (the newest, block 11, stays last)
    perm = rng.permutation(11)
    sp = s.reshape(1, 1, 12, bs).copy()
    sp[0, 0, :11] = sp[0, 0, perm]
    got = orc.candidate_blocks(sp.reshape(1, 1, T), start_pos=T - 1, ratio=1, topk_blocks=kb,
                               block_size=bs)
    inv = np.argsort(perm)                        # old block j now sits at inv[j]
    want = sorted(int(inv[j]) if j < 11 else 11 for j in base[0, 0])
    assert got[0, 0].tolist() == want


def test_level_two_with_everything_kept_is_plain_topk(orc):
    rng = np.random.default_rng(3)
    s = rng.standard_normal((2, 3, 40))
    for i in range(3):
        s[:, i, (37 + i + 1):] = -np.inf
    blocks = orc.candidate_blocks(s, start_pos=37, ratio=1, topk_blocks=10, block_size=4)
    masked = orc.apply_candidates(s, blocks, 4)
    assert np.array_equal(orc.topk(masked, 37, 1, 12), orc.topk(s, 37, 1, 12))
    # with fewer blocks, every pick lies in a kept block
    blocks = orc.candidate_blocks(s, start_pos=37, ratio=1, topk_blocks=4, block_size=4)
    idx = orc.topk(orc.apply_candidates(s, blocks, 4), 37, 1, 12)
    for b in range(2):
        for i in range(3):
            assert set(idx[b, i] // 4) <= set(blocks[b, i])


def test_refuses_bad_arguments(orc):
    with pytest.raises(orc.OracleError):
        orc.candidate_blocks(np.zeros((1, 1, 8)), start_pos=15, ratio=1, topk_blocks=2,
                             block_size=4)          # 16 rows but ld 8
    with pytest.raises(orc.OracleError):
        orc.candidate_blocks(np.zeros((1, 1, 8)), start_pos=7, ratio=1, topk_blocks=2,
                             block_size=0)
