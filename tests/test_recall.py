"""Recall / acceptance harness: the oracle's counting pinned by hand-counted blocks,
and the library's host reductions against the oracle's loops (CPU)."""
import math

import numpy as np

import oracle
from draft_selection_position_amd import recall as R


def _blocks():
    # 4 blocks, L = 3, 4 candidates listed (rank order); ids < 100
    cands = [
        [[5, 1, 2, 3], [7, 8, 9, 10], [11, 12, 13, 14]],  # true = top-1 everywhere
        [[6, 5, 1, 2], [7, 1, 2, 3], [20, 21, 22, 23]],   # true at rank 1, rank 0, absent
        [[9, 8, 7, 6], [1, 2, 3, 4], [11, 2, 3, 4]],      # absent at position 0
        [[5, 4, 3, 2], [1, 2, 3, 7], [11, 3, 4, 5]],      # top-1, rank 3, top-1
    ]
    trues = [[5, 7, 11], [5, 7, 11], [5, 7, 11], [5, 7, 11]]
    return cands, trues


def test_oracle_recall_hand_counted():
    cands, trues = _blocks()
    r1, e1 = oracle.recall.recall_at(cands, trues, 1)
    # position 0: blocks 0 and 3 of 4; position 1: of those two, block 0; position 2: block 0
    assert e1 == [4, 2, 1] and r1 == [0.5, 0.5, 1.0]
    r4, e4 = oracle.recall.recall_at(cands, trues, 4)
    # position 0: blocks 0, 1, 3; position 1: all three; position 2: blocks 0 and 3 of 3
    assert e4 == [4, 3, 3] and r4 == [0.75, 1.0, 2 / 3]
    paths = [[c[0] for c in cand] for cand in cands]  # top-1 drafts
    # accepted lengths 4, 1, 1, 2
    assert oracle.recall.mean_acceptance(paths, trues) == 2.0
    op = oracle.recall.oracle_selector_paths(cands, trues)
    # 4, 3, 1, 4
    assert oracle.recall.mean_acceptance(op, trues) == 3.0


def test_oracle_recall_no_eligible_block_is_nan():
    r, e = oracle.recall.recall_at([[[1, 2], [3, 4]]], [[9, 3]], 2)
    assert e == [1, 0] and r[0] == 0.0 and math.isnan(r[1])


def test_library_reductions_match_oracle_loops():
    rng = np.random.default_rng(3)
    B, L = 300, 6
    cand = np.stack([[rng.choice(40, 16, replace=False) for _ in range(L)] for _ in range(B)])
    true = rng.integers(0, 40, (B, L))
    true[:50] = cand[:50, :, 0]  # some blocks fully right
    for k in (1, 4, 16):
        r, e = R.recall_at(cand, true, k)
        ro, eo = oracle.recall.recall_at(cand.tolist(), true.tolist(), k)
        assert e.tolist() == eo
        np.testing.assert_array_equal(np.isnan(r), np.isnan(ro))
        np.testing.assert_allclose(r[~np.isnan(r)], np.array(ro)[~np.isnan(r)], rtol=0, atol=1e-15)
    paths = cand[:, :, 0]
    assert R.acceptance(paths, true) == oracle.recall.mean_acceptance(paths.tolist(), true.tolist())
    assert R.oracle_acceptance(cand, true) == oracle.recall.mean_acceptance(
        oracle.recall.oracle_selector_paths(cand.tolist(), true.tolist()), true.tolist())
