"""The worker pool that runs the oracle over whole workloads for the full-size GPU parity
tests must give exactly the oracle's own results: same sequences, same arrays, bit for bit."""
import numpy as np

import oracle
from workloads import make, variant

from .oracle_pool import Background, oracle_all, stack

FIELDS = ("cand_idx", "cand_val", "gate", "pair", "path", "scores", "slots", "margins")

CFGS = [
    variant("sampled", V=3000, d=64, batch=5, L=4, emb_std=0.3, name="pool_a"),
    variant("tiny", V=2000, d=48, batch=3, emb_std=0.3, name="pool_b"),
]


def _direct(cfg):
    return oracle.select(make(cfg))


def _same(got: dict, want: list):
    assert sorted(got) == list(range(len(want)))
    for f in FIELDS:
        np.testing.assert_array_equal(stack(got, f), np.stack([getattr(r, f) for r in want]), err_msg=f)


def test_oracle_all_equals_oracle():
    cfg = CFGS[0]
    _same(oracle_all(cfg), _direct(cfg))
    sub = oracle_all(cfg, seqs=[4, 1])
    want = _direct(cfg)
    assert sorted(sub) == [1, 4]
    for s in (1, 4):
        for f in FIELDS:
            np.testing.assert_array_equal(getattr(sub[s], f), getattr(want[s], f), err_msg=f)


def test_background_equals_oracle():
    bg = Background(CFGS, workers=2)
    try:
        assert bg.names() == {"pool_a", "pool_b"}
        for cfg in reversed(CFGS):
            _same(bg.get(cfg.name), _direct(cfg))
        assert bg.get("pool_a") is bg.get("pool_a")
    finally:
        bg.close()
