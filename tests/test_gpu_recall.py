"""The recall / acceptance harness on GPU outputs against the oracle's own selection."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make, variant

from .parity import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_recall_and_acceptance_match_oracle():
    import draft_selection_position_amd as dfs
    from draft_selection_position_amd import recall as R

    cfg = variant("tiny", batch=48, L=8)
    inp = make(cfg)
    dev = upload(inp)
    idx, _ = dfs.topk(dev["logits"])
    path, _ = dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], dev["W_h"])
    torch.cuda.synchronize()
    res = oracle.select(inp)
    cands = [r.cand_idx.tolist() for r in res]
    trues = inp.true_tokens.tolist()
    for k in (1, 16):
        r, e = R.recall_at(idx, inp.true_tokens, k)
        ro, eo = oracle.recall.recall_at(cands, trues, k)
        assert e.tolist() == eo
        np.testing.assert_allclose(r, ro, rtol=0, atol=1e-15)
    print("recall@1", np.round(r, 3), flush=True)
    assert R.oracle_acceptance(idx, inp.true_tokens) == oracle.recall.mean_acceptance(
        oracle.recall.oracle_selector_paths(cands, trues), trues)
    margins = np.stack([r_.margins for r_ in res])
    if (margins >= 1e-4).all():  # no near tie: the greedy paths are the oracle's
        assert R.acceptance(path, inp.true_tokens) == oracle.recall.mean_acceptance(
            [r_.path.tolist() for r_ in res], trues)
