"""dfs_lmhead_topk (top-16 straight from hidden states through the LM head) on the GPU:
bit-exact against the unfused chain dfs_lmhead_logits -> dfs_topk, and against the
fp64 oracle within the fp32 summation bound."""
import numpy as np
import pytest
import torch

import oracle
from workloads.configs import variant
from workloads.gen import bf16_bits_to_f32
from workloads.lmhead import make_hidden, make_lm_head

from .parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dfs_mod():
    import draft_selection_position_amd as dfs

    return dfs


def _inputs(rows, V, d, seed=0, std=0.05):
    rng = np.random.default_rng(seed)
    from workloads.gen import f32_to_bf16_bits

    h = f32_to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    W = f32_to_bf16_bits((rng.standard_normal((V, d)) * std).astype(np.float32))
    return h, W


def _chain_equal(h_dev, W_dev):
    dfs = dfs_mod()
    idx, val = dfs.lmhead_topk(h_dev, W_dev)
    U = dfs.lmhead_logits(h_dev, W_dev)
    idx2, val2 = dfs.topk(U)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), (idx[:2], idx2[:2])
    assert torch.equal(val.view(torch.int32), val2.view(torch.int32))
    return idx.cpu().numpy(), val.cpu().numpy(), U


def _oracle_check(h, W, idx, val, U_gpu, rows):
    """Logits within d 2^-24 sum|h w| of fp64; the top-16 is a valid top-16 of the exact
    logits up to twice that bound (near ties), with the GPU's own values."""
    hf = bf16_bits_to_f32(h[rows]).astype(np.float64)
    Wf = bf16_bits_to_f32(W).astype(np.float64)
    U = hf @ Wf.T
    eps = h.shape[-1] * 2.0 ** -24 * (np.abs(hf) @ np.abs(Wf).T) + 1e-30
    Ug = U_gpu[rows].astype(np.float64)
    assert (np.abs(Ug - U) <= eps).all()
    for j, rr in enumerate(rows):
        ids_o, _ = oracle.top16(U[j])
        gi = idx[rr].astype(np.int64)
        np.testing.assert_array_equal(val[rr], Ug[j][gi].astype(np.float32))
        e = 2 * eps[j].max()
        kth = val[rr][-1]
        must = np.nonzero(U[j] > kth + e)[0]  # clearly above the GPU's 16th: must be chosen
        assert set(must.tolist()) <= set(gi.tolist())
        assert (U[j][gi] >= np.sort(U[j])[-16] - e).all()  # nothing chosen clearly below the 16th
        assert len(set(gi.tolist())) == 16
        exact = set(ids_o.tolist()) == set(gi.tolist())
        if not exact:
            print(f"row {rr}: near-tie set difference", flush=True)


SHAPES = [
    # (rows, V, d): small tiles (16 x 256) with one/two row tiles; big tiles, ragged rows;
    # ragged column tiles; a single stripe; many stripes
    (1, 1000, 64), (16, 20001, 256), (29, 4099, 512), (33, 20000, 256), (200, 50000, 128),
    (130, 777, 1024), (1, 16, 64),
    # 256 x 256 tiles: exact tiles; ragged rows and columns; one column tile; deep K
    (256, 4096, 256), (300, 20001, 512), (513, 777, 128), (257, 70000, 64), (1024, 5000, 2048),
    # 256 x 256 tiles (from 2048 rows): ragged rows and columns
    (2100, 3000, 256),
]


@pytest.mark.parametrize("rows,V,d", SHAPES, ids=lambda v: str(v))
def test_lmhead_topk_equals_chain_and_oracle(rows, V, d):
    h, W = _inputs(rows, V, d, seed=rows + V)
    idx, val, U = _chain_equal(to_dev(h), to_dev(W))
    sample = sorted(set([0, rows - 1] + list(range(0, rows, max(1, rows // 6)))))
    _oracle_check(h, W, idx, val, U.cpu().numpy(), sample)


def test_lmhead_ties_and_duplicates():
    # Duplicate weight rows give exactly equal logits: every value comes as a pair of
    # ids (i, i + 1500), and the lower id must come first in each pair.
    rows, V, d = 40, 3000, 128
    h, W = _inputs(rows, V, d, seed=9)
    W[1500:3000] = W[0:1500]
    idx, val, _ = _chain_equal(to_dev(h), to_dev(W))
    assert (idx[:, 0::2] < 1500).all()
    np.testing.assert_array_equal(idx[:, 1::2], idx[:, 0::2] + 1500)
    np.testing.assert_array_equal(val[:, 1::2], val[:, 0::2])


def test_lmhead_single_stream_full_size():
    cfg = variant("single_stream")
    h = make_hidden(cfg).reshape(-1, cfg.d)
    W = make_lm_head(cfg)
    idx, val, U = _chain_equal(to_dev(h), to_dev(W))
    _oracle_check(h, W, idx, val, U.cpu().numpy(), list(range(0, 16, 3)))


def test_lmhead_throughput_full_size_chain():
    # 4096 x 151936 x 5120 in the launch configuration the bench times; chain exact on
    # every row, the oracle on a few.
    cfg = variant("throughput")
    h = make_hidden(cfg).reshape(-1, cfg.d)
    W = make_lm_head(cfg)
    hd, Wd = to_dev(h), to_dev(W)
    del W
    idx, val, U = _chain_equal(hd, Wd)
    Wn = make_lm_head(cfg)
    rows = [0, 1000, 4095]
    _oracle_check(h, Wn, idx, val, _rows_of(U, rows), rows)


def _rows_of(U, rows):
    out = np.zeros((max(rows) + 1, U.shape[1]), np.float32)
    out[rows] = U[rows].cpu().numpy()
    return out
