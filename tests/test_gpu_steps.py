"""GPU parity of dfs_gate, dfs_pair_scores and dfs_walk against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make, variant

from .oracle_pool import stack
from .parity import assert_scores, check_path, record, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_selection_position_amd as dfs

    dfs.lib()


def dfs_mod():
    import draft_selection_position_amd as dfs

    return dfs


# ---------------------------------------------------------------- gate

GATE_ATOL = 2e-5  # fp32 sums of d bf16 products; sigmoid slope <= 1/4


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_gate_full_size_configs(cfg, full_workload, full_oracle):
    # every row of the full-size gate against the oracle's fp64 gate
    inp, dev = full_workload(cfg.name)
    rows = cfg.batch * cfg.L
    print(f"gate {cfg.name}: rows {rows} d {cfg.d}", flush=True)
    g = dfs_mod().gate(dev["hidden"].view(-1, cfg.d), dev["W_h"])
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    want = stack(full_oracle(cfg.name), "gate").reshape(rows, -1)
    np.testing.assert_allclose(g, want, rtol=0, atol=GATE_ATOL)
    record("gate", cfg.name, rows, "rows", f"max abs error {np.abs(g - want).max():.2g}")
    print(f"gate {cfg.name}: max abs error {np.abs(g - want).max():.3g}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
# up to 512 rows the bf16 gate runs as independent tiles: 16 rows up to 64 rows (1 x 8,
# 37 x 72, 16 x 5120, 16 x 65536 with K split 16 ways), 32 rows beyond (300 x 1000 and
# 113 x 4096: ragged last tiles of 12 and 17 rows, 512 x 96); from 512 rows with d a multiple of 64 on
# 128 x 128 LDS-DMA tiles of 64-k steps: four ring steps unsplit (2049 x 256), one (4100 x 64),
# ragged rows over 8 splits (2100 x 5120, finished by its own kernel), 4 splits (4096 x 2048),
# 20 splits (600 x 16384); otherwise the 64-row tiles (3000 x 1000 and 1024 x 96: d not a
# multiple of 64).  W_h ~ N(0, 0.05^2), scaled down beyond d = 5120 so that h W_h keeps the
# scale it has there.
@pytest.mark.parametrize("rows,d", [(1, 8), (37, 72), (16, 5120), (300, 1000), (113, 4096), (16, 65536), (512, 96),
                                    (2049, 256), (4100, 64), (2100, 5120), (4096, 2048), (600, 16384),
                                    (3000, 1000), (1024, 96)])
def test_gate_shapes(rows, d, dtype):
    rng = np.random.default_rng(rows * 7 + d)
    h = rng.standard_normal((rows, d)).astype(np.float32)
    W = (rng.standard_normal((d, 256)) * 0.05 * np.sqrt(5120 / max(d, 5120))).astype(np.float32)
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits

        h, W = f32_to_bf16_bits(h), f32_to_bf16_bits(W)
    g = dfs_mod().gate(to_dev(h), to_dev(W))
    torch.cuda.synchronize()
    want = oracle.gate(oracle.widen(h, dtype), oracle.widen(W, dtype))
    np.testing.assert_allclose(g.cpu().numpy(), want, rtol=0, atol=GATE_ATOL)


# ---------------------------------------------------------------- pair scores and walk


def _oracle_steps(inp):
    """Oracle candidates, gate, pair tensor and walk for every sequence of inp."""
    return oracle.select(inp)


def _upload_steps(res, inp):
    cidx = torch.from_numpy(np.stack([r.cand_idx for r in res]).astype(np.int32)).cuda()
    cval = torch.from_numpy(np.stack([r.cand_val for r in res]).astype(np.float32)).cuda()
    gate = torch.from_numpy(np.stack([r.gate for r in res]).astype(np.float32)).cuda()
    prev = torch.from_numpy(inp.prev_token.astype(np.int32)).cuda()
    return cidx, cval, gate, prev


PAIR_CASES = [
    variant("tiny", V=3000, d=64, batch=3),
    variant("tiny", V=3000, d=64, batch=2, emb_std=0.3, L=16),
    variant("single_stream", V=5000, d=128, batch=4, emb_std=0.3),
    variant("single_stream", V=5000, d=128, batch=2, L=1, emb_std=0.3),
    variant("sampled", V=6000, d=64, batch=5, emb_std=0.3, L=7),
]


@pytest.mark.parametrize("cfg", PAIR_CASES, ids=lambda c: c.name)
def test_pair_scores_match_oracle(cfg):
    inp = make(cfg)
    res = _oracle_steps(inp)
    cidx, cval, gate, prev = _upload_steps(res, inp)
    A, B = to_dev(inp.A), to_dev(inp.B)
    pair = dfs_mod().pair_scores(cidx, cval, prev, gate, A, B)
    torch.cuda.synchronize()
    got = pair.cpu().numpy()
    # the oracle's pair tensor used the fp64 gate; the GPU got it rounded to fp32
    want = np.stack([r.pair for r in res])
    assert_scores(got, want, "pair")
    err = np.abs(got - want).max()
    print(f"pair {cfg.name}: max abs error {err:.3g}", flush=True)
    assert err < 5e-5  # much tighter than the tolerance: hi/lo bf16 split + fp32 sums


@pytest.mark.parametrize("name", ["small_batch", "throughput", "sampled"])
def test_pair_scores_full_size(name, full_workload, full_oracle):
    # the step chain on a full-size workload: every sequence's 16 x 16 score tiles against the
    # oracle's, element by element (the GPU's own top-16 and gate feed the pair step; both
    # were checked bit for bit / to the gate's bar against the same oracle results)
    dfs = dfs_mod()
    inp, dev = full_workload(name)
    cfg = inp.config
    idx, val = dfs.topk(dev["logits"])
    g = dfs.gate(dev["hidden"], dev["W_h"])
    pair = dfs.pair_scores(idx, val, dev["prev_token"], g, dev["A"], dev["B"])
    torch.cuda.synchronize()
    want = full_oracle(name)
    np.testing.assert_array_equal(idx.cpu().numpy().reshape(cfg.batch, cfg.L, 16), stack(want, "cand_idx"))
    got = pair.cpu().numpy()
    ref = stack(want, "pair")
    assert got.shape == ref.shape == (cfg.batch, cfg.L, 16, 16)
    assert_scores(got, ref, f"pair {name}")
    err = np.abs(got - ref)
    print(f"pair {name}: {cfg.batch} sequences, max abs error {err.max():.3g}, "
          f"max rel error {(err / np.maximum(np.abs(ref), 1e-30)).max():.3g}", flush=True)
    record("pair", name, cfg.batch * cfg.L * 256, "scores", f"max abs error {err.max():.2g}")


@pytest.mark.parametrize("cfg", PAIR_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("gumbel", 1.0), ("gumbel", 0.7), ("viterbi", 1.0)])
def test_walk_matches_oracle(cfg, mode, T):
    inp = make(variant(cfg, walk=mode, temperature=T, walk_seed=0xABCDEF123))
    res = _oracle_steps(inp)
    cidx = torch.from_numpy(np.stack([r.cand_idx for r in res]).astype(np.int32)).cuda()
    pair = torch.from_numpy(np.stack([r.pair for r in res]).astype(np.float32)).cuda()
    path, scores = dfs_mod().walk(pair, cidx, mode, T, inp.walk_seed)
    torch.cuda.synchronize()
    path, scores = path.cpu().numpy(), scores.cpu().numpy()
    for i, r in enumerate(res):
        check_path(path[i], scores[i], r, mode, T, inp.walk_seed, int(inp.seq_ids[i]))


def test_best_path_walk_on_planted_scores():
    # a score tensor where the greedy walk and the best path part ways, and one
    # where every score is equal (the read-back then takes slot 0 everywhere)
    L, B = 5, 3
    rng = np.random.default_rng(11)
    S = rng.standard_normal((B, L, 16, 16)).astype(np.float32)
    S[:, 0] = S[:, 0, :1]
    S[0] = 0.0
    S[1, 0, :, 0], S[1, 0, :, 1] = 3.0, 2.9
    S[1, 1, 1, 7] = 40.0
    cidx = np.stack([[rng.choice(5000, 16, replace=False) for _ in range(L)] for _ in range(B)])
    pair = torch.from_numpy(S).cuda()
    ci = torch.from_numpy(cidx.astype(np.int32)).cuda()
    vp, vs = dfs_mod().walk(pair, ci, "viterbi")
    gp, gs = dfs_mod().walk(pair, ci, "greedy")
    torch.cuda.synchronize()
    vp, vs, gp, gs = vp.cpu().numpy(), vs.cpu().numpy(), gp.cpu().numpy(), gs.cpu().numpy()
    for b in range(B):
        path, scores, slots, margins = oracle.viterbi(S[b].astype(np.float64), cidx[b])
        np.testing.assert_array_equal(vp[b], path)
        np.testing.assert_allclose(vs[b], scores, rtol=0, atol=1e-5)
        assert vs[b].astype(np.float64).sum() >= gs[b].astype(np.float64).sum() - 1e-4
    np.testing.assert_array_equal(vp[0], cidx[0, :, 0])
    assert vp[1, 0] == cidx[1, 0, 1] and vp[1, 1] == cidx[1, 1, 7]
    assert gp[1, 0] == cidx[1, 0, 0]
