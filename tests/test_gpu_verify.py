"""Draft distributions (dfs_select_draft) and speculative-sampling verification
(dfs_verify) on the GPU, against the oracle."""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle
from workloads import make, variant
from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits

from .parity import to_dev, upload

pytestmark = pytest.mark.gpu

NEAR_ACCEPT = 1e-4  # |u - p/q| below this: the fp32 and fp64 ratios may disagree
NEAR_DRAW = 1e-6    # the draw's target this close to an interval edge (fraction of the mass)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dfs_mod():
    import draft_selection_position_amd as dfs

    return dfs


@pytest.mark.parametrize("mode,T", [("gumbel", 1.0), ("gumbel", 0.6), ("greedy", 1.0), ("viterbi", 2.0)])
def test_draft_distributions_match_oracle(mode, T):
    cfg = variant("single_stream", emb_std=0.3, batch=5, V=20000, d=256, walk=mode, temperature=T,
                  walk_seed=4242)
    inp = make(cfg)
    dev = upload(inp)
    args = (dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], dev["W_h"])
    path, scores, q, cand = dfs_mod().select(*args, mode=mode, temperature=T, seed=cfg.walk_seed, draft=True)
    p2, s2 = dfs_mod().select(*args, mode=mode, temperature=T, seed=cfg.walk_seed)
    torch.cuda.synchronize()
    assert torch.equal(path, p2) and torch.equal(scores, s2)  # the export changes nothing
    path, q, cand = path.cpu().numpy(), q.cpu().numpy(), cand.cpu().numpy()
    for i in range(cfg.batch):
        res = oracle.select_sequence(inp, i)
        np.testing.assert_array_equal(cand[i], res.cand_idx)
        slots = np.array([int(np.nonzero(res.cand_idx[t] == path[i, t])[0][0]) for t in range(cfg.L)])
        want = oracle.verify.draft_probs(res.pair, slots, T)
        np.testing.assert_allclose(q[i], want, rtol=1e-4, atol=1e-6)
        np.testing.assert_allclose(q[i].sum(1), 1.0, atol=1e-5)


def _draw_within(tgt, cand, q, k, tok, T, seed, b, eps):
    """Is token `tok`'s interval of the inverse-CDF draw at row k within eps (fraction of
    the total) of the oracle's draw target?"""
    p = oracle.verify.softmax(tgt[k] / T)
    w = p.copy()
    if k < cand.shape[0]:
        w[cand[k]] = np.maximum(0.0, p[cand[k]] - q[k].astype(np.float64))
    c = np.cumsum(w)
    target = oracle.verify.draw_uniform(seed, b, k) * c[-1]
    lo = c[tok - 1] if tok > 0 else 0.0
    return w[tok] > 0 and lo - eps * c[-1] <= target <= c[tok] + eps * c[-1]


def _verify_case(cfg, noise, T_target, seed):
    """Draft with the sampled walk, then verify against target logits = the drafter's
    logits plus Gaussian noise (bf16), with one more target row after the block."""
    inp = make(cfg)
    dev = upload(inp)
    path, scores, q, cand = dfs_mod().select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"],
                                             dev["B"], dev["W_h"], mode="gumbel", temperature=cfg.temperature,
                                             seed=cfg.walk_seed, draft=True)
    rng = np.random.default_rng(seed)
    base = oracle.widen(inp.logits, cfg.dtype)
    nxt = rng.standard_normal((cfg.batch, 1, cfg.V)) * 1.5
    tgt = np.concatenate([base + rng.standard_normal(base.shape) * noise, nxt], axis=1).astype(np.float32)
    tgt_store = f32_to_bf16_bits(tgt) if cfg.dtype == "bf16" else tgt
    tgt_dev = to_dev(tgt_store)
    acc, tok = dfs_mod().verify(tgt_dev, path, cand, q, T_target, seed)
    torch.cuda.synchronize()
    tgt64 = bf16_bits_to_f32(tgt_store).astype(np.float64) if cfg.dtype == "bf16" else tgt.astype(np.float64)
    return (acc.cpu().numpy(), tok.cpu().numpy(), path.cpu().numpy(), cand.cpu().numpy(), q.cpu().numpy(),
            tgt64)


@pytest.mark.parametrize("cfg,noise,T", [
    (variant("single_stream", emb_std=0.3, batch=24, V=20000, d=256, walk="gumbel", walk_seed=7), 0.3, 1.0),
    (variant("single_stream", emb_std=0.3, batch=24, V=20001, d=256, walk="gumbel", walk_seed=8,
             temperature=0.7), 1.0, 0.8),
    (variant("tiny", emb_std=0.3, batch=16, walk="gumbel", walk_seed=9), 0.5, 1.0),
    (variant("sampled", emb_std=0.3, batch=8, V=50000, d=256, L=5, walk_seed=10), 0.2, 1.3),
    # the largest vocabulary the draw handles: 1023 segments of 4096 tokens per row
    (variant("single_stream", emb_std=0.3, batch=3, V=4190208, d=64, L=4, walk="gumbel", walk_seed=11), 0.3, 1.0),
], ids=lambda x: getattr(x, "name", str(x)))
def test_verify_matches_oracle(cfg, noise, T):
    acc, tok, path, cand, q, tgt = _verify_case(cfg, noise, T, seed=12345)
    near_acc = near_draw = 0
    for b in range(cfg.batch):
        v = oracle.verify.verify_block(tgt[b], path[b], cand[b], q[b].astype(np.float64), T, 12345, b)
        if v.accept_margin < NEAR_ACCEPT:
            near_acc += 1
            assert 0 <= acc[b] <= cfg.L and 0 <= tok[b] < cfg.V
            continue
        assert int(acc[b]) == v.accepted, (b, acc[b], v)
        if v.draw_margin < NEAR_DRAW:
            # near an interval edge: the GPU's token must still be one whose interval
            # lies within NEAR_DRAW of the draw (on the oracle's own sums)
            near_draw += 1
            assert _draw_within(tgt[b], cand[b], q[b], v.accepted, int(tok[b]), T, 12345, b, NEAR_DRAW)
            continue
        assert (int(acc[b]), int(tok[b])) == (v.accepted, v.token), (b, acc[b], tok[b], v)
    print(f"verify {cfg.name}: accepted mean {acc.mean():.2f}, {near_acc} accept and {near_draw} draw near ties",
          flush=True)
    if cfg.V < 1_000_000:
        assert near_acc + near_draw <= cfg.batch // 4
    else:
        # with millions of tokens a token's interval is narrower than NEAR_DRAW of the mass,
        # so nearly every draw is near an edge; each was checked to land within it above
        assert near_acc <= cfg.batch // 4


def test_verify_emitted_tokens_follow_the_target():
    # The theorem on the GPU: many blocks, one target row and one draft distribution,
    # drafts drawn from q on the host; the first emitted token must follow p.
    B, L, V = 40000, 1, 48
    rng = np.random.default_rng(77)
    cand1 = rng.choice(V, 16, replace=False).astype(np.int32)
    q1 = rng.dirichlet(np.ones(16)).astype(np.float32)
    z = (rng.standard_normal(V) * 1.2).astype(np.float32)
    tgt = np.broadcast_to(np.stack([z, z])[None], (B, 2, V)).copy()
    path = cand1[rng.choice(16, size=B, p=q1.astype(np.float64) / q1.sum())][:, None].astype(np.int32)
    cand = np.broadcast_to(cand1, (B, L, 16)).copy()
    q = np.broadcast_to(q1, (B, L, 16)).copy()
    acc, tok = dfs_mod().verify(torch.from_numpy(tgt).cuda(), torch.from_numpy(path).cuda(),
                                torch.from_numpy(cand).cuda(), torch.from_numpy(q).cuda(), 1.0, 2026)
    torch.cuda.synchronize()
    acc, tok = acc.cpu().numpy(), tok.cpu().numpy()
    first = np.where(acc >= 1, path[:, 0], tok)
    p = np.exp(z.astype(np.float64) - z.max())
    p /= p.sum()
    counts = np.bincount(first, minlength=V)
    stat = ((counts - B * p) ** 2 / (B * p)).sum()
    assert scipy.stats.chi2.sf(stat, V - 1) > 1e-3
    qfull = np.zeros(V)
    qfull[cand1] = q1 / q1.sum()
    rate = np.minimum(p, qfull).sum()
    assert abs((acc >= 1).mean() - rate) < 4 * np.sqrt(rate * (1 - rate) / B)


def test_verify_special_cases():
    B, L, V = 64, 3, 300
    rng = np.random.default_rng(5)
    cand = np.stack([[rng.choice(V, 16, replace=False) for _ in range(L)] for _ in range(B)]).astype(np.int32)
    q = rng.dirichlet(np.ones(16), size=(B, L)).astype(np.float32)
    path = np.take_along_axis(cand, rng.integers(0, 16, (B, L, 1)), axis=2)[:, :, 0].astype(np.int32)
    # target equal to the draft on the candidates, nothing elsewhere: all accepted
    tgt = np.full((B, L + 1, V), -np.inf, np.float32)
    for b in range(B):
        for t in range(L):
            tgt[b, t, cand[b, t]] = np.log(q[b, t])
    tgt[:, L] = rng.standard_normal((B, V))
    # (the draft's q is scaled down a little so that p / q >= 1 despite rounding)
    acc, tok = dfs_mod().verify(torch.from_numpy(tgt).cuda(), torch.from_numpy(path).cuda(),
                                torch.from_numpy(cand).cuda(), torch.from_numpy(q * np.float32(0.999)).cuda(),
                                1.0, 3)
    torch.cuda.synchronize()
    assert (acc.cpu().numpy() == L).all()
    # no target mass on any candidate: rejected at position 0, the draw is never a candidate
    tgt2 = rng.standard_normal((B, L + 1, V)).astype(np.float32)
    for b in range(B):
        tgt2[b, 0, cand[b, 0]] = -np.inf
    acc, tok = dfs_mod().verify(torch.from_numpy(tgt2).cuda(), torch.from_numpy(path).cuda(),
                                torch.from_numpy(cand).cuda(), torch.from_numpy(q).cuda(), 1.0, 3)
    torch.cuda.synchronize()
    acc, tok = acc.cpu().numpy(), tok.cpu().numpy()
    assert (acc == 0).all()
    assert not any(tok[b] in cand[b, 0] for b in range(B))
    for b in range(0, B, 8):
        v = oracle.verify.verify_block(tgt2[b].astype(np.float64), path[b], cand[b], q[b].astype(np.float64),
                                       1.0, 3, b)
        if v.draw_margin >= NEAR_DRAW:
            assert tok[b] == v.token
