"""GPU parity of the fused dfs_select against the oracle, on the five workloads and variants."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make, variant

from .parity import NEAR_TIE, check_path, record, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_selection_position_amd as dfs

    dfs.lib()


def _select(dev, cfg):
    import draft_selection_position_amd as dfs

    path, scores = dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], dev["W_h"],
                              mode=cfg.walk, temperature=cfg.temperature, seed=cfg.walk_seed)
    torch.cuda.synchronize()
    return path.cpu().numpy(), scores.cpu().numpy()


def _check(inp, path, scores, seqs):
    cfg = inp.config
    near = 0
    for i in seqs:
        res = oracle.select_sequence(inp, int(i))
        rep = check_path(path[i], scores[i], res, cfg.walk, cfg.temperature, cfg.walk_seed, int(inp.seq_ids[i]))
        near += len(rep["near_ties"])
    return near


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_select_full_size_configs(cfg, full_workload, full_oracle):
    # every sequence of the full-size workload against the oracle's whole-batch results
    inp, dev = full_workload(cfg.name)
    print(f"select {cfg.name}: batch {cfg.batch} L {cfg.L} V {cfg.V} d {cfg.d} walk {cfg.walk}", flush=True)
    path, scores = _select(dev, cfg)
    want = full_oracle(cfg.name)
    assert sorted(want) == list(range(cfg.batch))
    near = positions = 0
    for i in range(cfg.batch):
        res = want[i]
        rep = check_path(path[i], scores[i], res, cfg.walk, cfg.temperature, cfg.walk_seed, i)
        near += len(rep["near_ties"])
        positions += int((res.margins < NEAR_TIE).sum())
    record("select", cfg.name, cfg.batch, "sequences",
           f"{near} paths part at a near tie (oracle margin < {NEAR_TIE}; {positions} such steps)")
    print(f"select {cfg.name}: all {cfg.batch} sequences checked, {near} near-tie divergences, "
          f"{positions} oracle steps with margin < {NEAR_TIE}", flush=True)


VARIANTS = [
    variant("tiny", emb_std=0.3),  # the bilinear term moves the walk off the top-1
    variant("tiny", emb_std=0.3, L=1),
    variant("tiny", emb_std=0.3, L=3, V=32001, batch=5),
    variant("single_stream", emb_std=0.3, batch=6, V=32001, d=512),
    variant("single_stream", emb_std=0.3, batch=4, L=7, tie_levels=16, d=256),
    variant("sampled", emb_std=0.3, batch=6, V=50000, d=256, temperature=0.7, walk_seed=12345),
    variant("sampled", emb_std=0.3, batch=3, V=50000, d=256, L=5, temperature=2.0, walk_seed=2**63 + 5),
    variant("throughput", emb_std=0.3, batch=3, V=40000, d=1024),
    # 256 rows: 16-row gate tiles with a K split 2, 1 and 1 wide for d = 256, 128, 64, so
    # the pair kernel adds the partial sums itself (or the tiles finish the gate)
    variant("small_batch", emb_std=0.3, batch=16, V=20000, d=256),
    variant("small_batch", emb_std=0.3, batch=16, V=20000, d=128),
    variant("small_batch", emb_std=0.3, batch=16, V=20000, d=64),
    # 600 rows, d = 16384: the LDS-DMA gate over 20 K splits, all added by the pair kernel
    variant("small_batch", emb_std=0.3, batch=40, L=15, V=20000, d=16384),
    # either side of the batch size where the pair scores change path: up to 128 sequences a
    # wave per position writes the pair tensor and a second launch walks it, beyond that one
    # workgroup per sequence scores and walks
    variant("sampled", emb_std=0.3, batch=128, V=4096, d=256, temperature=0.9, walk_seed=99),
    variant("sampled", emb_std=0.3, batch=129, V=4096, d=256, temperature=0.9, walk_seed=99),
    # the best-total-path walk
    variant("tiny", emb_std=0.3, walk="viterbi"),
    variant("tiny", emb_std=0.3, L=1, walk="viterbi"),
    variant("single_stream", emb_std=0.3, batch=6, V=32001, d=512, walk="viterbi"),
    variant("single_stream", emb_std=0.3, batch=4, L=7, tie_levels=16, d=256, walk="viterbi"),
    variant("throughput", emb_std=0.3, batch=3, V=40000, d=1024, walk="viterbi"),
]


@pytest.mark.parametrize("cfg", VARIANTS, ids=lambda c: c.name)
def test_select_variants(cfg):
    inp = make(cfg)
    print(f"select variant {cfg.name}", flush=True)
    path, scores = _select(upload(inp), cfg)
    _check(inp, path, scores, range(cfg.batch))
    if cfg.emb_std >= 0.3 and cfg.walk == "greedy":
        # the bilinear term must matter: some step leaves the per-position top-1
        top1 = np.stack([oracle.top16_rows(oracle.widen(inp.logits[i], cfg.dtype))[0][:, 0]
                         for i in range(cfg.batch)])
        if cfg.L > 1:
            assert (path != top1).any()


@pytest.mark.parametrize("cfg", [variant("single_stream", emb_std=0.3, batch=5, V=20000, d=256),
                                 variant("small_batch", emb_std=0.3, batch=16, V=20000, d=256),
                                 variant("small_batch", emb_std=0.3, batch=16, V=20000, d=128),
                                 variant("small_batch", emb_std=0.3, batch=16, V=20000, d=64),
                                 variant("throughput", emb_std=0.3, batch=128, V=4096, d=256),
                                 variant("throughput", emb_std=0.3, batch=129, V=4096, d=256)],
                         ids=lambda c: f"{c.batch}x{c.L}x{c.V}_d{c.d}")
def test_select_equals_step_chain(cfg):
    import draft_selection_position_amd as dfs

    dev = upload(make(cfg))
    idx, val = dfs.topk(dev["logits"])
    g = dfs.gate(dev["hidden"], dev["W_h"])
    pair = dfs.pair_scores(idx, val, dev["prev_token"], g, dev["A"], dev["B"])
    for mode, T, seed in (("greedy", 1.0, 0), ("gumbel", 0.8, 77), ("viterbi", 1.0, 0)):
        path, scores = dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"],
                                  dev["W_h"], mode=mode, temperature=T, seed=seed)
        p2, s2 = dfs.walk(pair, idx, mode, T, seed)
        torch.cuda.synchronize()
        assert torch.equal(path, p2), mode
        assert torch.equal(scores, s2), mode


def test_select_is_deterministic(full_workload):
    inp, dev = full_workload("small_batch")
    first = _select(dev, inp.config)
    for _ in range(10):
        again = _select(dev, inp.config)
        np.testing.assert_array_equal(first[0], again[0])
        np.testing.assert_array_equal(first[1], again[1])


@pytest.mark.parametrize("name", ["small_batch", "sampled", "throughput"])
def test_select_equals_step_chain_full_size(name, full_workload):
    # the fused selector finishes the gate differently at each size (a finish kernel
    # of its own, or inside the pair kernel at 4096 rows) and packs W_h inside the
    # top-16 launch; none of that may change a bit
    import draft_selection_position_amd as dfs

    inp, dev = full_workload(name)
    cfg = inp.config
    path, scores = _select(dev, cfg)
    idx, val = dfs.topk(dev["logits"])
    g = dfs.gate(dev["hidden"], dev["W_h"])
    pair = dfs.pair_scores(idx, val, dev["prev_token"], g, dev["A"], dev["B"])
    p2, s2 = dfs.walk(pair, idx, cfg.walk, cfg.temperature, cfg.walk_seed)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(path, p2.cpu().numpy())
    np.testing.assert_array_equal(scores, s2.cpu().numpy())


@pytest.mark.parametrize("name", ["small_batch", "throughput"])
def test_best_path_full_size(name, full_workload):
    # the best-total-path walk at a full benchmark shape: sampled sequences against
    # the oracle, every sequence's total at least the greedy walk's
    import draft_selection_position_amd as dfs

    inp, dev = full_workload(name)
    cfg = variant(inp.config, walk="viterbi")
    args = (dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], dev["W_h"])
    vp, vs = dfs.select(*args, mode="viterbi")
    gp, gs = dfs.select(*args, mode="greedy")
    torch.cuda.synchronize()
    vs64, gs64 = vs.cpu().double().sum(1), gs.cpu().double().sum(1)
    assert bool((vs64 >= gs64 - 1e-3).all())
    vp, vs = vp.cpu().numpy(), vs.cpu().numpy()
    seqs = np.unique(np.r_[0, cfg.batch - 1, np.random.default_rng(5).choice(cfg.batch, 6, replace=False)])
    for i in seqs:
        res = oracle.select_sequence(inp, int(i))
        path, scores, slots, margins = oracle.viterbi(res.pair, res.cand_idx)
        res.path, res.scores, res.slots, res.margins = path, scores, slots, margins
        check_path(vp[i], vs[i], res, "viterbi", b=int(inp.seq_ids[i]))


def test_select_many_rows_unsplit_gate():
    # 16384 rows: the top-16 pass keeps every row whole, and the gate GEMM's 128 x 128 tiles
    # fill the chip without a K split (the sigmoid in its own epilogue); the fused call must
    # equal the step chain bit for bit and the oracle on sampled sequences
    import draft_selection_position_amd as dfs

    cfg = variant("throughput", emb_std=0.3, batch=1024, V=4096, d=256)
    inp = make(cfg)
    dev = upload(inp)
    print(f"select many rows: batch {cfg.batch} L {cfg.L} V {cfg.V} d {cfg.d}", flush=True)
    path, scores = _select(dev, cfg)
    idx, val = dfs.topk(dev["logits"])
    g = dfs.gate(dev["hidden"], dev["W_h"])
    pair = dfs.pair_scores(idx, val, dev["prev_token"], g, dev["A"], dev["B"])
    p2, s2 = dfs.walk(pair, idx, cfg.walk, cfg.temperature, cfg.walk_seed)
    torch.cuda.synchronize()
    assert np.array_equal(path, p2.cpu().numpy())
    assert np.array_equal(scores, s2.cpu().numpy())
    seqs = np.unique(np.r_[0, cfg.batch - 1, np.random.default_rng(4).choice(cfg.batch, 22, replace=False)])
    _check(inp, path, scores, seqs)


@pytest.mark.parametrize("batch,d,splits", [(263, 1024, 4), (375, 768, 3), (512, 512, 2), (131, 256, 1)],
                         ids=lambda v: str(v))
def test_select_ragged_rows_each_gate_split(batch, d, splits):
    # unsplit top-16 rows, row counts that are not a multiple of the gate's 128-row tiles,
    # and each K split the pair kernel adds up itself (1 to 4): the fused call must equal
    # the step chain bit for bit, and the oracle on sampled sequences
    import draft_selection_position_amd as dfs

    cfg = variant("throughput", emb_std=0.3, batch=batch, V=4096, d=d)
    rows = cfg.batch * cfg.L
    kb = d // 32
    items = -(-rows // 128) * 2
    s = min(max(-(-256 // items), 1), max(kb // 8, 1))
    assert -(-kb // -(-kb // s)) == splits  # the gate plan's split count for this shape
    inp = make(cfg)
    dev = upload(inp)
    print(f"select ragged rows: rows {rows} d {d} gate splits {splits}", flush=True)
    path, scores = _select(dev, cfg)
    idx, val = dfs.topk(dev["logits"])
    g = dfs.gate(dev["hidden"], dev["W_h"])
    pair = dfs.pair_scores(idx, val, dev["prev_token"], g, dev["A"], dev["B"])
    p2, s2 = dfs.walk(pair, idx, cfg.walk, cfg.temperature, cfg.walk_seed)
    torch.cuda.synchronize()
    assert np.array_equal(path, p2.cpu().numpy())
    assert np.array_equal(scores, s2.cpu().numpy())
    seqs = np.unique(np.r_[0, cfg.batch - 1, np.random.default_rng(6).choice(cfg.batch, 8, replace=False)])
    _check(inp, path, scores, seqs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_select_few_rows_adversarial_logits(dtype):
    """One sequence of 16 x 151936 (the fused launch whose chunks are held in registers):
    rows where every element reaches the threshold (all equal: more keys than a wave's
    buffer holds), ascending and descending rows, signed zeros, -inf and a few tied
    levels.  The drafted candidates equal the oracle's top-16 of every row."""
    import draft_selection_position_amd as dfs
    from workloads import f32_to_bf16_bits

    from .parity import to_dev

    cfg = variant("single_stream", emb_std=0.3, dtype=dtype, d=256)
    V = cfg.V
    rng = np.random.default_rng(11)
    patterns = [
        np.zeros(V, np.float32),
        np.arange(V, dtype=np.float32),
        np.arange(V, dtype=np.float32)[::-1].copy(),
        rng.choice(np.array([0.0, -0.0, 1.0], np.float32), V),
        np.where(rng.random(V) < 0.5, np.float32(-np.inf), np.float32(2.5)),
        np.round(rng.standard_normal(V)).astype(np.float32),
    ]
    rows = np.stack([patterns[i % len(patterns)] for i in range(cfg.L)])
    if dtype == "bf16":
        rows = f32_to_bf16_bits(rows)
    dev = upload(make(cfg))
    dev["logits"] = to_dev(rows.reshape(1, cfg.L, V))
    W = dfs.gate_pack(dev["W_h"]) if dtype == "bf16" else dev["W_h"]
    print(f"select few rows adversarial {dtype}", flush=True)
    _, _, _, cand = dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], W, draft=True)
    torch.cuda.synchronize()
    cand = cand.cpu().numpy().reshape(cfg.L, 16)
    for r in range(cfg.L):
        oi, _ = oracle.top16(oracle.widen(rows[r], dtype))
        np.testing.assert_array_equal(cand[r], oi, err_msg=f"row {r}")
