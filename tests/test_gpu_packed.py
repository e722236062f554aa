"""GPU: the pre-packed gate weight, the pair kernel's merge of split top-16 rows, and
calls on concurrent streams.  Every comparison here is bitwise: the packed and unpacked
weights, the fused selector and the step chain, and the two streams must agree exactly."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make, variant

from .parity import check_path, upload

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


# rows = batch * L: 8 and 16 (the gate's tiles ride in the top-16 launch when W_h is
# packed, per-position pair workgroups), 80, 195, 320 and 512 (the gate's tiles still in
# the top-16 launch, 256-way K split, one pair workgroup per sequence), 1 (one row split
# 64 ways), 600 (LDS-DMA gate); fp32 (tiny); d not a multiple of 32
SHAPES = [
    variant("tiny", emb_std=0.3),
    variant("single_stream", emb_std=0.3, V=151936, d=5120),
    variant("single_stream", emb_std=0.3, batch=5, V=20000, d=256),
    variant("single_stream", emb_std=0.3, batch=1, L=1, V=262144, d=512),
    variant("single_stream", emb_std=0.3, batch=3, L=7, V=32001, d=72),
    variant("small_batch", emb_std=0.3, batch=13, L=15, V=32001, d=72),
    variant("small_batch", emb_std=0.3, batch=20, L=16, V=20000, d=1024),
    variant("small_batch", emb_std=0.3, batch=32, L=16, V=20000, d=5120),
    variant("small_batch", emb_std=0.3, batch=40, L=15, V=20000, d=1024),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_packed_equals_unpacked_and_chain(cfg):
    dfs = dfs_mod()
    inp = make(cfg)
    dev = upload(inp)
    print(f"packed {cfg.name}: rows {cfg.batch * cfg.L} V {cfg.V} d {cfg.d}", flush=True)
    Wp = dfs.gate_pack(dev["W_h"])
    args = (dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"])
    g1 = dfs.gate(dev["hidden"], dev["W_h"])
    g2 = dfs.gate(dev["hidden"], Wp)
    idx, val = dfs.topk(dev["logits"])
    pair = dfs.pair_scores(idx, val, dev["prev_token"], g1, dev["A"], dev["B"])
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    for mode, T, seed in (("greedy", 1.0, 0), ("gumbel", 0.8, 77), ("viterbi", 1.0, 0)):
        p1, s1 = dfs.select(*args, dev["W_h"], mode=mode, temperature=T, seed=seed)
        p2, s2 = dfs.select(*args, Wp, mode=mode, temperature=T, seed=seed)
        p3, s3 = dfs.walk(pair, idx, mode, T, seed)
        d1 = dfs.select(*args, dev["W_h"], mode=mode, temperature=T, seed=seed, draft=True)
        d2 = dfs.select(*args, Wp, mode=mode, temperature=T, seed=seed, draft=True)
        torch.cuda.synchronize()
        assert torch.equal(p1, p2) and torch.equal(s1, s2), mode
        assert torch.equal(p1, p3) and torch.equal(s1, s3), mode
        for a, b in zip(d1, d2):
            assert torch.equal(a, b), mode
        assert torch.equal(d1[0], p1) and torch.equal(d1[1], s1), mode
        assert torch.equal(d1[3], idx.view(cfg.batch, cfg.L, 16)), mode  # the merged candidates
    # and the oracle, on every sequence
    path, scores = (x.cpu().numpy() for x in dfs.select(*args, Wp, mode=cfg.walk, temperature=cfg.temperature,
                                                        seed=cfg.walk_seed))
    for i in range(cfg.batch):
        res = oracle.select_sequence(inp, i)
        check_path(path[i], scores[i], res, cfg.walk, cfg.temperature, cfg.walk_seed, i)


def test_selector_class_with_packed_weight():
    dfs = dfs_mod()
    cfg = variant("single_stream", emb_std=0.3, batch=2, V=20000, d=256)
    dev = upload(make(cfg))
    sel = dfs.Selector(cfg.batch, cfg.L, cfg.V, cfg.d)
    args = (dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"])
    p1, s1 = (x.clone() for x in sel(*args, dev["W_h"]))
    p2, s2 = sel(*args, dfs.gate_pack(dev["W_h"]))
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(s1, s2)
    with pytest.raises(ValueError):
        sel(*args, dfs.gate_pack(torch.zeros((128, 256), dtype=torch.bfloat16, device="cuda")))


def test_two_streams_concurrently():
    """Calls without an explicit workspace on two streams at once (each stream gets its
    own cached scratch) equal the same calls made one after the other."""
    dfs = dfs_mod()
    cfgs = [variant("single_stream", emb_std=0.3, batch=4, V=60000, d=1024, base_seed=0xDF60 + s) for s in (0, 1)]
    devs = [upload(make(c)) for c in cfgs]
    want = []
    for dev in devs:
        want.append([x.clone() for x in dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"],
                                                    dev["B"], dev["W_h"])])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [[], []]
    for rep in range(20):
        for i, (s, dev) in enumerate(zip(streams, devs)):
            with torch.cuda.stream(s):
                got[i].append(dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"],
                                         dev["W_h"]))
    torch.cuda.synchronize()
    for i in range(2):
        for p, sc in got[i]:
            assert torch.equal(p, want[i][0]) and torch.equal(sc, want[i][1])
    keys = {k for k in dfs._WS._bufs if k[0] == devs[0]["logits"].device}
    assert len(keys) >= 3  # the default stream's buffer and one per side stream
