"""GPU parity of dfs_topk against the oracle's full stable sort (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make, variant

from .oracle_pool import stack
from .parity import record, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_selection_position_amd as dfs

    dfs.lib()  # a machine with a GPU but without the built library must fail, not skip


def _run(rows_np, dtype):
    import draft_selection_position_amd as dfs

    x = to_dev(rows_np)
    idx, val = dfs.topk(x)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def _check_rows(rows_np, dtype, idx, val, which):
    for r in which:
        oi, ov = oracle.top16(oracle.widen(rows_np[r], dtype))
        np.testing.assert_array_equal(idx[r], oi, err_msg=f"row {r}")
        np.testing.assert_array_equal(val[r].astype(np.float64), ov, err_msg=f"row {r}")
        assert not np.signbit(val[r][val[r] == 0]).any()


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_topk_full_size_configs(cfg, full_workload, full_oracle):
    # full-size launch; every row against the oracle's stable sort, bit for bit
    import draft_selection_position_amd as dfs

    inp, dev = full_workload(cfg.name)
    rows = cfg.batch * cfg.L
    print(f"topk {cfg.name}: rows {rows} V {cfg.V}", flush=True)
    idx, val = dfs.topk(dev["logits"].view(-1, cfg.V))
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    want = full_oracle(cfg.name)
    oi = stack(want, "cand_idx").reshape(rows, 16)
    ov = stack(want, "cand_val").reshape(rows, 16)
    bad = np.nonzero((idx != oi).any(1) | (val.astype(np.float64) != ov).any(1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:8].tolist()}"
    assert not np.signbit(val[val == 0]).any()
    record("topk", cfg.name, rows, "rows", "bit-exact ids and values")


VARIANTS = [
    dict(V=32001, batch=3),  # rows not 16-byte aligned
    dict(V=16, batch=2),
    dict(V=17, batch=2),
    dict(V=100, batch=2),
    dict(V=4103, batch=2),  # several chunks and a ragged tail
    dict(V=50000, batch=2, tie_levels=8),  # heavy ties at every level
    dict(V=50000, batch=2, neg_inf_frac=0.9997, peak_kind="none"),  # rows with < 16 finite values
    dict(V=151936, batch=2, zipf_ids=True),  # peaks clustered at low ids
    dict(V=262144, batch=1, L=3),
    dict(V=4190208, batch=1, L=2),  # rows of 8 MB (bf16), split into the most chunks
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kw", VARIANTS, ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
def test_topk_variants(kw, dtype):
    cfg = variant("single_stream", d=64, dtype=dtype, **kw)
    inp = make(cfg)
    rows = inp.logits.reshape(-1, cfg.V)
    print(f"topk variant {cfg.name}", flush=True)
    idx, val = _run(rows, dtype)
    _check_rows(rows, dtype, idx, val, range(rows.shape[0]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_adversarial_rows(dtype):
    V = 20000
    rng = np.random.default_rng(3)
    rows = np.stack([
        np.arange(V, dtype=np.float32),  # ascending: every element beats the running threshold
        np.arange(V, dtype=np.float32)[::-1],
        np.zeros(V, np.float32),  # all tied: ids 0..15
        rng.choice(np.array([0.0, -0.0, 1.0], np.float32), V),
        np.full(V, -np.inf, np.float32),
        np.where(rng.random(V) < 0.5, np.float32(-np.inf), np.float32(2.5)),
    ]).astype(np.float32)
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits

        rows = f32_to_bf16_bits(rows)
    idx, val = _run(rows, dtype)
    _check_rows(rows, dtype, idx, val, range(rows.shape[0]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_adversarial_rows_two_rounds(dtype):
    """More rows than one round of workgroups holds (2304 > 2048 workgroups): there the pass
    raises its shared threshold from all four waves' published list values at every merge.
    Rows that admit every element, rows of ties at one or a few levels, signed zeros, -inf,
    and unaligned rows (V = 6001)."""
    V = 6001
    rng = np.random.default_rng(5)
    base = [
        np.arange(V, dtype=np.float32),  # ascending: every element beats the running threshold
        np.arange(V, dtype=np.float32)[::-1].copy(),
        rng.permutation(V).astype(np.float32),
        np.zeros(V, np.float32),  # all tied: ids 0..15
        rng.choice(np.array([0.0, -0.0, 1.0], np.float32), V),
        np.full(V, -np.inf, np.float32),
        np.where(rng.random(V) < 0.5, np.float32(-np.inf), np.float32(2.5)),
        np.round(rng.standard_normal(V) * 2).astype(np.float32),  # a few levels, heavy ties
        rng.standard_normal(V).astype(np.float32),
    ]
    rows = np.stack([base[i % len(base)] for i in range(2304)])
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits

        rows = f32_to_bf16_bits(rows)
    print(f"topk adversarial rows 2304 x {V} {dtype}", flush=True)
    idx, val = _run(rows, dtype)
    _check_rows(rows, dtype, idx, val, range(rows.shape[0]))


def test_topk_repeatable():
    cfg = variant("small_batch", d=64, batch=8)
    x = to_dev(make(cfg).logits.reshape(-1, cfg.V))
    import draft_selection_position_amd as dfs

    first = [t.cpu() for t in dfs.topk(x)]
    for _ in range(5):
        again = [t.cpu() for t in dfs.topk(x)]
        assert all(torch.equal(a, b) for a, b in zip(first, again))
