"""GPU: dfs_select_packed_static (the library's own static scratch, no workspace argument)
against dfs_select_packed with a caller workspace, through the C ABI, on calls in a row
whose inputs shrink; results must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from workloads import make, variant

from .parity import check_path, upload

pytestmark = pytest.mark.gpu

TOO_LARGE = 9


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_selection_position_amd as dfs

    dfs.lib()


def _shape(dfs, cfg, dev):
    c = lambda t: dfs.BF16 if t == torch.bfloat16 else dfs.F32  # noqa: E731
    return dfs._Shape(cfg.batch, cfg.L, cfg.V, cfg.d, c(dev["logits"].dtype), c(dev["hidden"].dtype),
                      c(dev["A"].dtype))


def _static(dfs, cfg, dev, Wp, mode, T, seed):
    L = dfs.lib()
    s = _shape(dfs, cfg, dev)
    path = torch.empty((cfg.batch, cfg.L), dtype=torch.int32, device="cuda")
    scores = torch.empty((cfg.batch, cfg.L), dtype=torch.float32, device="cuda")
    rc = L.dfs_select_packed_static(dev["logits"].data_ptr(), dev["hidden"].data_ptr(), dev["prev_token"].data_ptr(),
                                    dev["A"].data_ptr(), dev["B"].data_ptr(), Wp.data_ptr(), 16, ctypes.byref(s),
                                    dfs._MODES[mode], float(T), int(seed), path.data_ptr(), scores.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0, dfs.status_str(rc)
    return path, scores


def test_static_scratch_matches_workspace_entry_point():
    import draft_selection_position_amd as dfs

    # largest first, then smaller: many rows (per-sequence pair kernel, LDS-DMA gate), then
    # few rows (gate tiles in the top-16 launch, per-position pair kernel), then fp32
    cfgs = [
        variant("small_batch", emb_std=0.3, batch=40, L=16, V=60000, d=2048),
        variant("single_stream", emb_std=0.3, batch=2, L=8, V=20000, d=256),
        variant("tiny", emb_std=0.3, batch=1, L=5, V=5000, d=128),
    ]
    for cfg in cfgs:
        inp = make(cfg)
        dev = upload(inp)
        Wp = dfs.gate_pack(dev["W_h"])
        print(f"static scratch: {cfg.name}", flush=True)
        for mode, T, seed in (("greedy", 1.0, 0), ("gumbel", 0.9, 31), ("viterbi", 1.0, 0)):
            p1, s1 = _static(dfs, cfg, dev, Wp, mode, T, seed)
            p2, s2 = dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], Wp,
                                mode=mode, temperature=T, seed=seed)
            p3, s3 = _static(dfs, cfg, dev, Wp, mode, T, seed)  # again: nothing carried over
            torch.cuda.synchronize()
            assert torch.equal(p1, p2) and torch.equal(s1, s2), (cfg.name, mode)
            assert torch.equal(p1, p3) and torch.equal(s1, s3), (cfg.name, mode)
        path, scores = (x.cpu().numpy() for x in _static(dfs, cfg, dev, Wp, cfg.walk, cfg.temperature, cfg.walk_seed))
        for i in range(cfg.batch):
            check_path(path[i], scores[i], oracle.select_sequence(inp, i), cfg.walk, cfg.temperature, cfg.walk_seed, i)


def test_static_scratch_rejects_oversized_calls():
    import draft_selection_position_amd as dfs

    L = dfs.lib()
    s = dfs._Shape(4096, 16, 151936, 5120, dfs.BF16, dfs.BF16, dfs.BF16)
    assert L.dfs_select_workspace_bytes(ctypes.byref(s)) > 32 << 20
    out = torch.full((16,), 7, dtype=torch.int32, device="cuda")
    rc = L.dfs_select_packed_static(out.data_ptr(), out.data_ptr(), out.data_ptr(), out.data_ptr(), out.data_ptr(),
                                    out.data_ptr(), 16, ctypes.byref(s), 0, 1.0, 0, out.data_ptr(), out.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == TOO_LARGE
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 7)  # nothing was launched
