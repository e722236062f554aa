"""dfs_conv2 (two-tap dynamic depthwise convolution) on the GPU against the oracle."""
import numpy as np
import pytest
import torch

from oracle import conv as oconv
from workloads.configs import variant
from workloads.conv import make_conv
from workloads.gen import bf16_bits_to_f32

from .parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dfs_mod():
    import draft_selection_position_amd as dfs

    return dfs


def _wide(a, dtype):
    return (bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


def _run(ci):
    y = dfs_mod().conv2(to_dev(ci.x), to_dev(ci.x_prev), to_dev(ci.base), to_dev(ci.W_c))
    torch.cuda.synchronize()
    y = y.cpu()
    return _wide(y.view(torch.int16).numpy().view(np.uint16), "bf16") if ci.dtype == "bf16" else \
        y.numpy().astype(np.float64)


def _check(ci, y_gpu, seqs=None):
    """|y_gpu - y| within the bound of fp32 sums (D 2^-24 sum |x W| on the correction,
    2^-22 on the two products) plus, for bf16 output, one rounding (2^-8 relative)."""
    x, xp = _wide(ci.x, ci.dtype), _wide(ci.x_prev, ci.dtype)
    base, W = _wide(ci.base, ci.dtype), _wide(ci.W_c, ci.dtype)
    y = oconv.conv2(x, xp, base, W)
    D = x.shape[-1]
    cabs = oconv.correction(np.abs(x), np.abs(W))  # [B, L, G, 2]
    cerr = np.repeat(np.swapaxes(cabs, -1, -2), 16, axis=-1) * (D * 2.0 ** -24)  # [B, L, 2, D]
    pred = np.concatenate([xp[:, None], x[:, :-1]], axis=1)
    k = oconv.coefficients(x, base, W)
    e1 = np.abs(x) * cerr[:, :, 0] + np.abs(pred) * cerr[:, :, 1] + \
        2.0 ** -22 * (np.abs(k[:, :, 0] * x) + np.abs(k[:, :, 1] * pred)) + 1e-30
    rel = 2.0 ** -8 if ci.dtype == "bf16" else 0.0
    bound = rel * np.abs(y) + 2.0 * e1
    err = np.abs(y_gpu - y)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert (err <= bound).all(), (worst, y_gpu[worst], y[worst], bound[worst])
    return float((err / np.maximum(np.abs(y), 1e-6)).max())


CASES = [
    # (batch, L, D): one tile; ragged rows and a 32-column last N tile; three waves busy; full width
    (3, 5, 256), (37, 16, 1280), (5, 7, 768), (2, 16, 5120), (1, 1, 512), (9, 3, 4096),
    # enough rows for unsplit 128 x 64 tiles, with a 32-column last tile
    (688, 16, 1280),
    # a K split whose epilogue walks runs of four positions per thread, L not a multiple of 4
    (4096, 7, 1024),
]


@pytest.mark.parametrize("batch,L,D", CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("corr", [0.002, 0.02])
def test_conv2_bf16_matches_oracle(batch, L, D, corr):
    ci = make_conv(variant("throughput", batch=batch, L=L, d=D), corr_std=corr)
    worst = _check(ci, _run(ci))
    print(f"conv2 bf16 {batch}x{L}x{D} corr {corr}: worst relative error {worst:.2e}", flush=True)


@pytest.mark.parametrize("batch,L,D", [
    # one 8-row tile; ragged rows; only the first of four waves has a K slice; five K slices
    # over four waves and a ragged last row tile; the widest workload
    (1, 8, 1024), (3, 5, 512), (2, 16, 256), (37, 16, 256), (5, 7, 1280), (4, 16, 5120),
], ids=lambda v: str(v))
def test_conv2_f32_matches_oracle(batch, L, D):
    ci = make_conv(variant("tiny", batch=batch, L=L, d=D), corr_std=0.02)
    _check(ci, _run(ci))


def test_conv2_full_size_sampled_sequences():
    # The throughput shape (256 x 16 x 5120, bf16) in one launch, as timed; 40 sequences
    # checked against the oracle (the generator regenerates any subset bit-identically).
    cfg = variant("throughput")
    ci = make_conv(cfg)
    y = _run(ci)
    seqs = np.random.default_rng(3).choice(cfg.batch, 40, replace=False)
    sub = make_conv(cfg, seqs=seqs)
    _check(sub, y[seqs])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv2_identity_and_shift_are_exact(dtype):
    cfg = variant("throughput", batch=6, L=9, d=1024, dtype=dtype)
    ci = make_conv(cfg)
    one = np.zeros((2, 1024), np.float32)
    one[0] = 1.0
    shift = one[::-1].copy()
    W = np.zeros_like(ci.W_c)
    for kern, want in ((one, ci.x), (shift, np.concatenate([ci.x_prev[:, None], ci.x[:, :-1]], axis=1))):
        b = (np.asarray(kern.view(np.uint32) >> 16, np.uint16) if dtype == "bf16" else kern)
        y = dfs_mod().conv2(to_dev(ci.x), to_dev(ci.x_prev), to_dev(b), to_dev(W))
        torch.cuda.synchronize()
        got = y.cpu().view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else y.cpu().numpy()
        np.testing.assert_array_equal(got, want)


def test_conv2_is_deterministic_and_writes_out():
    ci = make_conv(variant("throughput", batch=8, L=16, d=2048), corr_std=0.02)
    args = (to_dev(ci.x), to_dev(ci.x_prev), to_dev(ci.base), to_dev(ci.W_c))
    y1 = dfs_mod().conv2(*args)
    out = torch.full_like(y1, 7)
    y2 = dfs_mod().conv2(*args, out=out)
    torch.cuda.synchronize()
    assert y2.data_ptr() == out.data_ptr()
    assert torch.equal(y1, y2)


def test_conv2_fixed_shape_object_matches_function():
    ci = make_conv(variant("throughput", batch=3, L=16, d=1024), corr_std=0.02)
    args = (to_dev(ci.x), to_dev(ci.x_prev), to_dev(ci.base), to_dev(ci.W_c))
    c = dfs_mod().Conv2(3, 16, 1024)
    y = c(*args)
    torch.cuda.synchronize()
    assert torch.equal(y, dfs_mod().conv2(*args))
    with pytest.raises(ValueError):
        c(args[0][:, :8].contiguous(), *args[1:])
