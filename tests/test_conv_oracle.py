"""Pins of the convolution oracle (oracle/conv.py) against what the post and the
mathematics fix: a static kernel is an ordinary two-tap convolution along the
block (numpy.convolve), identity and shift kernels, the group sharing of the
correction, which tap reads which position, and scalar brute force."""
import math

import numpy as np
import pytest

from oracle import conv
from workloads.conv import make_conv
from workloads.configs import variant
from workloads.gen import bf16_bits_to_f32


def _rand(seed, B=2, L=5, D=64, corr=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, D))
    xp = rng.standard_normal((B, D))
    base = rng.standard_normal((2, D))
    W = rng.standard_normal((D // 16, 2, D)) * corr
    return x, xp, base, W


def test_static_kernel_is_numpy_convolve_along_the_block():
    # With W_c = 0 every channel is the sequence (x_prev, x_0, ..., x_{L-1}) convolved
    # with the fixed two-tap kernel (base0, base1); output t is convolve index t + 1.
    x, xp, base, W = _rand(1)
    y = conv.conv2(x, xp, base, np.zeros_like(W))
    B, L, D = x.shape
    for b in range(B):
        for ch in range(D):
            seq = np.concatenate([[xp[b, ch]], x[b, :, ch]])
            full = np.convolve(seq, [base[0, ch], base[1, ch]])
            np.testing.assert_allclose(y[b, :, ch], full[1:L + 1], rtol=1e-14, atol=1e-14)


def test_identity_and_shift_kernels_are_exact():
    x, xp, base, W = _rand(2)
    Z = np.zeros_like(W)
    one = np.zeros_like(base)
    one[0] = 1.0
    np.testing.assert_array_equal(conv.conv2(x, xp, one, Z), x)
    shift = np.zeros_like(base)
    shift[1] = 1.0
    y = conv.conv2(x, xp, shift, Z)
    np.testing.assert_array_equal(y[:, 0], xp)  # position 0 reads the last verified token
    np.testing.assert_array_equal(y[:, 1:], x[:, :-1])  # later positions read their predecessor


def test_taps_groups_and_positions_by_a_planted_case():
    # Only W_c[g=1, tap, j] = alpha is non-zero, base = 0, x_t = s_t e_j with j in group 1.
    # Tap 0: y_t[j] = alpha s_t^2; tap 1: y_t[j] = alpha s_t s_{t-1} (s_{-1} from x_prev);
    # every other channel is 0.  A swapped tap, a wrong group map (ch % G) or a wrong
    # predecessor changes these values.
    B, L, D, j, alpha = 1, 4, 64, 20, 0.75
    s = np.array([1.5, -2.0, 0.5, 3.0])
    sp = -1.25
    x = np.zeros((B, L, D))
    x[0, :, j] = s
    xp = np.zeros((B, D))
    xp[0, j] = sp
    base = np.zeros((2, D))
    for tap, want in ((0, alpha * s * s), (1, alpha * s * np.concatenate([[sp], s[:-1]]))):
        W = np.zeros((D // 16, 2, D))
        W[1, tap, j] = alpha
        y = conv.conv2(x, xp, base, W)
        np.testing.assert_allclose(y[0, :, j], want, rtol=1e-15)
        mask = np.ones(D, bool)
        mask[j] = False
        assert not y[0][:, mask].any()


def test_correction_is_shared_by_exactly_sixteen_channels():
    # Changing group g's correction weights changes channels 16g..16g+15 only, each by
    # (delta . x_t) times its own input (tap 0) -- a closed form.
    x, xp, base, W = _rand(3, D=96)
    g = 4
    delta = np.random.default_rng(9).standard_normal(96)
    W2 = W.copy()
    W2[g, 0] += delta
    dy = conv.conv2(x, xp, base, W2) - conv.conv2(x, xp, base, W)
    inside = np.zeros(96, bool)
    inside[16 * g:16 * g + 16] = True
    assert np.abs(dy[:, :, ~inside]).max() == 0.0
    want = (x @ delta)[:, :, None] * x[:, :, inside]
    np.testing.assert_allclose(dy[:, :, inside], want, rtol=1e-10, atol=1e-12)


def test_position_zero_alone_reads_x_prev():
    x, xp, base, W = _rand(4)
    xp2 = xp + 1.0
    dy = conv.conv2(x, xp2, base, W) - conv.conv2(x, xp, base, W)
    assert np.abs(dy[:, 1:]).max() == 0.0
    k = conv.coefficients(x, base, W)
    np.testing.assert_allclose(dy[:, 0], k[:, 0, 1, :] * 1.0, rtol=1e-14)


def test_scalar_brute_force_with_fsum():
    x, xp, base, W = _rand(5, B=2, L=3, D=32)
    y = conv.conv2(x, xp, base, W)
    B, L, D = x.shape
    for b in range(B):
        for t in range(L):
            pred = xp[b] if t == 0 else x[b, t - 1]
            for ch in range(D):
                g = ch // 16
                k0 = base[0, ch] + math.fsum(W[g, 0, i] * x[b, t, i] for i in range(D))
                k1 = base[1, ch] + math.fsum(W[g, 1, i] * x[b, t, i] for i in range(D))
                assert y[b, t, ch] == pytest.approx(k0 * x[b, t, ch] + k1 * pred[ch], rel=1e-12, abs=1e-13)


def test_bad_shapes_are_rejected():
    x, xp, base, W = _rand(6)
    with pytest.raises(ValueError):
        conv.conv2(x, xp, base, W[:, :1])
    with pytest.raises(ValueError):
        conv.conv2(x, xp[:, :-1], base, W)


def test_generator_subsets_and_dtypes():
    cfg = variant("throughput", batch=6, L=4, d=256)
    full = make_conv(cfg)
    part = make_conv(cfg, seqs=[5, 1])
    np.testing.assert_array_equal(part.x, full.x[[5, 1]])
    np.testing.assert_array_equal(part.x_prev, full.x_prev[[5, 1]])
    np.testing.assert_array_equal(part.W_c, full.W_c)
    assert full.x.dtype == np.uint16 and full.W_c.shape == (16, 2, 256)
    xs = bf16_bits_to_f32(full.x)
    assert abs(xs.std() - 1.0) < 0.05
    tiny = make_conv(variant("tiny", L=3))
    assert tiny.x.dtype == np.float32 and tiny.x.shape == (1, 3, 1024)
