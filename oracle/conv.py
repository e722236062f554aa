"""Two-tap dynamic depthwise convolution, in fp64.  TEST INFRASTRUCTURE ONLY.

Source: the blog post "DFlash 2: Keep Drafting Parallel" (Inco AI, 2026),
section "A Lightweight Local Convolution" (wpnews.pro copy), with the equation
kept in the twiscan.com Chinese translation and the decomputer.nl Dutch one:

    Conv_k(x)_t = k_{t,0} (elementwise) x_t + k_{t,1} (elementwise) x_{t-1}

Two taps, one on the current block position and one on its predecessor.  Each
coefficient is a learned base kernel plus a small correction computed from the
current hidden state, and every 16 channels share one correction.  Position 0
reads the last verified token's representation; every later position reads its
in-block predecessor.  All positions are computed at once.

Readings of what the pages leave open (kept identical in the HIP library):
  * "current hidden state" is the convolution's own input at position t, x_t.
  * The correction is linear: c_t = W_c x_t, with W_c of shape [D/16, 2, D]
    (group g, tap) -> one weight vector over the D input channels; no bias (a
    per-group bias would fold into the base kernel) and no nonlinearity.
  * k_{t,tap}[ch] = base[tap, ch] + c_t[ch // 16, tap], base of shape [2, D];
    tap 0 multiplies x_t, tap 1 multiplies the predecessor.
  * The predecessor of position 0 is x_prev [D], one vector per sequence.
Consistency check of the reading (not a pin): five drafter layers with a
convolution before and after each attention and feed-forward sublayer are 20
convolutions, each with 2D base weights and D * 2D/16 correction weights; at a
hidden width of 2560 that is 20 * (5120 + 819200) = 16.5M parameters, the
post's figure.  (The width is not on the pages.)
"""
from __future__ import annotations

import numpy as np

GROUP = 16  # channels sharing one correction


def correction(x: np.ndarray, W_c: np.ndarray) -> np.ndarray:
    """c [..., D/16, 2] = W_c x for every position: x [..., D], W_c [D/16, 2, D]."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W_c, np.float64)
    G, taps, D = W.shape
    if taps != 2 or D != x.shape[-1] or G * GROUP != D:
        raise ValueError(f"W_c must be [D/16, 2, D] for D = {x.shape[-1]}, got {W.shape}")
    return (x @ W.reshape(G * taps, D).T).reshape(x.shape[:-1] + (G, taps))


def coefficients(x: np.ndarray, base: np.ndarray, W_c: np.ndarray) -> np.ndarray:
    """k [..., 2, D]: base[tap, ch] + c[..., ch // 16, tap]."""
    c = correction(x, W_c)  # [..., G, 2]
    per_channel = np.repeat(np.swapaxes(c, -1, -2), GROUP, axis=-1)  # [..., 2, D]
    return np.asarray(base, np.float64) + per_channel


def conv2(x: np.ndarray, x_prev: np.ndarray, base: np.ndarray, W_c: np.ndarray) -> np.ndarray:
    """y [B, L, D] for x [B, L, D], x_prev [B, D], base [2, D], W_c [D/16, 2, D]."""
    x = np.asarray(x, np.float64)
    xp = np.asarray(x_prev, np.float64)
    if x.ndim != 3 or xp.shape != (x.shape[0], x.shape[2]):
        raise ValueError("x must be [B, L, D] and x_prev [B, D]")
    pred = np.concatenate([xp[:, None, :], x[:, :-1, :]], axis=1)  # x_{t-1}, x_{-1} = x_prev
    k = coefficients(x, base, W_c)  # [B, L, 2, D]
    return k[:, :, 0, :] * x + k[:, :, 1, :] * pred
