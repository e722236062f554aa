"""Pins of the fused-LM-head top-16 oracle (oracle/lmhead.py): a one-hot hidden state
selects one weight column (closed form), scalar fsum dot products on a tiny case, and
the top-16 of the result equals heapq.nlargest over the brute-force logits."""
import heapq
import math

import numpy as np

from oracle import lmhead
from workloads.configs import variant
from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits
from workloads.lmhead import make_lm_head


def test_one_hot_hidden_selects_a_weight_column():
    rng = np.random.default_rng(1)
    V, d = 300, 64
    W = rng.standard_normal((V, d)).astype(np.float32)
    h = np.zeros((3, d), np.float32)
    h[0, 5] = 1.0
    h[1, 63] = -2.0
    h[2, 0] = 0.5
    U = lmhead.logits(h, W, "f32")
    np.testing.assert_array_equal(U[0], W[:, 5].astype(np.float64))
    np.testing.assert_array_equal(U[1], -2.0 * W[:, 63].astype(np.float64))
    ids, vals = lmhead.top16(h, W, "f32")
    want = sorted(range(V), key=lambda i: (-float(W[i, 5]), i))[:16]
    assert list(ids[0]) == want


def test_scalar_dot_products_and_heap_top16():
    rng = np.random.default_rng(2)
    V, d = 97, 32
    W = f32_to_bf16_bits(rng.standard_normal((V, d)).astype(np.float32) * 0.3)
    h = f32_to_bf16_bits(rng.standard_normal((2, d)).astype(np.float32))
    Wf, hf = bf16_bits_to_f32(W).astype(np.float64), bf16_bits_to_f32(h).astype(np.float64)
    U = lmhead.logits(h, W, "bf16")
    ids, vals = lmhead.top16(h, W, "bf16")
    for r in range(2):
        brute = [math.fsum(hf[r, k] * Wf[v, k] for k in range(d)) for v in range(V)]
        np.testing.assert_allclose(U[r], brute, rtol=1e-13, atol=1e-13)
        top = heapq.nlargest(16, ((b, -v) for v, b in enumerate(brute)))
        assert list(ids[r]) == [-nv for _, nv in top]
        np.testing.assert_allclose(vals[r], [b for b, _ in top], rtol=1e-13, atol=1e-13)


def test_generator_blocks_and_scale():
    cfg = variant("single_stream", d=256)
    W = make_lm_head(cfg, V=9000)
    W2 = make_lm_head(cfg, V=9000, threads=1)
    np.testing.assert_array_equal(W, W2)
    assert W.shape == (9000, 256) and W.dtype == np.uint16
    assert abs(bf16_bits_to_f32(W).std() - 0.02) < 0.001
