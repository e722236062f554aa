"""Top-16 straight from the drafter's hidden state, in fp64.  TEST INFRASTRUCTURE ONLY.

Source: blog post "DFlash 2: Keep Drafting Parallel" (Inco AI, 2026), section "A
Lightweight Path Selector": the selector reads the drafter's own logits U_t and
needs no extra backbone or LM-head pass.  The logits are the drafter's LM head
applied to its hidden state, U_t = W_lm h_t over the vocabulary, and the
candidates are the 16 largest of them (section "The Right Tokens Are Already
There").  Computing the top-16 directly from h_t and W_lm gives the same
candidates without the logits ever being stored.

Readings: W_lm is [V, d] (one row of d weights per token); no bias; the order and
tie rules are those of ``selector.top16`` (value descending, then lower id).
"""
from __future__ import annotations

import numpy as np

from .selector import top16_rows, widen


def logits(hidden: np.ndarray, W_lm: np.ndarray, dtype: str) -> np.ndarray:
    """U [rows, V] = h W_lm^T in fp64 from exactly widened inputs."""
    h = widen(hidden, dtype).reshape(-1, np.shape(hidden)[-1])
    return h @ widen(W_lm, dtype).T


def top16(hidden: np.ndarray, W_lm: np.ndarray, dtype: str):
    """(ids [rows, 16], values [rows, 16]) of U = h W_lm^T, full sort per row."""
    return top16_rows(logits(hidden, W_lm, dtype))
