"""Draft probabilities and speculative-sampling verification.  TEST INFRASTRUCTURE ONLY.

The post drafts a block, lets the target model verify it, and notes that sampling
drafts are accepted by rejection sampling, which keeps the target's output
distribution exact (blog post "DFlash 2: Keep Drafting Parallel": section "A
Lightweight Path Selector" for sampling from the same scores, and its discussion
of verification).  The verification rule is the standard one for speculative
sampling (Leviathan, Kalman, Matias, ICML 2023; Chen et al., 2023): draft token
x_t with draft probability q_t(x_t) is accepted with probability
min(1, p_t(x_t) / q_t(x_t)); at the first rejection the output token is drawn
from norm(max(0, p_t - q_t)); when all L are accepted one more token is drawn
from p_L.  The emitted tokens then follow the target distribution p exactly.

Readings taken here (kept identical in the HIP library):
  * q_t is the sampled walk's own distribution: softmax over the 16 candidates of
    S_t(a, .) / T for the drafted predecessor a (the Gumbel-max walk draws from
    exactly this); q is zero off the candidates.
  * the target distribution is softmax(z_t / T_target) over the vocabulary, z the
    target's logits at block position t (row L: the token after the block).
  * random numbers: Philox4x32-10 under key (seed low, seed high); the accept test
    at (block b, position t) uses u = ((x >> 9) + 1/2) 2^-23 from word 0 of counter
    (0, t, b, 1) and accepts when u < p/q; the draw at row k uses
    u = ((x0 >> 9) 2^23 + (x1 >> 9) + 1/2) 2^-46 from words 0, 1 of counter
    (0, k, b, 2) and returns the smallest v whose running sum of weights reaches
    u times their total (inverse CDF, vocabulary order).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import philox4x32_10, uniform_from_word

_MASK = 0xFFFFFFFF


def _key(seed: int):
    return (seed & _MASK, (seed >> 32) & _MASK)


def accept_uniform(seed: int, b: int, t: int) -> float:
    return uniform_from_word(philox4x32_10((0, t, b, 1), _key(seed))[0])


def draw_uniform(seed: int, b: int, k: int) -> float:
    x0, x1 = philox4x32_10((0, k, b, 2), _key(seed))[:2]
    return ((x0 >> 9) * 2.0 ** 23 + (x1 >> 9) + 0.5) * 2.0 ** -46


def softmax(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    return e / e.sum()


def draft_probs(S: np.ndarray, slots: np.ndarray, temperature: float) -> np.ndarray:
    """q [L, 16]: q[t] = softmax(S_t(slot[t-1], .) / T), slot[-1] = 0 (the verified token's row)."""
    L = S.shape[0]
    q = np.empty((L, S.shape[2]))
    prev = 0
    for t in range(L):
        q[t] = softmax(S[t, prev] / temperature)
        prev = int(slots[t])
    return q


def inverse_cdf(w: np.ndarray, u: float) -> tuple[int, float]:
    """Smallest v with sum(w[:v+1]) >= u * sum(w), and the distance of u * sum(w) to
    the nearest boundary of v's interval, as a fraction of sum(w)."""
    c = np.cumsum(np.asarray(w, np.float64))
    total = c[-1]
    target = u * total
    v = int(np.searchsorted(c, target, side="left"))
    v = min(v, len(c) - 1)
    while w[v] <= 0.0 and v > 0:  # rounding past the end: the last token with weight
        v -= 1
    lo = c[v - 1] if v > 0 else 0.0
    return v, float(min(c[v] - target, target - lo) / total)


@dataclass
class Verdict:
    accepted: int          # draft tokens accepted, 0..L
    token: int             # the token drawn at row `accepted` (correction or bonus)
    accept_margin: float   # smallest |u - p/q| over the decisions taken
    draw_margin: float     # distance of the draw to its interval's edge, fraction of the total


def verify_block(target: np.ndarray, path, cand: np.ndarray, q: np.ndarray, temperature: float,
                 seed: int, b: int) -> Verdict:
    """Speculative-sampling verification of one drafted block.

    target [L+1, V] logits, path [L] drafted ids, cand [L, 16] candidate ids,
    q [L, 16] draft probabilities of the candidates (rows of ``draft_probs``)."""
    L = len(path)
    margin = np.inf
    for t in range(L):
        p = softmax(np.asarray(target[t], np.float64) / temperature)
        hits = np.nonzero(np.asarray(cand[t]) == int(path[t]))[0]
        if hits.size != 1:
            raise ValueError(f"drafted token at {t} is not one of the candidates")
        ratio = p[int(path[t])] / q[t, hits[0]]
        u = accept_uniform(seed, b, t)
        margin = min(margin, abs(u - ratio))
        if u < ratio:
            continue
        w = p.copy()
        w[np.asarray(cand[t])] = np.maximum(0.0, p[np.asarray(cand[t])] - q[t])
        y, dm = inverse_cdf(w, draw_uniform(seed, b, t))
        return Verdict(t, y, float(margin), dm)
    p = softmax(np.asarray(target[L], np.float64) / temperature)
    y, dm = inverse_cdf(p, draw_uniform(seed, b, L))
    return Verdict(L, y, float(margin), dm)
