"""The DFlash 2 path selector, step by step, in fp64.  TEST INFRASTRUCTURE ONLY.

Sources (the blog post "DFlash 2: Keep Drafting Parallel", Inco AI, August 2026):
  * wpnews.pro copy, section "The Right Tokens Are Already There": DFlash's own
    top-16 candidate list per position almost always holds the right token.
  * wpnews.pro copy, section "A Lightweight Path Selector", and the twiscan.com
    Chinese translation of the same section, which keeps the score equation
        S_t(a, b) = U_t(b) + < A(a) (elementwise) H(h_t), B(b) >
    with U_t(b) the drafter's own logit for candidate b at position t, A and B
    256-wide token embeddings and H(h_t) a context gate.  All adjacent pairs are
    scored at once; the only sequential part is one walk over the scores that
    starts at the last verified token and, greedily, takes the best successor at
    each step (sampling draws from the same scores).  No extra backbone or LM-head
    pass is made.

Readings of points the pages leave open (kept identical in the HIP library):
  * H(h_t) = sigmoid(h_t W_h) with W_h of shape [d, 256]; A, B are [V, 256] tables.
  * U_t(b) is the raw logit; h_t is the hidden state of the candidate's position t.
  * Top-16 order: value descending, ties to the lower token id; -0 equals +0.
  * Position 0's predecessor is the last verified token; its single score row is
    repeated over the 16 predecessor slots of the [L, 16, 16] tensor.
  * Greedy takes the lowest slot among equal scores.  Sampling is Gumbel-max:
    argmax_j S/T + g(seed, b, t, j) in fp64 (see philox.py).
  * Reported score of step t is the un-noised S_t(path[t-1], path[t]).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import gumbel

K = 16  # candidates kept per position
E = 256  # embedding / gate width


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exactly widen stored values to fp64: bf16 bit patterns (uint16) or fp32."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def top16(row: np.ndarray, k: int = K) -> tuple[np.ndarray, np.ndarray]:
    """The k largest entries of one row of logits, by a full stable sort.

    DFlash 2 keeps the 16 best candidates of each block position instead of only
    the top one (wpnews.pro, "The Right Tokens Are Already There").  Order: value
    descending, then token id ascending; -0 and +0 are the same value.
    Returns (ids int64 [k], values fp64 [k]).
    """
    v = np.asarray(row, dtype=np.float64)
    if v.ndim != 1 or v.shape[0] < k:
        raise ValueError("top16 needs a 1-D row with at least k entries")
    if np.isnan(v).any():
        raise ValueError("NaN logits are outside the selector's contract")
    v = v + 0.0  # -0 -> +0
    ids = np.arange(v.shape[0])
    order = np.lexsort((ids, -v))  # primary key -v, secondary key id
    top = order[:k]
    return top.astype(np.int64), v[top]


def top16_rows(rows: np.ndarray, k: int = K) -> tuple[np.ndarray, np.ndarray]:
    """``top16`` applied to every row of a [R, V] fp64 array."""
    rows = np.asarray(rows, dtype=np.float64)
    ids = np.empty((rows.shape[0], k), np.int64)
    vals = np.empty((rows.shape[0], k), np.float64)
    for r in range(rows.shape[0]):
        ids[r], vals[r] = top16(rows[r], k)
    return ids, vals


def gate(h: np.ndarray, W_h: np.ndarray) -> np.ndarray:
    """Context gate H(h_t) = sigmoid(h_t W_h), fp64; h is [..., d], W_h is [d, 256].

    The pages name a gate computed from the drafter's hidden state that weights
    the embedding match (wpnews.pro, "A Lightweight Path Selector"); the sigmoid
    of a linear map is this implementation's parameterisation of it.
    """
    z = np.asarray(h, np.float64) @ np.asarray(W_h, np.float64)
    with np.errstate(over="ignore"):  # exp(-z) = inf gives the exact limit 0
        return 1.0 / (1.0 + np.exp(-z))


def pair_scores(cand_idx: np.ndarray, cand_val: np.ndarray, prev_token: int, g: np.ndarray,
                A_rows, B_rows) -> np.ndarray:
    """All adjacent-pair scores of one sequence: S[t, i, j], fp64 [L, 16, 16].

    S_t(a, b) = U_t(b) + sum_e A[a, e] * g_t[e] * B[b, e]   (twiscan.com
    translation, score equation of the path-selector section).  For t >= 1 the
    predecessor a runs over the 16 candidates of position t-1 (slot i) and b over
    the 16 candidates of position t (slot j); for t = 0 the predecessor is the
    last verified token and the one row is repeated over i.

    ``A_rows(ids)`` / ``B_rows(ids)`` return the fp64 embedding rows of token ids.
    """
    cand_idx = np.asarray(cand_idx)
    U = np.asarray(cand_val, np.float64)
    L = cand_idx.shape[0]
    S = np.empty((L, K, K), np.float64)
    for t in range(L):
        Bt = B_rows(cand_idx[t])  # [16, 256], candidate b = slot j
        if t == 0:
            a = A_rows(np.array([prev_token]))  # [1, 256]
        else:
            a = A_rows(cand_idx[t - 1])  # [16, 256], predecessor a = slot i
        bil = (a * g[t][None, :]) @ Bt.T  # [1 or 16, 16]
        S[t] = U[t][None, :] + bil
    return S


def walk(S: np.ndarray, cand_idx: np.ndarray, mode: str = "greedy", temperature: float = 1.0,
         seed: int = 0, b: int = 0):
    """One walk over precomputed scores, from the last verified token.

    Greedy: at each step take the best successor of the previous pick (lowest
    slot on ties).  Viterbi: the path of largest total score (see ``viterbi``).  Gumbel: take argmax_j S/T + g(seed, b, t, j), which draws the
    successor from softmax(S/T) over the 16 candidates (wpnews.pro, "A Lightweight
    Path Selector": sampling uses the same scores).
    Returns (path int64 [L], scores fp64 [L], slots int64 [L], margins fp64 [L]);
    margins[t] is best minus second best of the (noised) row used at step t.
    """
    if mode == "viterbi":
        return viterbi(S, cand_idx)
    L = S.shape[0]
    path = np.empty(L, np.int64)
    scores = np.empty(L, np.float64)
    slots = np.empty(L, np.int64)
    margins = np.empty(L, np.float64)
    i = 0  # predecessor slot; row 0 of S_0 is the last verified token's row
    for t in range(L):
        row = S[t, i]
        if mode == "greedy":
            key = row
        elif mode == "gumbel":
            if not temperature > 0.0:
                raise ValueError("sampled walk needs temperature > 0")
            noise = np.array([gumbel(seed, b, t, j) for j in range(K)])
            key = row / temperature + noise
        else:
            raise ValueError(f"unknown walk mode {mode!r}")
        j = int(np.argmax(key))  # first maximum -> lowest slot on ties
        srt = np.sort(key)
        margins[t] = srt[-1] - srt[-2]
        path[t] = cand_idx[t, j]
        scores[t] = row[j]
        slots[t] = j
        i = j
    return path, scores, slots, margins


def viterbi(S: np.ndarray, cand_idx: np.ndarray):
    """The path whose summed pair scores are largest, by dynamic programming.

    The post calls pairwise scoring the simplest selector and leaves better ones
    open (wpnews.pro, "A Lightweight Path Selector"); the greedy walk takes the
    best successor step by step, this takes the best whole path over the same
    [L, 16, 16] scores.  best[0][j] = S_0(prev, j); best[t][j] =
    max_i best[t-1][i] + S_t(i, j), keeping the lowest i among equal values; the
    last slot is the lowest j of largest best[L-1][j]; the path is read back.
    Returns (path, scores, slots, margins) like ``walk``; scores[t] is
    S_t(slot[t-1], slot[t]) and margins holds the gap between the best and the
    second best choice at every decision taken on the way back (final slot, then
    each predecessor), so every other path totals at least min(margins) less.
    """
    L = S.shape[0]
    best = S[0, 0].astype(np.float64).copy()
    back = np.zeros((L, K), np.int64)
    for t in range(1, L):
        cand = best[:, None] + S[t]  # [i, j]: best path to i, then step i -> j
        back[t] = np.argmax(cand, axis=0)  # first maximum -> lowest i
        best = cand[back[t], np.arange(K)]
    slots = np.empty(L, np.int64)
    margins = np.empty(L, np.float64)

    def gap(v):
        srt = np.sort(v)
        return srt[-1] - srt[-2]

    slots[L - 1] = int(np.argmax(best))
    margins[L - 1] = gap(best)
    # recompute the DP tables to read the decision gaps on the way back
    table = [S[0, 0].astype(np.float64).copy()]
    for t in range(1, L):
        table.append((table[-1][:, None] + S[t]).max(axis=0))
    for t in range(L - 1, 0, -1):
        slots[t - 1] = back[t, slots[t]]
        margins[t - 1] = gap(table[t - 1] + S[t][:, slots[t]])
    scores = np.empty(L, np.float64)
    scores[0] = S[0, 0, slots[0]]
    for t in range(1, L):
        scores[t] = S[t, slots[t - 1], slots[t]]
    path = np.array([cand_idx[t, slots[t]] for t in range(L)], np.int64)
    return path, scores, slots, margins


@dataclass
class SequenceResult:
    cand_idx: np.ndarray  # int64 [L, 16]
    cand_val: np.ndarray  # fp64 [L, 16]
    gate: np.ndarray  # fp64 [L, 256]
    pair: np.ndarray  # fp64 [L, 16, 16]
    path: np.ndarray  # int64 [L]
    scores: np.ndarray  # fp64 [L]
    slots: np.ndarray  # int64 [L]
    margins: np.ndarray  # fp64 [L]


def select_sequence(inp, i: int) -> SequenceResult:
    """The whole selector for row ``i`` of a batch ``inp`` (a ``workloads.Inputs``).

    top-16 per position, gate per position, every adjacent pair scored, one walk.
    """
    dt = inp.dtype
    logits = widen(inp.logits[i], dt)  # [L, V]
    cand_idx, cand_val = top16_rows(logits)
    g = gate(widen(inp.hidden[i], dt), widen(inp.W_h, dt))

    def A_rows(ids):
        return widen(inp.A[np.asarray(ids)], dt)

    def B_rows(ids):
        return widen(inp.B[np.asarray(ids)], dt)

    S = pair_scores(cand_idx, cand_val, int(inp.prev_token[i]), g, A_rows, B_rows)
    path, scores, slots, margins = walk(S, cand_idx, inp.walk, inp.temperature, inp.walk_seed,
                                        int(inp.seq_ids[i]))
    return SequenceResult(cand_idx, cand_val, g, S, path, scores, slots, margins)


def select(inp, rows=None) -> list[SequenceResult]:
    """``select_sequence`` for rows ``rows`` of the batch (default: all)."""
    rows = range(inp.nseq) if rows is None else rows
    return [select_sequence(inp, int(i)) for i in rows]
