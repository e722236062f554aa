"""Seeded generators for the selector's inputs.

Every tensor has its own counter-keyed numpy stream
``SeedSequence(base_seed, spawn_key=(tag, b))``: per-sequence tensors (logits,
hidden states, the last verified token) are keyed by the global sequence index
``b``, so any subset of sequences can be regenerated bit-identically without
generating the rest of the batch.  Normals are drawn in fp32 and, for bf16
workloads, rounded to bf16 once (round to nearest, ties to even); the bf16 bit
patterns are the input that every consumer sees.

Nothing here computes any part of the selector.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import E, Config, config_by_name

TAG_LOGITS, TAG_PEAKS, TAG_HIDDEN, TAG_PREV, TAG_A, TAG_B, TAG_WH = range(7)


def _rng(base_seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(base_seed, spawn_key=key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the 16-bit patterns.

    Inputs must be finite or +-inf (no NaN), which is all the generators produce.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = u >> 16
    lsb &= 1
    u += lsb
    u += 0x7FFF
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """One batch of selector inputs, as host arrays.

    Float tensors are ``np.uint16`` bf16 bit patterns when ``dtype == "bf16"``
    and ``np.float32`` when ``dtype == "f32"``.
    """

    config: Config
    seq_ids: np.ndarray  # int64 [nseq]: global sequence index of each row of the batch
    logits: np.ndarray  # [nseq, L, V]
    hidden: np.ndarray  # [nseq, L, d]
    prev_token: np.ndarray  # int32 [nseq]
    A: np.ndarray  # [V, 256]
    B: np.ndarray  # [V, 256]
    W_h: np.ndarray  # [d, 256]
    true_tokens: np.ndarray | None = None  # int32 [nseq, L] for "true_token" workloads

    @property
    def dtype(self) -> str:
        return self.config.dtype

    @property
    def nseq(self) -> int:
        return int(self.seq_ids.shape[0])

    @property
    def walk(self) -> str:
        return self.config.walk

    @property
    def temperature(self) -> float:
        return self.config.temperature

    @property
    def walk_seed(self) -> int:
        return self.config.walk_seed

    def subset(self, idx) -> "Inputs":
        """Rows ``idx`` of this batch (tables shared, not copied)."""
        idx = np.asarray(idx, dtype=np.int64)
        return Inputs(
            self.config, self.seq_ids[idx], self.logits[idx], self.hidden[idx],
            self.prev_token[idx], self.A, self.B, self.W_h,
            None if self.true_tokens is None else self.true_tokens[idx],
        )


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _sequence_logits(cfg: Config, b: int) -> tuple[np.ndarray, np.ndarray | None]:
    L, V = cfg.L, cfg.V
    rng = _rng(cfg.base_seed, TAG_LOGITS, b)
    x = rng.standard_normal((L, V), dtype=np.float32)
    x *= np.float32(cfg.logit_sigma)
    prng = _rng(cfg.base_seed, TAG_PEAKS, b)
    true_tokens = None
    if cfg.peak_kind == "true_token":
        true_tokens = prng.integers(0, V, size=L, dtype=np.int64).astype(np.int32)
        x[np.arange(L), true_tokens] += np.float32(cfg.peak_margin)
    elif cfg.peak_kind in ("zipf", "zipf_decay"):
        r = np.arange(1, 17, dtype=np.float64)
        rank_w = r ** -1.1
        if cfg.zipf_ids:
            p = np.arange(1, V + 1, dtype=np.float64) ** -1.1
            p /= p.sum()
        for t in range(L):
            if cfg.peak_kind == "zipf_decay" and L > 1:
                m = cfg.peak_margin + (cfg.peak_margin_end - cfg.peak_margin) * t / (L - 1)
            else:
                m = cfg.peak_margin
            if cfg.zipf_ids:
                ids = prng.choice(V, size=16, replace=False, p=p)
            else:
                ids = prng.choice(V, size=16, replace=False)
            top = float(x[t].max())
            x[t, ids] = (top + m * rank_w).astype(np.float32)
    elif cfg.peak_kind != "none":
        raise ValueError(f"unknown peak_kind {cfg.peak_kind!r}")
    if cfg.tie_levels > 0:
        step = np.float32(8.0 * cfg.logit_sigma / cfg.tie_levels)
        np.round(x / step, out=x)
        x *= step
    if cfg.neg_inf_frac > 0.0:
        qrng = _rng(cfg.base_seed, TAG_PEAKS + 100, b)
        mask = qrng.random((L, V)) < cfg.neg_inf_frac
        x[mask] = -np.inf
    return _store(x, cfg.dtype), true_tokens


def _sequence_hidden(cfg: Config, b: int) -> np.ndarray:
    rng = _rng(cfg.base_seed, TAG_HIDDEN, b)
    h = rng.standard_normal((cfg.L, cfg.d), dtype=np.float32)
    h *= np.float32(cfg.hidden_std)
    return _store(h, cfg.dtype)


def _table(cfg: Config, tag: int, rows: int) -> np.ndarray:
    rng = _rng(cfg.base_seed, tag)
    w = rng.standard_normal((rows, E), dtype=np.float32)
    w *= np.float32(cfg.emb_std)
    return _store(w, cfg.dtype)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make(cfg: Config | str, seqs=None, threads: int | None = None) -> Inputs:
    """Generate the inputs of workload ``cfg`` for sequences ``seqs``.

    ``seqs`` defaults to the whole batch ``range(cfg.batch)``.  Any subset gives
    the same per-sequence data as the full batch.
    """
    if isinstance(cfg, str):
        cfg = config_by_name(cfg)
    seq_ids = np.arange(cfg.batch, dtype=np.int64) if seqs is None else np.asarray(seqs, np.int64)
    if seq_ids.ndim != 1 or (seq_ids.size and (seq_ids.min() < 0 or seq_ids.max() >= cfg.batch)):
        raise ValueError("seqs must be sequence indices in [0, batch)")
    nseq = seq_ids.shape[0]
    store_dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    logits = np.empty((nseq, cfg.L, cfg.V), dtype=store_dt)
    hidden = np.empty((nseq, cfg.L, cfg.d), dtype=store_dt)
    true_tokens = np.empty((nseq, cfg.L), np.int32) if cfg.peak_kind == "true_token" else None

    def one(i: int) -> None:
        b = int(seq_ids[i])
        logits[i], tt = _sequence_logits(cfg, b)
        if true_tokens is not None:
            true_tokens[i] = tt
        hidden[i] = _sequence_hidden(cfg, b)

    nthreads = threads or _workers()
    if nthreads > 1 and nseq > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(nseq)))
    else:
        for i in range(nseq):
            one(i)
    prev = np.array(
        [_rng(cfg.base_seed, TAG_PREV, int(b)).integers(0, cfg.V) for b in seq_ids], dtype=np.int32
    )
    A = _table(cfg, TAG_A, cfg.V)
    B = _table(cfg, TAG_B, cfg.V)
    W_h = _table(cfg, TAG_WH, cfg.d)
    return Inputs(cfg, seq_ids, logits, hidden, prev, A, B, W_h, true_tokens)
