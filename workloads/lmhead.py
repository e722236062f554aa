"""Seeded LM-head weights for computing the top-16 straight from hidden states.

The hidden states are the selector workload's own (``gen.make``: h_t ~ N(0, 1) per
sequence), so the fused path and the selector see the same drafter outputs.  The
head W_lm [V, d] ~ N(0, std) is drawn in row blocks, each block from its own stream
``SeedSequence(base_seed, spawn_key=(TAG_WLM, block))``, in parallel; normals in
fp32, rounded to bf16 once.  With std = 0.02 and h ~ N(0, 1) the logits have std
0.02 sqrt(d) (1.43 at d = 5120), the scale of the workloads' logits.

Nothing here computes any part of the selector.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config, config_by_name
from .gen import _rng, _sequence_hidden, _store, _workers

TAG_WLM = 30
BLOCK_ROWS = 4096


def make_lm_head(cfg: Config | str, std: float = 0.02, V: int | None = None,
                 threads: int | None = None) -> np.ndarray:
    """W_lm [V, d] (bf16 bits or fp32 by the workload's dtype)."""
    if isinstance(cfg, str):
        cfg = config_by_name(cfg)
    V = cfg.V if V is None else V
    d = cfg.d
    out = np.empty((V, d), np.uint16 if cfg.dtype == "bf16" else np.float32)

    def block(i: int) -> None:
        r0 = i * BLOCK_ROWS
        r1 = min(V, r0 + BLOCK_ROWS)
        w = _rng(cfg.base_seed, TAG_WLM, i).standard_normal((r1 - r0, d), dtype=np.float32)
        w *= np.float32(std)
        out[r0:r1] = _store(w, cfg.dtype)

    nb = -(-V // BLOCK_ROWS)
    n = threads or _workers()
    if n > 1 and nb > 1:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(block, range(nb)))
    else:
        for i in range(nb):
            block(i)
    return out


def make_hidden(cfg: Config | str, seqs=None) -> np.ndarray:
    """The workload's hidden states h [nseq, L, d] alone (identical to ``gen.make``'s)."""
    if isinstance(cfg, str):
        cfg = config_by_name(cfg)
    seqs = range(cfg.batch) if seqs is None else [int(b) for b in seqs]
    seqs = list(seqs)
    out = np.empty((len(seqs), cfg.L, cfg.d), np.uint16 if cfg.dtype == "bf16" else np.float32)

    def one(i: int) -> None:
        out[i] = _sequence_hidden(cfg, seqs[i])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(seqs))))
    return out
