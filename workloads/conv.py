"""Seeded inputs of the two-tap dynamic depthwise convolution.

Shapes follow one convolution site of a parallel drafter: x [batch, L, D] (the
sublayer's input at every block position), x_prev [batch, D] (the last verified
token's representation at the same site), base [2, D] and W_c [D/16, 2, D].
Streams are keyed like the selector's inputs (``SeedSequence(base_seed,
spawn_key=(tag, b))``), per sequence for x and x_prev, so any subset of a batch
regenerates bit-identically.  Normals are drawn in fp32 and rounded to bf16 once
for bf16 workloads.

Nothing here computes any part of the convolution.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import Config, config_by_name
from .gen import _rng, _store, _workers

TAG_X, TAG_XPREV, TAG_BASE, TAG_WC = 20, 21, 22, 23


@dataclass
class ConvInputs:
    config: Config
    seq_ids: np.ndarray  # int64 [nseq]
    x: np.ndarray  # [nseq, L, D] (bf16 bits or fp32)
    x_prev: np.ndarray  # [nseq, D]
    base: np.ndarray  # [2, D]
    W_c: np.ndarray  # [D/16, 2, D]

    @property
    def dtype(self) -> str:
        return self.config.dtype


def make_conv(cfg: Config | str, seqs=None, base_std: float = 0.5, corr_std: float = 0.002,
              threads: int | None = None) -> ConvInputs:
    """x, x_prev ~ N(0, hidden_std); base ~ N(0, base_std); W_c ~ N(0, corr_std).

    At the default corr_std the correction c = W_c x has std 0.002 sqrt(D) (0.14 at
    D = 5120), small next to the base kernel, as the post describes it; tests raise
    it to make the correction matter."""
    if isinstance(cfg, str):
        cfg = config_by_name(cfg)
    D, L = cfg.d, cfg.L
    if D % 16:
        raise ValueError("D must be a multiple of 16")
    seq_ids = np.arange(cfg.batch, dtype=np.int64) if seqs is None else np.asarray(seqs, np.int64)
    store_dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    x = np.empty((len(seq_ids), L, D), store_dt)
    xp = np.empty((len(seq_ids), D), store_dt)

    def one(i: int) -> None:
        b = int(seq_ids[i])
        v = _rng(cfg.base_seed, TAG_X, b).standard_normal((L, D), dtype=np.float32)
        v *= np.float32(cfg.hidden_std)
        x[i] = _store(v, cfg.dtype)
        p = _rng(cfg.base_seed, TAG_XPREV, b).standard_normal(D, dtype=np.float32)
        p *= np.float32(cfg.hidden_std)
        xp[i] = _store(p, cfg.dtype)

    n = threads or _workers()
    if n > 1 and len(seq_ids) > 1:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(one, range(len(seq_ids))))
    else:
        for i in range(len(seq_ids)):
            one(i)
    base = _rng(cfg.base_seed, TAG_BASE).standard_normal((2, D), dtype=np.float32) * np.float32(base_std)
    W = _rng(cfg.base_seed, TAG_WC).standard_normal((D // 16, 2, D), dtype=np.float32) * np.float32(corr_std)
    return ConvInputs(cfg, seq_ids, x, xp, _store(base, cfg.dtype), _store(W, cfg.dtype))
