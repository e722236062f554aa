"""The oracle over whole workloads, fanned out over worker processes.

Test infrastructure: it runs the CPU oracle (oracle/) only.  Workers are started fresh
("spawn": a new interpreter, nothing inherited), never forked, so a test process that
already uses the GPU may start them; each regenerates its own sequences from the seeded
generators (per-sequence streams, so any subset of a batch is bit-identical to the whole)
and runs single-threaded.  `Background` starts the work for whole workloads at once and
lets the GPU tests collect it when they need it, so the oracle runs beside them.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle


def _worker(args):
    cfg, seqs = args
    from threadpoolctl import threadpool_limits

    from workloads import make

    with threadpool_limits(1):
        inp = make(cfg, seqs=seqs, threads=1)
        return [(int(s), oracle.select_sequence(inp, j)) for j, s in enumerate(seqs)]


def workers_for(n: int) -> int:
    """Worker processes for n sequences: one per core this process may use, at most 16 (a
    one-GPU machine's share of its host) and at most n."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(16, cores, n))


def _chunks(seqs, w):
    return [seqs[i::w] for i in range(w) if seqs[i::w]]


def oracle_all(cfg, seqs=None) -> dict:
    """{sequence index: oracle.SequenceResult} for sequences `seqs` (default: the whole
    batch) of workload config `cfg` (a workloads.Config)."""
    seqs = list(range(cfg.batch)) if seqs is None else [int(s) for s in seqs]
    w = workers_for(len(seqs))
    if w == 1:
        return dict(_worker((cfg, seqs)))
    chunks = _chunks(seqs, w)
    with mp.get_context("spawn").Pool(len(chunks)) as pool:
        parts = pool.map(_worker, [(cfg, c) for c in chunks])
    out = {}
    for p in parts:
        out.update(p)
    return out


class Background:
    """Whole-batch oracle results for several workloads, computed by one worker pool in the
    background; `get(name)` waits for that workload's results."""

    def __init__(self, cfgs, workers=None):
        total = sum(c.batch for c in cfgs)
        self.workers = workers or workers_for(total)
        self._pool = mp.get_context("spawn").Pool(self.workers)
        self._pending = {}
        self._done = {}
        for cfg in cfgs:
            # one chunk per worker and workload: each chunk pays for the workload's tables once
            chunks = _chunks(list(range(cfg.batch)), min(self.workers, cfg.batch))
            self._pending[cfg.name] = [self._pool.apply_async(_worker, ((cfg, c),)) for c in chunks]

    def names(self):
        return set(self._pending) | set(self._done)

    def get(self, name: str, timeout: float = 900.0) -> dict:
        if name not in self._done:
            out = {}
            for a in self._pending.pop(name):
                out.update(a.get(timeout))
            self._done[name] = out
        return self._done[name]

    def close(self):
        self._pool.terminate()
        self._pool.join()


def stack(results: dict, field: str) -> np.ndarray:
    """One field of every sequence's result, stacked in sequence order."""
    return np.stack([getattr(results[s], field) for s in sorted(results)])
