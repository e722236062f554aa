"""Helpers of the GPU parity tests: upload seeded inputs, compare with the oracle.

Bars (scores are fp32 on the GPU from bf16/fp32 inputs, fp64 in the oracle):
  * top-16 ids and values: bit-exact (integer keys on identical input bits);
  * scores: within 2e-3 relative or 1e-3 absolute;
  * greedy and sampled paths: identical, except at a step whose oracle best-minus-
    second margin is below 1e-4 (a near tie).  From the first such step on, each
    GPU step must instead be the oracle's best choice (within 1e-4) given the GPU's
    own predecessor ("conditional parity").
"""
from __future__ import annotations

import numpy as np

import oracle
from workloads.device import to_dev, upload  # noqa: F401  (re-exported for the tests)

TOL_ABS = 1e-3
TOL_REL = 2e-3
NEAR_TIE = 1e-4

# (what, workload) -> (units checked, unit name, note); printed at the end of the run
FULL_SIZE: dict = {}


def record(what: str, workload: str, checked: int, unit: str, note: str = "all exact") -> None:
    FULL_SIZE[(what, workload)] = (int(checked), unit, note)


def scores_ok(gpu, ref) -> np.ndarray:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    return (err <= TOL_ABS) | (err <= TOL_REL * np.abs(ref))


def assert_scores(gpu, ref, what="scores"):
    ok = scores_ok(gpu, ref)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        g = np.asarray(gpu, np.float64)
        r = np.asarray(ref, np.float64)
        raise AssertionError(f"{what}: {int((~ok).sum())} outside tolerance; first "
                             + ", ".join(f"{tuple(i)}: gpu {g[tuple(i)]:.7g} oracle {r[tuple(i)]:.7g}" for i in bad))


def check_path(gpu_path, gpu_scores, res: "oracle.SequenceResult", mode="greedy", temperature=1.0, seed=0,
               b=0) -> dict:
    """Compare one sequence's GPU walk with the oracle's; returns a small report."""
    if mode == "viterbi":
        return check_best_path(gpu_path, gpu_scores, res, b)
    L = res.path.shape[0]
    near_ties = []
    conditional = False
    i_prev = 0
    for t in range(L):
        hits = np.nonzero(res.cand_idx[t] == int(gpu_path[t]))[0]
        if hits.size != 1:
            raise AssertionError(f"seq {b} step {t}: GPU token {int(gpu_path[t])} is not a candidate")
        j = int(hits[0])
        if not conditional and int(gpu_path[t]) != int(res.path[t]):
            if res.margins[t] < NEAR_TIE:
                near_ties.append(t)
                conditional = True
            else:
                raise AssertionError(f"seq {b} step {t}: GPU took {int(gpu_path[t])}, oracle "
                                     f"{int(res.path[t])} (margin {res.margins[t]:.3g})")
        row = res.pair[t, i_prev]
        if conditional:
            key = row.copy()
            if mode == "gumbel":
                key = row / temperature + np.array([oracle.gumbel(seed, b, t, jj) for jj in range(16)])
            if key[j] < key.max() - NEAR_TIE:
                raise AssertionError(f"seq {b} step {t}: conditional parity broken ({key.max() - key[j]:.3g})")
        if not scores_ok(gpu_scores[t], row[j]):
            raise AssertionError(f"seq {b} step {t}: score {float(gpu_scores[t])!r} vs oracle {row[j]!r}")
        i_prev = j
    return {"near_ties": near_ties, "exact": not near_ties}


def check_best_path(gpu_path, gpu_scores, res: "oracle.SequenceResult", b=0) -> dict:
    """The GPU's best-total path against the oracle's (Viterbi): the same slots when the
    oracle's optimum leads every other path by NEAR_TIE or more (its smallest decision gap);
    otherwise the GPU path must total, on the oracle's fp64 scores, within NEAR_TIE of the
    optimum.  Per-step scores within the score tolerance either way."""
    L = res.path.shape[0]
    slots, i_prev, total = [], 0, 0.0
    for t in range(L):
        hits = np.nonzero(res.cand_idx[t] == int(gpu_path[t]))[0]
        if hits.size != 1:
            raise AssertionError(f"seq {b} step {t}: GPU token {int(gpu_path[t])} is not a candidate")
        j = int(hits[0])
        s_ref = res.pair[t, i_prev, j]
        if not scores_ok(gpu_scores[t], s_ref):
            raise AssertionError(f"seq {b} step {t}: score {float(gpu_scores[t])!r} vs oracle {s_ref!r}")
        total += s_ref
        slots.append(j)
        i_prev = j
    best = float(np.sum(res.scores))
    if res.margins.min() >= NEAR_TIE:
        if not np.array_equal(np.asarray(slots), res.slots):
            raise AssertionError(f"seq {b}: GPU best path {slots} != oracle {res.slots.tolist()} "
                                 f"(oracle margin {res.margins.min():.3g})")
        return {"near_ties": [], "exact": True}
    if total < best - NEAR_TIE:
        raise AssertionError(f"seq {b}: GPU path totals {total!r}, optimum {best!r}")
    return {"near_ties": [] if slots == res.slots.tolist() else [int(np.argmin(res.margins))],
            "exact": slots == res.slots.tolist()}
