"""The five drafter-shaped workloads, plus test-only variants.

Shapes follow a parallel drafter's output for one draft block: ``batch``
sequences, ``L`` block positions, vocabulary ``V``, hidden width ``d``; k = 16
candidates and a 256-wide embedding everywhere.  Block lengths 8 and 16 are the
ones the DFlash 2 post uses for its released drafters (DFlash 2: Keep Drafting
Parallel, twiscan.com translation, captions of Tables 4 and 5).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

K = 16
E = 256


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    L: int
    V: int
    d: int
    dtype: str  # "f32" or "bf16": dtype of every float tensor of the workload
    logit_sigma: float
    # "true_token": one seeded token per position gets +peak_margin (literal reading);
    # "zipf": 16 planted ids per position at background max + m * r^-1.1, r = 1..16;
    # "zipf_decay": as "zipf" with m_t falling linearly from peak_margin to peak_margin_end;
    # "none": background only.
    peak_kind: str
    peak_margin: float
    peak_margin_end: float = 0.0
    emb_std: float = 0.02  # std of A, B and W_h
    hidden_std: float = 1.0
    walk: str = "greedy"  # "greedy", "gumbel" or "viterbi"
    temperature: float = 1.0
    walk_seed: int = 0
    base_seed: int = 0xDF50
    # test-only data shapes
    tie_levels: int = 0  # >0: logits quantised to this many levels (tie stress)
    neg_inf_frac: float = 0.0  # fraction of each row set to -inf
    zipf_ids: bool = False  # planted ids drawn with p(id) ~ (id+1)^-1.1 instead of uniform


CONFIGS = [
    Config("tiny", 1, 8, 32000, 1024, "f32", 1.0, "true_token", 4.0, base_seed=0xDF50 + 0),
    Config("single_stream", 1, 16, 151936, 5120, "bf16", 1.5, "zipf", 4.0, base_seed=0xDF50 + 1),
    Config("small_batch", 32, 16, 151936, 5120, "bf16", 1.5, "zipf", 4.0, base_seed=0xDF50 + 2),
    Config("throughput", 256, 16, 151936, 5120, "bf16", 1.5, "zipf_decay", 4.0, 1.5,
           base_seed=0xDF50 + 3),
    Config("sampled", 64, 16, 262144, 4096, "bf16", 2.0, "zipf", 4.0, walk="gumbel",
           temperature=1.0, walk_seed=0x5EED, base_seed=0xDF50 + 4),
]


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown workload {name!r}; known: {[c.name for c in CONFIGS]}")


def variant(base: Config | str, **changes) -> Config:
    """A copy of ``base`` with some fields changed (test-only variants)."""
    if isinstance(base, str):
        base = config_by_name(base)
    if "name" not in changes:
        changes["name"] = base.name + "+" + ",".join(f"{k}={v}" for k, v in sorted(changes.items()))
    return dataclasses.replace(base, **changes)
