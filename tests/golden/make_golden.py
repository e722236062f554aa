"""Writes tests/golden/*.json from the CPU oracle only (run: python tests/golden/make_golden.py).

The pages print no worked numeric example of the selector, so the stored values
here are the oracle's own output on small seeded workloads.  They freeze the
oracle: a later change of its arithmetic must regenerate them, and the commit
that does so names the passage of "DFlash 2: Keep Drafting Parallel" (or the
reading of it) that justifies the change.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import make, variant  # noqa: E402

CASES = {
    "tiny_greedy": variant("tiny", V=700, d=96, L=5, batch=2),
    "amplified_greedy": variant("small_batch", V=900, d=64, L=6, batch=2, emb_std=0.3),
    "sampled_gumbel": variant("sampled", V=800, d=64, L=6, batch=2, emb_std=0.3),
}


def main():
    for name, cfg in CASES.items():
        inp = make(cfg)
        out = []
        for r in oracle.select(inp):
            out.append({
                "cand_idx": r.cand_idx.tolist(),
                "cand_val": r.cand_val.tolist(),
                "path": r.path.tolist(),
                "scores": [float(s) for s in r.scores],
                "slots": r.slots.tolist(),
            })
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump({"config": cfg.name, "sequences": out}, f)
        print("wrote", name)


if __name__ == "__main__":
    main()
