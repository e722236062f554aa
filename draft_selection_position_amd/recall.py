"""Recall and acceptance of draft paths against known true tokens (synthetic harness).

The post measures how often DFlash's right token sits in its own top-16 list, per
draft position and conditioned on every earlier position being right (blog post
"DFlash 2: Keep Drafting Parallel", section "The Right Tokens Are Already There",
Table 1), and the acceptance length an oracle selector would reach by always
picking the right candidate when it is in the list.  With seeded inputs whose
true token per position is known (the tiny workload plants one), the same
quantities can be read off this library's outputs:

  recall_at(cand, true, k)   per position t: among blocks whose earlier positions
                             are all right (true token in the top-k there), the
                             fraction whose true token is in the top-k at t
  acceptance(path, true)     mean over blocks of the number of leading positions
                             the path gets right, plus the verifier's own token
  oracle_acceptance(cand, true)  the same for a selector that takes the true token
                             whenever it is among the 16 candidates

These are host-side reductions over small int32 outputs ([B, L, 16] candidates,
[B, L] paths); everything on the device is the library's own kernels.
``python -m draft_selection_position_amd.recall --batch 2048`` runs the harness.
"""
from __future__ import annotations

import numpy as np


def _np(x):
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x)


def recall_at(cand, true, k: int = 16):
    """(recall [L] float64, eligible [L] int64): conditional recall@k per position.

    cand [B, L, >=k] candidate ids in rank order, true [B, L] ids.  A position with
    no eligible block has recall NaN."""
    cand, true = _np(cand), _np(true)
    hit = (cand[:, :, :k] == true[:, :, None]).any(axis=2)  # [B, L]
    prefix_ok = np.ones(hit.shape[0], bool)
    rec = np.full(hit.shape[1], np.nan)
    elig = np.zeros(hit.shape[1], np.int64)
    for t in range(hit.shape[1]):
        elig[t] = int(prefix_ok.sum())
        if elig[t]:
            rec[t] = hit[prefix_ok, t].mean()
        prefix_ok &= hit[:, t]
    return rec, elig


def _leading(ok):
    # number of leading True per row
    return np.where(ok.all(axis=1), ok.shape[1], np.argmin(ok, axis=1))


def acceptance(path, true) -> float:
    """Mean accepted length of draft paths [B, L]: leading matches plus one."""
    path, true = _np(path), _np(true)
    return float(np.mean(_leading(path == true) + 1))


def oracle_acceptance(cand, true) -> float:
    """Mean accepted length of a selector that picks the true token whenever it is
    among the 16 candidates of each position."""
    cand, true = _np(cand), _np(true)
    return float(np.mean(_leading((cand == true[:, :, None]).any(axis=2)) + 1))


def main(argv=None) -> int:
    import argparse
    import json

    import torch

    import draft_selection_position_amd as dfs
    from workloads import make, variant

    ap = argparse.ArgumentParser(description="recall / acceptance harness on the tiny workload's planted tokens")
    ap.add_argument("--batch", type=int, default=2048)
    ap.add_argument("--L", type=int, default=8)
    args = ap.parse_args(argv)
    cfg = variant("tiny", batch=args.batch, L=args.L)
    inp = make(cfg)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in
           (("logits", inp.logits), ("hidden", inp.hidden), ("A", inp.A), ("B", inp.B), ("W_h", inp.W_h))}
    dev["prev_token"] = torch.from_numpy(inp.prev_token.astype(np.int32)).cuda()
    idx, _ = dfs.topk(dev["logits"])
    out = {"workload": cfg.name, "blocks": cfg.batch, "L": cfg.L}
    for k in (1, 16):
        r, e = recall_at(idx, inp.true_tokens, k)
        out[f"recall@{k}"] = [round(float(x), 4) for x in r]
        out[f"eligible@{k}"] = e.tolist()
    out["acceptance_top1"] = acceptance(idx[:, :, 0], inp.true_tokens)
    out["acceptance_oracle_top16"] = oracle_acceptance(idx, inp.true_tokens)
    for mode in ("greedy", "viterbi"):
        path, _ = dfs.select(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], dev["W_h"],
                             mode=mode)
        out[f"acceptance_{mode}"] = acceptance(path, inp.true_tokens)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
