"""Recall and acceptance against known true tokens, by explicit loops.  TEST INFRASTRUCTURE ONLY.

Source: blog post "DFlash 2: Keep Drafting Parallel", section "The Right Tokens Are
Already There" (Table 1 and its caption): recall@1 and recall@16 per draft
position, each conditioned on every earlier position being right, and the
acceptance length of an oracle selector over the top-16 lists, which counts the
verifier's own next token as well.

Readings: "earlier positions right" means the true token was within the top-k at
each earlier position for recall@k; an accepted length is the number of leading
positions a path gets right, plus one for the verifier's token.
"""
from __future__ import annotations

import math


def recall_at(cands, trues, k):
    """cands: per block, per position, the ranked candidate ids; trues: per block,
    per position, the true id.  Returns (recall per position, eligible blocks per
    position); recall is nan where no block is eligible."""
    L = len(trues[0])
    eligible = [0] * L
    hits = [0] * L
    for cand, true in zip(cands, trues):
        for t in range(L):
            eligible[t] += 1
            if true[t] in list(cand[t][:k]):
                hits[t] += 1
            else:
                break
    return [h / e if e else math.nan for h, e in zip(hits, eligible)], eligible


def accepted_length(path, true):
    """Leading positions where path equals the true tokens, plus one."""
    n = 0
    for p, tt in zip(path, true):
        if p != tt:
            break
        n += 1
    return n + 1


def mean_acceptance(paths, trues):
    return sum(accepted_length(p, t) for p, t in zip(paths, trues)) / len(paths)


def oracle_selector_paths(cands, trues):
    """The path an oracle selector drafts: the true token while it is among the
    candidates, then (the block is rejected there anyway) the top candidate."""
    paths = []
    for cand, true in zip(cands, trues):
        path, ok = [], True
        for t in range(len(true)):
            ok = ok and true[t] in list(cand[t])
            path.append(true[t] if ok else cand[t][0])
        paths.append(path)
    return paths
