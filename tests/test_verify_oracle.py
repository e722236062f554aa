"""Pins of the verification oracle (CPU): the speculative-sampling theorem and its
special cases, the inverse-CDF draw by definition, the draft probabilities."""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import verify as V

RNG = np.random.default_rng(20260807)


def test_draft_probs_are_softmax_rows_of_the_walk():
    L = 5
    S = RNG.standard_normal((L, 16, 16))
    S[0] = S[0, 0][None, :]
    slots = RNG.integers(0, 16, L)
    for T in (1.0, 0.3, 4.0):
        q = V.draft_probs(S, slots, T)
        prev = 0
        for t in range(L):
            np.testing.assert_allclose(q[t], scipy.special.softmax(S[t, prev] / T), rtol=1e-13)
            prev = slots[t]
        np.testing.assert_allclose(q.sum(1), 1.0, rtol=1e-14)
    q = V.draft_probs(S, slots, 1e-9)  # T -> 0: one-hot on each row's argmax
    np.testing.assert_array_equal(q.argmax(1), [S[t, 0 if t == 0 else slots[t - 1]].argmax() for t in range(L)])
    assert np.allclose(q.max(1), 1.0)


def test_inverse_cdf_by_definition():
    for _ in range(200):
        n = int(RNG.integers(1, 40))
        w = RNG.random(n) * (RNG.random(n) < 0.7)
        if w.sum() == 0:
            w[0] = 1.0
        u = float(RNG.random())
        total = math.fsum(w)
        acc, want = 0.0, None
        for v in range(n):
            acc = math.fsum(w[: v + 1])
            if acc >= u * total and w[v] > 0:
                want = v
                break
        got, margin = V.inverse_cdf(w, u)
        if margin > 1e-12:  # away from an interval edge the two sums agree
            assert got == want
        assert w[got] > 0


def _case(Vsize=24, L=1, seed=0):
    rng = np.random.default_rng(seed)
    cand = np.stack([rng.choice(Vsize, 16, replace=False) for _ in range(L)])
    q = np.stack([scipy.special.softmax(rng.standard_normal(16)) for _ in range(L)])
    target = rng.standard_normal((L + 1, Vsize)) * 1.5
    return cand, q, target


def _chi2_ok(counts, probs):
    keep = probs > 0
    assert counts[~keep].sum() == 0  # nothing drawn where the target has no mass
    exp = probs[keep] * counts.sum()
    stat = ((counts[keep] - exp) ** 2 / exp).sum()
    return scipy.stats.chi2.sf(stat, keep.sum() - 1) > 1e-3


def test_emitted_token_follows_the_target_distribution():
    # Draft x ~ q (drawn here with numpy), verify: the first emitted token (x if
    # accepted, else the draw) must be distributed as p_0, whatever q is; and the
    # acceptance rate must be sum_x min(p(x), q(x)).
    cand, q, target = _case()
    p0 = scipy.special.softmax(target[0])
    N = 30000
    drafts = RNG.choice(16, size=N, p=q[0])
    counts = np.zeros(24)
    accepted = 0
    for s in range(N):
        x = int(cand[0, drafts[s]])
        v = V.verify_block(target, [x], cand, q, 1.0, seed=s, b=3)
        first = x if v.accepted >= 1 else v.token
        accepted += v.accepted >= 1
        counts[first] += 1
    assert _chi2_ok(counts, p0)
    qfull = np.zeros(24)
    qfull[cand[0]] = q[0]
    rate = np.minimum(p0, qfull).sum()
    assert abs(accepted / N - rate) < 4 * math.sqrt(rate * (1 - rate) / N)


def test_target_equal_to_draft_accepts_everything_and_bonus_follows_target():
    L = 3
    cand, q, _ = _case(L=L, seed=7)
    target = np.full((L + 1, 24), -np.inf)
    for t in range(L):
        target[t, cand[t]] = np.log(q[t])  # p_t == q_t, zero elsewhere
    target[L] = RNG.standard_normal(24)
    pL = scipy.special.softmax(target[L])
    counts = np.zeros(24)
    for s in range(4000):
        path = [int(cand[t, RNG.choice(16, p=q[t])]) for t in range(L)]
        v = V.verify_block(target, path, cand, q, 1.0, seed=s, b=0)
        assert v.accepted == L
        counts[v.token] += 1
    assert _chi2_ok(counts, pL)


def test_target_mass_off_the_candidates_rejects_at_once():
    cand, q, target = _case(seed=11)
    target[0, cand[0]] = -np.inf  # the target never wants a candidate
    p0 = scipy.special.softmax(target[0])
    counts = np.zeros(24)
    for s in range(4000):
        v = V.verify_block(target, [int(cand[0, 0])], cand, q, 1.0, seed=s, b=1)
        assert v.accepted == 0
        assert v.token not in cand[0]
        counts[v.token] += 1
    assert _chi2_ok(counts, p0)


def test_verdicts_are_deterministic_per_seed_and_block():
    cand, q, target = _case(L=2, seed=5)
    path = [int(cand[0, 0]), int(cand[1, 3])]
    a = V.verify_block(target, path, cand, q, 0.8, seed=99, b=4)
    assert a == V.verify_block(target, path, cand, q, 0.8, seed=99, b=4)
    with pytest.raises(ValueError):
        V.verify_block(target, [999, 0], cand, q, 1.0, seed=1, b=0)
