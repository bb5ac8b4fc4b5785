"""Distribution preservation of the sampled acceptance rule, and the sampler behind it.

The rule (Leviathan et al., Def. 3.7 / Thm. 3.8, cited by the strata2signal page)
must emit sequences with exactly the target's autoregressive probabilities; the
spec pin is exact enumeration on an 8-token vocabulary to within 1e-12.
"""
import time

import numpy as np
import pytest
from scipy.stats import chi2 as chi2d

from oracle.accept import accept_sampled, one_position_output, rule_outcomes
from oracle.enumerate_rule import ToyLM, autoregressive_distribution, chained_distribution


@pytest.mark.parametrize("k,n", [(2, 4), (3, 3)])
def test_enumeration_reproduces_target(k, n):
    V = 8
    p_lm = ToyLM(V, seed=11, scale=1.5)
    q_lm = ToyLM(V, seed=23, scale=2.0)
    base = (5,)
    got = chained_distribution(p_lm, q_lm, base, k, n)
    want = autoregressive_distribution(p_lm, base, n)
    assert abs(sum(got.values()) - 1.0) < 1e-12
    err = max(abs(got.get(y, 0.0) - w) for y, w in want.items())
    assert err <= 1e-12, err
    assert set(got) <= set(want)


def test_enumeration_k3_n4():
    t = time.time()
    V = 8
    p_lm = ToyLM(V, seed=5, scale=1.0)
    q_lm = ToyLM(V, seed=6, scale=2.5)
    got = chained_distribution(p_lm, q_lm, (1, 2), 3, 4)
    want = autoregressive_distribution(p_lm, (1, 2), 4)
    assert max(abs(got.get(y, 0.0) - w) for y, w in want.items()) <= 1e-12
    assert time.time() - t < 120


def test_enumeration_detects_a_wrong_rule():
    # a plausible mistake (residual drawn from p instead of max(0, p - q)) must break the pin
    import oracle.accept as acc
    orig = acc.rule_outcomes

    def wrong(p_rows, q_rows, drafts):
        k = len(drafts)
        out, reach = {}, 1.0
        for i in range(1, k + 1):
            p, q, d = np.asarray(p_rows[i - 1]), np.asarray(q_rows[i - 1]), int(drafts[i - 1])
            keep = min(1.0, p[d] / q[d])
            for x in range(p.size):
                key = tuple(drafts[: i - 1]) + (x,)
                out[key] = out.get(key, 0.0) + reach * (1 - keep) * p[x]
            reach *= keep
        for x in range(len(p_rows[k])):
            key = tuple(drafts) + (x,)
            out[key] = out.get(key, 0.0) + reach * p_rows[k][x]
        return out

    import oracle.enumerate_rule as en
    en.rule_outcomes = wrong
    try:
        p_lm, q_lm = ToyLM(8, 11, 1.5), ToyLM(8, 23, 2.0)
        got = chained_distribution(p_lm, q_lm, (5,), 2, 2)
        want = autoregressive_distribution(p_lm, (5,), 2)
        assert max(abs(got.get(y, 0.0) - w) for y, w in want.items()) > 1e-4
    finally:
        en.rule_outcomes = orig


def test_one_position_identity():
    rng = np.random.default_rng(3)
    for _ in range(100):
        V = int(rng.integers(2, 20))
        p = rng.dirichlet(np.ones(V) * 0.5)
        q = rng.dirichlet(np.ones(V) * 0.5)
        assert np.max(np.abs(one_position_output(p, q) - p)) < 1e-14


def test_rule_identical_drafter_always_accepts():
    rng = np.random.default_rng(4)
    V, k = 8, 3
    p_rows = [rng.dirichlet(np.ones(V)) for _ in range(k + 1)]
    drafts = [1, 2, 3]
    out = rule_outcomes(p_rows, p_rows[:k], drafts)
    # q == p at every draft: every draft is kept, the bonus follows p_k
    assert all(len(y) == k + 1 and y[:k] == tuple(drafts) for y in out)
    assert abs(sum(out.values()) - 1) < 1e-15


def test_sampler_follows_rule():
    """Philox-driven sampler vs the exact rule on one round (V=8, k=2): chi-square over outcomes."""
    V, k, n = 8, 2, 30_000
    rng = np.random.default_rng(9)
    zrows = (rng.standard_normal((k + 1, V)) * 1.5).astype(np.float32)
    T = 0.7
    p_rows = []
    for j in range(k + 1):
        zz = zrows[j].astype(np.float64) / T
        e = np.exp(zz - zz.max())
        p_rows.append(e / e.sum())
    q_rows = [rng.dirichlet(np.ones(V)).astype(np.float32) for _ in range(k)]
    drafts = [int(np.argmax(q_rows[0])), int(np.argmax(q_rows[1]))]
    exact = rule_outcomes(p_rows, [q.astype(np.float64) for q in q_rows], drafts)
    counts = {}
    for lane in range(n):
        c, em = accept_sampled(zrows, drafts, q_rows, T, seed=77, lane=lane, kv_len=100)
        assert 1 <= c <= k + 1 and len(em) == c
        counts[tuple(em)] = counts.get(tuple(em), 0) + 1
    assert set(counts) <= set(exact)
    keys = [y for y in exact if exact[y] * n >= 5]
    obs = np.array([counts.get(y, 0) for y in keys], float)
    exp = np.array([exact[y] * n for y in keys])
    rest_o = n - obs.sum()
    rest_e = n - exp.sum()
    if rest_e >= 5:
        obs = np.append(obs, rest_o)
        exp = np.append(exp, rest_e)
    stat = ((obs - exp) ** 2 / exp).sum()
    assert chi2d.sf(stat, len(obs) - 1) > 1e-3
