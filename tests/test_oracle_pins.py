"""Pins of the oracle's small pieces against what the pages and the mathematics fix."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import (accept_greedy, bf16, philox4x32_10, plan_drafts, plan_drafts_bruteforce,
                    uniform01)
from oracle.accept import argmax_lowest
from oracle.metrics import acceptance_summary, implied_alpha, textbook_tokens_per_round
from oracle.philox import race_uniforms, accept_uniform


# ---------------------------------------------------------------- row budget
def test_row_budget_worked_example():
    for k, budget, lanes, want in read_golden("row_budget_worked_example.txt"):
        assert plan_drafts(int(k), int(budget), int(lanes)) == int(want), (k, budget, lanes)


def test_row_budget_closed_form_equals_bruteforce():
    # the closed form min(k, rows/lanes - 1) is the largest draft count whose round fits the budget
    for k in range(0, 17):
        for budget in range(0, 65):
            for lanes in range(1, 65):
                assert plan_drafts(k, budget, lanes) == plan_drafts_bruteforce(k, budget, lanes)


def test_row_budget_rejects_bad_lanes():
    with pytest.raises(ValueError):
        plan_drafts(3, 8, 0)


# ---------------------------------------------------------------- greedy walk
def test_greedy_walk_table():
    V = 16
    model_tokens = [3, 7, 1, 9, 12]          # the model's own token after anchor, d1, d2, d3, d4
    logits = np.zeros((5, V), np.float32)
    for j, t in enumerate(model_tokens):
        logits[j, t] = 5.0
    for case, pattern, want in read_golden("greedy_walk_table.txt"):
        drafts = [model_tokens[i] if pattern[i] == "1" else (model_tokens[i] + 1) % V for i in range(4)]
        c, emitted = accept_greedy(logits, drafts)
        assert c == int(want), case
        assert len(emitted) == c
        # kept drafts, then the model's own token at the first mismatch (or after the last draft)
        assert emitted == model_tokens[:c]


def test_greedy_run_bounds_random():
    rng = np.random.default_rng(0)
    for _ in range(200):
        k = int(rng.integers(0, 9))
        logits = rng.standard_normal((k + 1, 32)).astype(np.float32)
        drafts = rng.integers(0, 32, size=k)
        c, em = accept_greedy(logits, drafts)
        assert 1 <= c <= k + 1 and len(em) == c


def test_argmax_lowest_index_on_ties():
    assert argmax_lowest(np.array([1.0, 3.0, 3.0, 2.0], np.float32)) == 1


# ---------------------------------------------------------------- Philox
def test_philox_known_answers():
    for row in read_golden("philox4x32_10_kat.txt"):
        w = [int(x, 16) for x in row]
        out = philox4x32_10(w[0:4], w[4:6])
        assert [int(x) for x in out] == w[6:10]


def test_philox_distinct_counters_distinct_outputs():
    n = 200_000
    ctr = np.arange(n, dtype=np.uint64)
    out = philox4x32_10((ctr, 5, 1, 0), (123, 456))
    packed = (out[0].astype(np.uint64) << np.uint64(32)) | out[1].astype(np.uint64)
    assert np.unique(packed).size == n           # a bijection cannot collide on 64 of 128 bits here


def test_uniform_conversion_range_and_chi2():
    assert uniform01(np.uint32(0)) == 0.5 * 2.0 ** -23
    assert uniform01(np.uint32(0xFFFFFFFF)) == (2.0 ** 23 - 0.5) * 2.0 ** -23
    u = race_uniforms(seed=99, pos=17, lane=3, vocab=400_000)
    assert np.all((u > 0) & (u < 1))
    assert np.all(u.astype(np.float32).astype(np.float64) == u)        # exact in float32
    counts, _ = np.histogram(u, bins=100, range=(0, 1))
    exp = u.size / 100
    chi2 = ((counts - exp) ** 2 / exp).sum()
    from scipy.stats import chi2 as chi2d
    assert chi2d.sf(chi2, 99) > 1e-4


def test_accept_and_race_streams_differ():
    a = accept_uniform(7, np.arange(8), 0)
    r = np.array([race_uniforms(7, p, 0, 1)[0] for p in range(8)])
    assert not np.any(a == r)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_rounding_matches_library_conversion():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32) * 10.0,
        # exact ties between two bf16 neighbours, both parities of the kept bit
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- acceptance accounting
def test_acceptance_receipt_arithmetic():
    g = {r[0]: [float(v) for v in r[1:]] for r in read_golden("acceptance_receipt.txt")}
    acc, prop, rounds = g["accepted"][0], g["proposed"][0], g["rounds"][0]
    assert round(100 * acc / prop, 1) == g["rate_percent"][0]
    assert round(1 + acc / rounds, 2) == g["tokens_per_round"][0]
    by_slot = np.array(g["by_slot"])
    assert round(1 + by_slot.sum(), 2) == g["tokens_per_round"][0]
    cond = [by_slot[0]] + [by_slot[i] / by_slot[i - 1] for i in range(1, 4)]
    assert np.allclose(np.round(cond, 3), g["conditional"], atol=1e-3)
    assert round(implied_alpha(g["tokens_per_round"][0], int(g["depth"][0])), 2) == g["implied_alpha"][0]


def test_acceptance_summary_senses_agree():
    rng = np.random.default_rng(2)
    k = 4
    c = rng.integers(1, k + 2, size=500)
    s = acceptance_summary(c, np.full(500, k))
    assert np.isclose(s["tokens_per_round"], 1 + s["by_slot"].sum())     # 1 + sum of slots
    assert np.isclose(s["tokens_per_round"], 1 + s["accepted"] / s["rounds"])


@pytest.mark.parametrize("alpha", [0.35, 0.5, 0.7, 0.9])
def test_tokens_per_round_matches_textbook_with_planted_alpha(alpha):
    # planted i.i.d. matches against the model's own greedy tokens -> E[c] = (1 - a^(g+1)) / (1 - a)
    gamma, V, n = 7, 64, 4000
    rng = np.random.default_rng(int(alpha * 100))
    cs = []
    for _ in range(n):
        logits = rng.standard_normal((gamma + 1, V)).astype(np.float32)
        t = [argmax_lowest(logits[j]) for j in range(gamma + 1)]
        hit = rng.random(gamma) < alpha
        drafts = [t[i] if hit[i] else (t[i] + 1 + int(rng.integers(0, V - 1))) % V for i in range(gamma)]
        cs.append(accept_greedy(logits, drafts)[0])
    cs = np.array(cs, float)
    want = textbook_tokens_per_round(alpha, gamma)
    assert abs(cs.mean() - want) < 4 * cs.std() / np.sqrt(n)
