"""Pins of the per-row presence / frequency penalties in the oracle.

The reading (oracle/penalty.py) is that row j of a lane is penalised with the counts of
everything it conditions on: the lane's tokens up to the anchor and the drafts d_1 .. d_j.
The pins check it against a plain decoder that keeps one running count of the tokens it
has fed, step by step (a different computation reaching the same counts), and the
method's invariant with penalties on: speculative greedy decoding commits the plain
greedy continuation of the penalised model.
"""
import numpy as np

import synth
from helpers import oracle_cache
from oracle import OracleModel, accept_greedy
from oracle.accept import argmax_lowest
from oracle.penalty import add_counts, penalized_rows, penalty

PRES, FREQ = 0.05, 0.03


def _tiny():
    cfg = synth.get_config("tiny-fp32")
    m = OracleModel(cfg, synth.model_weights(cfg))
    prompt = [int(t) for t in synth.prompt_tokens(cfg)]
    cache = oracle_cache(cfg, 1, 0, 24)
    m.prefill(cache, [prompt], chunk=16)
    return cfg, m, prompt, cache


def test_zero_penalties_change_nothing():
    z = np.random.default_rng(1).standard_normal((4, 50)).astype(np.float32)
    out = penalized_rows(z, [3, 7, 7, 9], np.arange(50) % 3, 0.0, 0.0)
    assert np.array_equal(out, z)


def test_verify_rows_equal_plain_penalised_steps():
    cfg, m, prompt, cache = _tiny()
    counts = np.bincount(prompt, minlength=cfg.vocab)          # the lane's tokens up to its anchor
    toks = [prompt[-1], 17, 17, 99, prompt[3]]                  # anchor + drafts (repeats on purpose)
    z = m.verify_round(cache.copy(), [toks]).logits
    rows = penalized_rows(z, toks, counts, PRES, FREQ)
    # plain decoding: one column per step, one running count of the tokens fed so far
    plain = cache.copy()
    running = counts.copy()
    for j, t in enumerate(toks):
        if j > 0:
            running[t] += 1
        res = m.verify_round(plain, [[t]])
        zj = res.logits[0]
        m.commit(plain, res, [1])
        want = (zj - penalty(running, PRES, FREQ)).astype(np.float32)
        assert np.array_equal(rows[j], want), j
    # a different reading -- every row penalised with the anchor-time counts -- differs
    same = (z - penalty(counts, PRES, FREQ)[None, :]).astype(np.float32)
    assert not np.array_equal(same[2:], rows[2:])


def test_large_frequency_penalty_avoids_seen_tokens():
    z = np.zeros((3, 10), np.float32)
    z[:, 4] = 1.0
    rows = penalized_rows(z, [0, 4, 5], np.eye(10, dtype=np.int64)[2], 0.0, 100.0)
    assert argmax_lowest(rows[0]) == 4                           # 4 not seen yet at row 0
    assert argmax_lowest(rows[1]) == 0 and rows[1][4] < -90     # row 1 saw draft d_1 = 4
    assert rows[2][5] < -90 and rows[2][2] < -90


def test_speculative_greedy_with_penalties_equals_plain_greedy():
    cfg, m, prompt, cache = _tiny()
    counts0 = np.bincount(prompt, minlength=cfg.vocab)
    # plain greedy with penalties: running counts over everything fed
    plain = cache.copy()
    counts = counts0.copy()
    cur, ref = prompt[-1], []
    for _ in range(40):
        res = m.verify_round(plain, [[cur]])
        nxt = argmax_lowest((res.logits[0] - penalty(counts, PRES, FREQ)).astype(np.float32))
        m.commit(plain, res, [1])
        ref.append(nxt)
        counts[nxt] += 1
        cur = nxt
    # speculative: drafts planted from the reference, committed runs added to the counts
    rng = np.random.default_rng(3)
    spec = cache.copy()
    counts = counts0.copy()
    anchor, out = prompt[-1], []
    while len(out) < 30:
        P = len(out)
        drafts = [ref[P + i] if rng.random() < 0.7 else int(rng.integers(0, cfg.vocab)) for i in range(cfg.k)]
        toks = [anchor] + drafts
        res = m.verify_round(spec, [toks])
        c, emitted = accept_greedy(penalized_rows(res.logits, toks, counts, PRES, FREQ), drafts)
        m.commit(spec, res, [c])
        add_counts(counts, emitted)
        out += emitted
        anchor = emitted[-1]
    assert out == ref[:len(out)]


def test_presence_and_frequency_terms_by_hand():
    # Hand-computed: a token seen c times loses presence * [c > 0] + frequency * c.
    # Counts 0, 1, 3 with presence 0.5 and frequency 0.25 lose 0, 0.75 and 1.25; with
    # frequency 0 every seen token loses exactly the presence, whatever its count.  A
    # swapped pair (0.25 * [c > 0] + 0.5 c) would give 0, 0.75, 1.75; a presence that
    # scales with the count (0.5 c + 0.25 c) would give 0, 0.75, 2.25.
    counts = np.array([0, 1, 3, 0], np.int64)
    z = np.array([[1.0, 1.0, 1.0, -2.0]], np.float32)
    got = penalized_rows(z, [0], counts, 0.5, 0.25)
    assert np.array_equal(got[0], np.array([1.0, 0.25, -0.25, -2.0], np.float32))
    got = penalized_rows(z, [0], counts, 0.5, 0.0)
    assert np.array_equal(got[0], np.array([1.0, 0.5, 0.5, -2.0], np.float32))
    got = penalized_rows(z, [0], counts, 0.0, 0.25)
    assert np.array_equal(got[0], np.array([1.0, 0.75, 0.25, -2.0], np.float32))
    # row 1 also counts its draft d_1 = token 0 (count 0 -> 1) and row 2 its d_2 = token 1
    # (count 1 -> 2): row 1 token 0 loses 0.75; row 2 token 1 loses 0.5 + 0.5 = 1.0
    z3 = np.zeros((3, 4), np.float32)
    got = penalized_rows(z3, [2, 0, 1], counts, 0.5, 0.25)
    assert np.array_equal(got[0], np.array([0.0, -0.75, -1.25, 0.0], np.float32))
    assert np.array_equal(got[1], np.array([-0.75, -0.75, -1.25, 0.0], np.float32))
    assert np.array_equal(got[2], np.array([-0.75, -1.0, -1.25, 0.0], np.float32))
