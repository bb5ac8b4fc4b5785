"""Pins of the copy-from-the-conversation (n-gram prompt lookup) drafter in the oracle.

The pages ("Speculative decoding", mashbox docs, "Where it runs") say only that the
drafter looks up the last few tokens earlier in the request and proposes what followed
them there; the pins check the readings written in oracle/ngram.py against hand-built
histories whose right answer is fixed by construction, and the method's own invariant:
speculative greedy decoding with these drafts commits exactly the plain greedy
continuation (mashbox docs, "What it does for you").
"""
import numpy as np

import synth
from helpers import oracle_cache
from oracle import OracleModel, ngram_draft, round_tokens, speculative_greedy_ngram


def test_periodic_history_continues_the_period():
    period = [5, 6, 7, 8]
    h = period * 5 + [5, 6]
    drafts, n = ngram_draft(h, 7, 3)
    assert n == 3
    # the text is periodic, so the copy is the next 7 tokens of the period
    assert drafts == [(period * 10)[len(h) + i] for i in range(7)]


def test_longest_suffix_wins_over_a_more_recent_shorter_one():
    #     0  1  2  3   4  5  6  7   8   9 10 11
    h = [1, 2, 3, 9, 4, 2, 3, 7, 3, 1, 2, 3]
    assert ngram_draft(h, 1, 3)[0] == [9]        # "1 2 3" at 0, followed by 9
    assert ngram_draft(h, 1, 2)[0] == [7]        # "2 3" most recently at 5, followed by 7
    assert ngram_draft(h, 1, 1)[0] == [1]        # "3" most recently at 8, followed by 1
    assert ngram_draft(h, 1, 3, n_min=3)[1] == 3


def test_most_recent_occurrence_among_equal_lengths():
    h = [1, 2, 5, 1, 2, 6, 1, 2]
    assert ngram_draft(h, 2, 2) == ([6, 1], 2)


def test_copy_runs_over_its_own_proposals():
    assert ngram_draft([4, 4], 3, 1) == ([4, 4, 4], 1)
    # match at 0 followed by "1 2", then the copy reads the tokens it proposed
    assert ngram_draft([1, 2, 1, 2], 5, 2) == ([1, 2, 1, 2, 1], 2)


def test_no_match_no_drafts_and_the_round_falls_back_to_the_anchor():
    h = list(range(10, 30))
    assert ngram_draft(h, 4, 3) == ([], 0)
    assert ngram_draft([7], 4, 3) == ([], 0)            # a lone anchor has nothing earlier
    assert round_tokens(h, 4, 3) == ([29, 29, 29, 29, 29], 0)
    assert round_tokens([3, 1, 3], 2, 2) == ([3, 1, 3], 1)


def test_n_range_bounds():
    h = [2, 3, 2, 3, 2, 3]
    for n_max in range(1, 6):
        d, n = ngram_draft(h, 4, n_max)
        assert n == min(n_max, 4)                       # the suffix of length 5 never recurs
        assert d == [2, 3, 2, 3]


def test_speculative_greedy_with_ngram_drafts_equals_plain_greedy_tiny():
    """Tiny fp32 decoder, two lanes, 12 rounds at k = 3: the committed tokens are the
    plain greedy continuation of each lane, and every round commits 1 .. k + 1."""
    cfg = synth.get_config("tiny-fp32")
    m = OracleModel(cfg, synth.model_weights(cfg))
    prompts = [synth.prompt_tokens(cfg), synth.uniform_tokens(cfg.input_seed, 91, 64, cfg.vocab)]
    prompts[1][32:] = prompts[1][:32]                    # a lane whose prompt repeats itself
    base = oracle_cache(cfg, 2, 0, 24)
    m.prefill(base, [list(map(int, p)) for p in prompts], chunk=16)   # the last token stays the anchor
    anchors = [int(p[-1]) for p in prompts]
    ref = m.plain_greedy(base.copy(), anchors, 12 * (cfg.k + 1) + 2)
    out, counts = speculative_greedy_ngram(m, base, [list(map(int, p)) for p in prompts], 12, cfg.k, 3)
    assert counts.min() >= 1 and counts.max() <= cfg.k + 1
    for l in range(2):
        assert out[l] == [int(t) for t in ref[l][: len(out[l])]]
    assert list(base.kv_len) == [63 + len(o) for o in out]
