"""Per-request miss back-off (mashbox docs, "What it does for you"): the oracle against
hand-traced passes that follow the rules the page states (4 passes in a row that keep no
guess, a wait of 16 passes, doubled by each further 4 up to 256, a kept guess setting it
back to 16 unless waiting, calls that start during a wait making no guesses, the rest of
the call in which a wait begins still guessing, calls without guesses not counting toward
misses), and the C ABI's host implementation against the oracle on seeded sequences.
"""
import ctypes as C

import numpy as np

from oracle.backoff import Backoff, call_begin, pass_end
from speculative_decoding_verify_round_amd import binding as B


def run(kept_fn, n_calls, passes_per_call=1, lanes=1, k=3, budget=8):
    """Drive the oracle; returns the passes (1-based) in which each request guessed."""
    st = [Backoff() for _ in range(lanes)]
    guessed = [[] for _ in range(lanes)]
    p = 0
    for _ in range(n_calls):
        spec, drafts = call_begin(st, k, budget)
        for _ in range(passes_per_call):
            p += 1
            for l in range(lanes):
                if drafts[l] > 0:
                    guessed[l].append(p)
            pass_end(st, [kept_fn(l, p) if drafts[l] > 0 else 0 for l in range(lanes)], spec)
    return guessed, st


def spans(ps):
    out, start = [], None
    for i, p in enumerate(ps):
        if start is None:
            start = p
        if i + 1 == len(ps) or ps[i + 1] != p + 1:
            out.append((start, p))
            start = None
    return out


def test_waits_double_up_to_256():
    g, _ = run(lambda l, p: 0, 800)
    # 4 misses, then waits of 16, 32, 64, 128, 256, 256 passes
    assert spans(g[0]) == [(1, 4), (21, 24), (57, 60), (125, 128), (257, 260), (517, 520), (777, 780)]


def test_kept_guess_resets_the_wait_to_16():
    keep = {4, 30}
    g, st = run(lambda l, p: 1 if p in keep else 0, 90)
    # misses 1-3, kept at 4, misses 5-8 -> wait 16 (9-24); 25-28 miss -> wait 32 (29-60);
    # 61-64 miss -> wait 64 (65-128)... the kept guess at 30 falls inside a wait and is not made
    assert spans(g[0])[:3] == [(1, 8), (25, 28), (61, 64)]
    keep2 = {4, 26}
    g2, _ = run(lambda l, p: 1 if p in keep2 else 0, 90)
    # kept at 26 (outside a wait) sets the wait back to 16: misses 27-30 -> wait 16 (31-46)
    assert spans(g2[0])[:3] == [(1, 8), (25, 30), (47, 50)]


def test_wait_beginning_mid_call_and_calls_starting_in_it():
    g, _ = run(lambda l, p: 0, 10, passes_per_call=3)
    # calls of 3 passes: the 4th miss (pass 4) starts a 16-pass wait; passes 5 and 6 of that
    # call still guess and count toward it (it ends after pass 20); the call of passes 19-21
    # starts inside the wait and makes no guesses; guessing resumes at pass 22, the 4th miss
    # after that is pass 25, the first of a call that may guess, so 25-27 still guess
    assert spans(g[0]) == [(1, 6), (22, 27)]
    # the same at one pass per call: the wait is passes 5-20, guessing resumes at 21
    g1, _ = run(lambda l, p: 0, 30, passes_per_call=1)
    assert spans(g1[0])[:2] == [(1, 4), (21, 24)]


def test_kept_guess_inside_a_wait_does_not_reset_it():
    # calls of 3 passes: the 4th miss (pass 4) starts a 16-pass wait, the next one will be 32;
    # pass 6 (the rest of that call) keeps a guess inside the wait and changes nothing: after
    # 22-24 and 25 miss, the wait begun at 25 lasts 32 passes (26-57), not 16
    g, _ = run(lambda l, p: 1 if p == 6 else 0, 20, passes_per_call=3)
    assert spans(g[0]) == [(1, 6), (22, 27), (58, 60)]
    g_out, _ = run(lambda l, p: 1 if p == 23 else 0, 20, passes_per_call=3)
    # a guess kept at 23, outside a wait: misses 24-27 trigger a 16-pass wait (28-43); the
    # call of 43-45 starts inside it, so guessing resumes at 46, and the 4th miss (49) starts
    # a 32-pass wait while 50-51 still guess
    assert spans(g_out[0]) == [(1, 6), (22, 27), (46, 51)]


def test_calls_without_guesses_do_not_count():
    # five lanes on a budget of 8 draft nothing: no call speculates, no wait ever starts
    g, st = run(lambda l, p: 0, 40, lanes=5, k=3, budget=8)
    assert all(not x for x in g)
    assert all(s.miss_run == 0 and s.wait_left == 0 and s.wait_len == 16 for s in st)
    # two lanes: one waiting, one guessing; the waiting one's passes only shorten its wait
    g2, _ = run(lambda l, p: 1 if l == 1 else 0, 30, lanes=2)
    assert spans(g2[0])[:2] == [(1, 4), (21, 24)]
    assert spans(g2[1]) == [(1, 30)]


def _c_states(n):
    arr = (B.SpecBackoff * n)()
    assert B.load_library().spec_backoff_init(arr, n) == 0
    return arr


def test_c_abi_matches_oracle_on_seeded_sequences():
    lib = B.load_library()
    rng = np.random.default_rng(5)
    for trial in range(60):
        lanes = int(rng.integers(1, 9))
        k = int(rng.integers(0, 8))
        budget = int(rng.choice([0, 8, 16, 64]))
        P = int(rng.integers(1, 6))
        p_keep = float(rng.choice([0.0, 0.1, 0.5]))
        st = [Backoff() for _ in range(lanes)]
        cs = _c_states(lanes)
        drafts_c = (C.c_int32 * lanes)()
        kept_c = (C.c_int32 * lanes)()
        for call in range(120):
            spec, drafts = call_begin(st, k, budget)
            r = lib.spec_backoff_call(cs, lanes, k, budget, drafts_c)
            assert r == int(spec) and list(drafts_c) == drafts, (trial, call)
            for _ in range(P):
                kept = [int(rng.random() < p_keep) * int(rng.integers(1, k + 1)) if drafts[l] else 0
                        for l in range(lanes)]
                pass_end(st, kept, spec)
                for l in range(lanes):
                    kept_c[l] = kept[l]
                assert lib.spec_backoff_pass(cs, lanes, kept_c, int(spec)) == 0
                for l in range(lanes):
                    assert (cs[l].miss_run, cs[l].wait_len, cs[l].wait_left, bool(cs[l].may_guess)) == \
                        (st[l].miss_run, st[l].wait_len, st[l].wait_left, st[l].may_guess), (trial, call, l)


def test_c_abi_validation():
    lib = B.load_library()
    cs = _c_states(2)
    d = (C.c_int32 * 2)()
    assert lib.spec_backoff_init(None, 2) == B.SPEC_E_INVAL
    assert lib.spec_backoff_init(cs, 0) == B.SPEC_E_INVAL
    assert lib.spec_backoff_call(cs, 2, -1, 8, d) == B.SPEC_E_INVAL
    assert lib.spec_backoff_call(cs, 2, 3, -1, d) == B.SPEC_E_INVAL
    assert lib.spec_backoff_call(cs, 2, 3, 8, None) == B.SPEC_E_INVAL
    assert lib.spec_backoff_pass(cs, 2, None, 1) == B.SPEC_E_INVAL
    assert lib.spec_backoff_pass(None, 2, d, 1) == B.SPEC_E_INVAL
