"""Copy-from-the-conversation drafter (n-gram prompt lookup).  TEST INFRASTRUCTURE ONLY.

What the pages say the drafter does:
  * "Speculative decoding" (mashbox docs, "Where it runs", `--speculation ngram`):
    the drafter looks up the last few tokens earlier in the request and proposes
    the tokens that followed them there;
  * "Draft heads and speculative decoding, in plain words" (research.strata2signal.com,
    the drafter table, row "No model at all"): the text so far, an n-gram that recurs
    or a copy of the prompt; nothing to ship.

The pages fix none of the details; the readings taken here:
  * "the last few tokens" is the history's suffix of length n, tried from n_max down
    to n_min: the longest suffix that occurs earlier wins;
  * "earlier in the request" is the most recent earlier occurrence: the largest start p
    with p + n < len (the occurrence is followed by at least one token);
  * "the tokens that followed them there" are history[p + n], history[p + n + 1], ...;
    a copy that reaches the end of the history goes on over the tokens it has just
    proposed (an overlapping copy, as in LZ77), so k drafts exist whenever a match does;
  * no match, no drafts.

The round loop keeps k + 1 columns per lane so that no round needs a host round trip:
a lane without a match is given its anchor token k times as filler guesses.  Any guess
is checked by the model, so the output is the plain greedy output either way (mashbox
docs, "What it does for you": a greedy request keeps the model's top token at every
position).
"""
from typing import List, Sequence, Tuple

import numpy as np

from .accept import accept_greedy


def ngram_draft(history: Sequence[int], k: int, n_max: int, n_min: int = 1) -> Tuple[List[int], int]:
    """Drafts for one lane and the length of the suffix that matched (0: no match)."""
    h = [int(t) for t in history]
    L = len(h)
    for n in range(min(n_max, L - 1), n_min - 1, -1):
        suffix = h[L - n:]
        for p in range(L - n - 1, -1, -1):          # most recent first
            if h[p:p + n] == suffix:
                ext = list(h)
                for i in range(k):                  # overlapping copy
                    ext.append(ext[p + n + i])
                return ext[L:], n
    return [], 0


def round_tokens(history: Sequence[int], k: int, n_max: int, n_min: int = 1) -> Tuple[List[int], int]:
    """The lane's columns for one round: its anchor (the last token of the history)
    followed by k guesses (the drafts, or the anchor repeated when nothing matches)."""
    drafts, n = ngram_draft(history, k, n_max, n_min)
    anchor = int(history[-1])
    return [anchor] + (drafts if drafts else [anchor] * k), n


def speculative_greedy_ngram(model, cache, histories: Sequence[Sequence[int]], rounds: int, k: int, n_max: int,
                             n_min: int = 1):
    """Greedy rounds with n-gram drafts on every lane: the histories end with each lane's
    anchor (the token at position kv_len).  Returns (per-lane tokens committed after the
    starting histories, per-round committed counts [rounds][L])."""
    hist = [[int(t) for t in h] for h in histories]
    start = [len(h) for h in hist]
    counts = []
    for _ in range(rounds):
        toks = [round_tokens(h, k, n_max, n_min)[0] for h in hist]
        res = model.verify_round(cache, toks)
        committed = []
        for l, rows in enumerate(res.lane_rows):
            c, emitted = accept_greedy(res.logits[rows.start:rows.stop], toks[l][1:])
            committed.append(c)
            hist[l] += emitted
        model.commit(cache, res, committed)
        counts.append(committed)
    return [h[s:] for h, s in zip(hist, start)], np.array(counts, np.int64)
