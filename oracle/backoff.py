"""Per-request miss back-off of a drafter.  TEST INFRASTRUCTURE ONLY.

"Speculative decoding" (mashbox docs, "What it does for you", the paragraph on
requests whose guesses keep missing), restated:
  * the engine runs several passes (verify rounds) in one device call and decides once
    per call whether it speculates: a call in which no request has a guess runs without
    speculation; here the call speculates when some request may guess (is not waiting
    when the call starts) and the row budget leaves it at least one draft;
  * in a call that speculates every pass counts for each request that may guess,
    whether or not it has a guess in that pass; in a call that does not, passes do not
    count toward misses, only toward the wait of a request already waiting;
  * after 4 counted passes in a row in which the model keeps none of the request's
    guesses, the request waits 16 passes; a call that starts during the wait makes no
    guesses for it; the rest of the call in which the wait began still guesses, and
    those passes count toward the wait, kept guesses or not;
  * each further 4 such passes in a row double the wait, up to 256;
  * a pass that keeps a guess sets the wait back to 16, unless the request is waiting.

Readings: the miss count starts again after each wait is triggered (the next 4 misses
in a row trigger the next, doubled wait); a kept guess outside a wait clears it; the
passes of a call that does not speculate never clear it.  With the row budget ("The
row budget", ignis), a request that may guess drafts min(k, rows / lanes - 1), lanes
being every active lane of the round, waiting ones included; one that may not drafts 0.
"""
from dataclasses import dataclass
from typing import List, Sequence

from .planner import plan_drafts

MISS_PASSES = 4
FIRST_WAIT = 16
MAX_WAIT = 256


@dataclass
class Backoff:
    miss_run: int = 0          # counted passes in a row with no kept guess, since the last trigger
    wait_len: int = FIRST_WAIT  # length of the next wait
    wait_left: int = 0         # passes of the current wait still to go (0: not waiting)
    may_guess: bool = True     # decided at the start of the current call


def call_begin(states: Sequence[Backoff], k: int, row_budget: int) -> (bool, List[int]):
    """Start of a device call: who may guess, whether the call speculates, drafts per request."""
    lanes = len(states)
    plan = plan_drafts(k, row_budget, lanes)
    for s in states:
        s.may_guess = s.wait_left == 0
    speculates = plan > 0 and any(s.may_guess for s in states)    # some request has guesses
    return speculates, [plan if (speculates and s.may_guess) else 0 for s in states]


def pass_end(states: Sequence[Backoff], kept: Sequence[int], speculates: bool) -> None:
    """End of one pass of the call: kept[i] = guesses of request i the model kept."""
    for s, kp in zip(states, kept):
        if speculates and s.may_guess:
            if s.wait_left > 0:                 # the wait began in this call: the pass counts toward it
                s.wait_left -= 1
            elif kp > 0:
                s.miss_run = 0
                s.wait_len = FIRST_WAIT
            else:
                s.miss_run += 1
                if s.miss_run == MISS_PASSES:
                    s.miss_run = 0
                    s.wait_left = s.wait_len
                    s.wait_len = min(2 * s.wait_len, MAX_WAIT)
        elif s.wait_left > 0:
            s.wait_left -= 1
