"""Acceptance accounting, as the strata2signal page ("Acceptance: three numbers
with one name") defines its three senses of "acceptance", and the textbook
tokens-per-round formula from its section on the 2022 paper.

  * guesses accepted / guesses proposed;
  * tokens a round = 1 + accepted / rounds (the model's own token plus kept guesses);
  * by slot: the share of rounds in which guess i survived; 1 + their sum is
    tokens a round again; and each slot given the one before;
  * textbook: (1 - alpha^(gamma+1)) / (1 - alpha) tokens a round for gamma
    guesses that each survive independently with probability alpha.
"""
from typing import Dict, Sequence

import numpy as np


def acceptance_summary(committed: Sequence[int], drafts: Sequence[int]) -> Dict[str, object]:
    """committed[n]: tokens committed by lane-round n (= accepted + 1); drafts[n]: guesses proposed."""
    c = np.asarray(committed, np.int64)
    g = np.asarray(drafts, np.int64)
    accepted = int((c - 1).sum())
    proposed = int(g.sum())
    kmax = int(g.max()) if g.size else 0
    by_slot = np.array([np.mean(c - 1 >= i) for i in range(1, kmax + 1)]) if kmax else np.zeros(0)
    cond = np.array([by_slot[0]] + [by_slot[i] / by_slot[i - 1] if by_slot[i - 1] > 0 else 0.0
                                    for i in range(1, kmax)]) if kmax else np.zeros(0)
    return {
        "accepted": accepted, "proposed": proposed,
        "rate": accepted / proposed if proposed else 0.0,
        "rounds": int(c.size),
        "tokens_per_round": 1.0 + accepted / c.size if c.size else 0.0,
        "by_slot": by_slot, "conditional": cond,
    }


def textbook_tokens_per_round(alpha: float, gamma: int) -> float:
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def implied_alpha(tokens_per_round: float, gamma: int) -> float:
    """The single i.i.d. survival rate that gives `tokens_per_round` at depth gamma (bisection)."""
    lo, hi = 0.0, 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if textbook_tokens_per_round(mid, gamma) < tokens_per_round:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)
