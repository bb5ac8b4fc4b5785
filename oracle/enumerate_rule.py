"""Exact enumeration of the sampled acceptance rule on a toy vocabulary.

Distribution preservation ("Speculative decoding", gpillon.github.io/ignis:
sampling keeps its distribution; the strata2signal page: the right acceptance
rule samples "without changing the distribution", Leviathan et al. Theorem
3.8): chaining verify rounds must emit token sequences with exactly the
target's autoregressive probabilities prod_i p(y_i | y_<i), whatever the
drafter proposes.

The toy target p(. | context) and drafter q(. | context) are softmaxes of
seeded random logits, one table row per context.  A round from a context
enumerates every draft tuple (d_1..d_k, probability prod q), applies
oracle.accept.rule_outcomes, and the rounds are chained by dynamic programming
over emitted prefixes until N tokens are out.
"""
import itertools
from typing import Dict, Tuple

import numpy as np

from .accept import rule_outcomes


class ToyLM:
    def __init__(self, vocab: int, seed: int, scale: float):
        self.V, self.seed, self.scale = vocab, seed, scale
        self._cache: Dict[Tuple[int, ...], np.ndarray] = {}

    def __call__(self, ctx: Tuple[int, ...]) -> np.ndarray:
        p = self._cache.get(ctx)
        if p is None:
            r = np.random.default_rng([self.seed, len(ctx), *ctx])
            z = r.standard_normal(self.V) * self.scale
            e = np.exp(z - z.max())
            p = e / e.sum()
            self._cache[ctx] = p
        return p


def round_distribution(p_lm: ToyLM, q_lm: ToyLM, ctx: Tuple[int, ...], k: int) -> Dict[Tuple[int, ...], float]:
    """Exact distribution of the tokens one round emits from `ctx` (anchor included in ctx)."""
    V = p_lm.V
    out: Dict[Tuple[int, ...], float] = {}
    for drafts in itertools.product(range(V), repeat=k):
        pr = 1.0
        q_rows = []
        for i in range(k):
            q = q_lm(ctx + drafts[:i])
            q_rows.append(q)
            pr *= q[drafts[i]]
        if pr == 0.0:
            continue
        p_rows = [p_lm(ctx + drafts[:j]) for j in range(k + 1)]
        for y, w in rule_outcomes(p_rows, q_rows, drafts).items():
            out[y] = out.get(y, 0.0) + pr * w
    return out


def chained_distribution(p_lm: ToyLM, q_lm: ToyLM, base: Tuple[int, ...], k: int, n: int):
    """Distribution of the first n emitted tokens when rounds are chained from `base`."""
    final: Dict[Tuple[int, ...], float] = {}
    frontier: Dict[Tuple[int, ...], float] = {(): 1.0}
    while frontier:
        nxt: Dict[Tuple[int, ...], float] = {}
        for pre, w in frontier.items():
            for y, pw in round_distribution(p_lm, q_lm, base + pre, k).items():
                seq = pre + y
                if len(seq) >= n:
                    key = seq[:n]
                    final[key] = final.get(key, 0.0) + w * pw
                else:
                    nxt[seq] = nxt.get(seq, 0.0) + w * pw
        frontier = nxt
    return final


def autoregressive_distribution(p_lm: ToyLM, base: Tuple[int, ...], n: int):
    """prod_i p(y_i | base, y_<i) over all length-n sequences."""
    V = p_lm.V
    out = {}
    for y in itertools.product(range(V), repeat=n):
        pr = 1.0
        for i in range(n):
            pr *= p_lm(base + y[:i])[y[i]]
        out[y] = pr
    return out
