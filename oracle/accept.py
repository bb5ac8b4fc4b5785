"""Acceptance: greedy longest prefix, and the textbook rejection rule.

Greedy ("Speculative decoding", gpillon.github.io/ignis, "One round, step by
step", step 4; "Draft heads and speculative decoding",
research.strata2signal.com, "Guess, then check"): walk along the drafts while
each equals the token the model itself would have chosen at that position; at
the first mismatch keep the model's own token; if every draft matches, the
model's token after the last draft is kept too.  The committed run has between
1 and k + 1 tokens.

Sampled (the textbook rule the strata2signal page cites: Leviathan, Kalman &
Matias 2022, Definition 3.7 / Theorem 3.8): draft d_i, drawn by the drafter
from q_i, is kept with probability min(1, p_{i-1}(d_i) / q_i(d_i)); on the
first rejection a token is drawn from the residual max(0, p_{i-1} - q_i)
(normalised) and the round ends; if every draft is kept a bonus token is drawn
from p_k.  p_j = softmax(z_j / T) is the target's distribution at row j.

Two implementations of the sampled rule live here:
  * rule_outcomes: the rule as exact float64 outcome probabilities (used to
    prove distribution preservation by enumeration);
  * accept_sampled: the sampler that draws with Philox4x32-10 uniforms; its
    decisions are taken in float32, the precision the kernels take them in.
Residual and bonus draws use the exponential race: the winner is
argmin_v E_v / w_v with E_v = -ln U_v, which samples v with probability
w_v / sum(w) for any non-negative weights.
"""
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .philox import accept_uniform, race_uniforms


def argmax_lowest(z) -> int:
    """Index of the maximum, lowest index on ties."""
    z = np.asarray(z)
    return int(np.flatnonzero(z == z.max())[0])


def row_stats(logits, next_tokens, temperature: float = 1.0) -> Dict[str, np.ndarray]:
    """Per-row statistics the LM head reports.

    max: max logit; lse: log sum exp(z / T); argmax: lowest-index argmax;
    z_next: logit of the row's next draft token (NaN where there is none).
    """
    z = np.asarray(logits, np.float32)
    R = z.shape[0]
    zd = z.astype(np.float64) / temperature
    m = zd.max(axis=1)
    lse = m + np.log(np.exp(zd - m[:, None]).sum(axis=1))
    am = np.array([argmax_lowest(z[r]) for r in range(R)], np.int64)
    zn = np.full(R, np.nan, np.float32)
    for r in range(R):
        t = int(next_tokens[r])
        if t >= 0:
            zn[r] = z[r, t]
    return {"max": z.max(axis=1), "lse": lse, "argmax": am, "z_next": zn}


def accept_greedy(lane_logits, drafts: Sequence[int]) -> Tuple[int, List[int]]:
    """lane_logits: [k+1, V] rows of one lane; drafts: d_1..d_k.

    Returns (c, emitted): c = a + 1 with a the longest matching prefix, emitted
    = d_1..d_a followed by the model's own token at row a.
    """
    k = len(drafts)
    t = [argmax_lowest(lane_logits[j]) for j in range(k + 1)]
    a = 0
    while a < k and int(drafts[a]) == t[a]:
        a += 1
    return a + 1, [int(d) for d in drafts[:a]] + [t[a]]


def _probs32(z, inv_t: np.float32):
    """Target distribution at one row, as float32 values (the kernels' precision)."""
    z = np.asarray(z, np.float32)
    m = z.max()
    arg = (z - m).astype(np.float32) * inv_t
    e = np.exp(arg.astype(np.float64)).astype(np.float32)
    Z = np.float32(e.astype(np.float64).sum())
    return (e / Z).astype(np.float32)


def _race(E, w) -> int:
    """argmin E / w over w > 0 (float32), lowest index on ties; -1 if every weight is 0."""
    E = np.asarray(E, np.float32)
    w = np.asarray(w, np.float32)
    with np.errstate(divide="ignore"):
        key = np.where(w > 0, (E / np.where(w > 0, w, np.float32(1))).astype(np.float32),
                       np.float32(np.inf))
    if not np.isfinite(key).any():
        return -1
    return argmax_lowest(-key)


def accept_sampled(lane_logits, drafts: Sequence[int], q_rows, temperature: float,
                   seed: int, lane: int, kv_len: int) -> Tuple[int, List[int]]:
    """The textbook rule with Philox uniforms.

    lane_logits: [k+1, V] float32; drafts: d_1..d_k; q_rows[i-1]: drafter q_i
    (float32 [V]) for draft d_i.  Draft d_i sits at absolute position kv_len + i;
    the bonus token at kv_len + k + 1.
    """
    k = len(drafts)
    V = lane_logits.shape[1]
    inv_t = np.float32(1.0 / temperature)
    for i in range(1, k + 1):
        pos = kv_len + i
        p = _probs32(lane_logits[i - 1], inv_t)
        q = np.asarray(q_rows[i - 1], np.float32)
        d = int(drafts[i - 1])
        u = np.float32(accept_uniform(seed, pos, lane))
        if np.float32(u * q[d]) < p[d]:
            continue
        E = (-np.log(race_uniforms(seed, pos, lane, V))).astype(np.float32)
        w = np.maximum(np.float32(0), (p - q).astype(np.float32))
        x = _race(E, w)
        if x < 0:                     # residual vanished in floating point: draw from p
            x = _race(E, p)
        return i, [int(t) for t in drafts[: i - 1]] + [x]
    # every draft kept: bonus token from p_k by the race on Gumbel keys z/T - ln E
    pos = kv_len + k + 1
    E = (-np.log(race_uniforms(seed, pos, lane, V))).astype(np.float32)
    z = np.asarray(lane_logits[k], np.float32)
    g = (z * inv_t - np.log(E).astype(np.float32)).astype(np.float32)
    return k + 1, [int(t) for t in drafts] + [argmax_lowest(g)]


# ---------------------------------------------------------------------- exact rule
def rule_outcomes(p_rows, q_rows, drafts) -> Dict[Tuple[int, ...], float]:
    """Exact float64 distribution of the emitted tokens of one round, given the drafts.

    p_rows[j] (j = 0..k): target distribution after the anchor and d_1..d_j;
    q_rows[i-1] (i = 1..k): drafter distribution of d_i.
    """
    k = len(drafts)
    out: Dict[Tuple[int, ...], float] = {}
    reach = 1.0                                   # probability that d_1..d_{i-1} were all kept
    for i in range(1, k + 1):
        p = np.asarray(p_rows[i - 1], np.float64)
        q = np.asarray(q_rows[i - 1], np.float64)
        d = int(drafts[i - 1])
        keep = min(1.0, p[d] / q[d]) if q[d] > 0 else 1.0
        rej = reach * (1.0 - keep)
        if rej > 0:
            w = np.maximum(0.0, p - q)
            s = w.sum()
            r = w / s if s > 0 else p
            prefix = tuple(int(t) for t in drafts[: i - 1])
            for x in np.flatnonzero(r > 0):
                key = prefix + (int(x),)
                out[key] = out.get(key, 0.0) + rej * r[x]
        reach *= keep
    if reach > 0:
        pk = np.asarray(p_rows[k], np.float64)
        prefix = tuple(int(t) for t in drafts)
        for x in np.flatnonzero(pk > 0):
            key = prefix + (int(x),)
            out[key] = out.get(key, 0.0) + reach * pk[x]
    return out


def one_position_output(p, q) -> np.ndarray:
    """Output distribution of one draft position under the rule, averaged over d ~ q.

    sum_d q(d) [min(1, p(d)/q(d)) 1{x = d} + (1 - sum_v min(p, q)) r(x)], with
    r = max(0, p - q) normalised.  Equals p by the theorem.
    """
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    keep = np.where(q > 0, np.minimum(1.0, p / np.where(q > 0, q, 1.0)), 1.0)
    w = np.maximum(0.0, p - q)
    s = w.sum()
    r = w / s if s > 0 else p
    rej_mass = 1.0 - np.minimum(p, q).sum()
    return q * keep + rej_mass * r
