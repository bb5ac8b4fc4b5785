"""Per-row presence and frequency penalties in the verify round.  TEST INFRASTRUCTURE ONLY.

The FreeToken tracking issue ("Speculative decoding: MTP and DFlash", section
"Design") lists per-row presence and frequency penalties as part of the target-side
verify; the strata2signal page ("Tokens a round is a ceiling, not the speed-up", row
"Sampler settings") notes that a repeat penalty changes which tokens the model takes,
and so which guesses survive.

Readings (the pages give no formula):
  * the usual form: a token that occurs c times in what the row conditions on loses
    presence * [c > 0] + frequency * c from its logit, before temperature, softmax,
    argmax and every acceptance decision;
  * "per row": row j of a lane conditions on the lane's tokens up to its anchor and on
    the round's drafts d_1 .. d_j, so its counts are the lane's counts plus those
    drafts -- exactly the counts a plain one-token step at the same position would use,
    which keeps speculative decoding equal to plain decoding with the same penalties;
  * counts come from the caller (the lane's tokens so far, up to and including the
    anchor) and grow by each round's committed run.
The penalised logit is evaluated in float32, the precision the kernels use.
"""
from typing import Sequence

import numpy as np


def penalty(counts, presence: float, frequency: float) -> np.ndarray:
    c = np.asarray(counts)
    return (np.float32(presence) * (c > 0).astype(np.float32) + np.float32(frequency) * c.astype(np.float32)).astype(
        np.float32)


def penalized_rows(lane_logits, lane_tokens: Sequence[int], counts, presence: float, frequency: float) -> np.ndarray:
    """lane_logits [cols, V] of one lane's rows; lane_tokens = anchor, d_1 .. d_k; counts [V]
    of the lane's tokens up to its anchor.  Row j is penalised with counts + d_1 .. d_j."""
    z = np.asarray(lane_logits, np.float32)
    out = np.empty_like(z)
    c = np.array(counts, np.int64)
    for j in range(z.shape[0]):
        if j > 0:
            c[int(lane_tokens[j])] += 1
        out[j] = (z[j] - penalty(c, presence, frequency)).astype(np.float32)
    return out


def add_counts(counts, tokens: Sequence[int]) -> None:
    """counts [V] += one per token (the committed run of a round)."""
    for t in tokens:
        counts[int(t)] += 1
