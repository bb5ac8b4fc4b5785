"""Oracle for the speculative-decoding verify round.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU implementation of what the verify round
computes, written from the pages' description of the method:

  * "Speculative decoding" (gpillon.github.io/ignis), section "One round, step
    by step": anchor plus k drafts per lane, one pass over all columns, the
    longest run of drafts the model would have chosen plus its own next token,
    the state advanced by exactly the committed run;
  * the same page, section "The row budget": drafts per lane;
  * "Draft heads and speculative decoding" (research.strata2signal.com),
    sections "Guess, then check" (the greedy walk and its worked table) and
    "Acceptance" (tokens per round); the textbook acceptance rule it cites
    (Leviathan, Kalman & Matias 2022, Definition 3.7 / Theorem 3.8);
  * the FreeToken tracking issue, "Per-request state": verify reads the live
    recurrent state and stages scratch, commit rolls the state to the accepted
    count;
  * "Speculative decoding" (mashbox docs, "Where it runs"): the copy-from-the-
    conversation drafter (n-gram prompt lookup).

Every dot product and reduction is accumulated in float64 and rounded once to
float32; values are rounded to bf16 exactly where a bf16 model stores them.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
this package.  It shares no code with the HIP path and imports nothing from it.
"""
from .numerics import bf16, f32, rmsnorm, rope, silu, sigmoid  # noqa: F401
from .philox import philox4x32_10, uniform01, accept_uniform, race_uniforms  # noqa: F401
from .planner import plan_drafts, plan_drafts_bruteforce  # noqa: F401
from .model import OracleModel, KVCache, RoundResult  # noqa: F401
from .accept import (  # noqa: F401
    row_stats, accept_greedy, accept_sampled, rule_outcomes, one_position_output,
)
from .ngram import ngram_draft, round_tokens, speculative_greedy_ngram  # noqa: F401
