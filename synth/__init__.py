"""Seeded synthetic inputs for the speculative-decoding verify round.

This module is shared by the oracle side (tests, the CPU baseline) and the GPU
side (tests, bench, smoke).  It holds model *shapes* and random-number recipes
only: no step of the verify round's arithmetic lives here.  Values destined for
bf16 storage are rounded with torch's own bfloat16 conversion (a library
primitive), so nothing here duplicates the oracle's rounding code or the
kernels'.

Recipes (the pages give model families and sizes, not data):
  * every matrix ~ N(0, 0.02) (standard deviation), drawn per tensor from
    numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id]))),
    then rounded to bf16 for bf16 models; norm gains are 1.0;
  * synthetic KV context ~ N(0, 1), placed in randomly permuted pages;
  * gated-delta-rule initial state ~ N(0, 1/128);
  * drafter distributions q = softmax of N(0, 2) logits, draft ~ q.
"""
from .configs import CONFIGS, ModelConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    model_weights, layer_weights, head_weights, prompt_tokens, kv_context,
    block_table, gdn_state, drafter_rows, planted_drafts, uniform_tokens, hidden_states,
)
