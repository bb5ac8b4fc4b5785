"""Seeded generators.  Every function is a pure function of (config, seed, ids).

Numbers are produced on the host with numpy's PCG64 so that the oracle and the
GPU path see the same values; values that a bf16 model stores in bf16 are
rounded by torch's bfloat16 conversion and handed out as float32 arrays that
hold bf16-representable values.
"""
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from .configs import ModelConfig

WEIGHT_STD = 0.02

# tensor ids (part of the recipe: changing them changes every weight)
TID_EMBED = 0
TID_LM_HEAD = 1
TID_LAYER_BASE = 100
TID_PER_LAYER = 16
TIDX_IN, TIDX_O, TIDX_GATE, TIDX_UP, TIDX_DOWN = 0, 1, 2, 3, 4


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, ids)])))


def _to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    return a


def _normal(seed: int, tid: int, shape, std: float, dtype: str) -> np.ndarray:
    a = _rng(seed, tid).standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return _to_storage(a, dtype)


def head_weights(cfg: ModelConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Embedding [V, H], LM head [V, H] (untied) and the final norm gain [H]."""
    seed = cfg.weight_seed if seed is None else seed
    out = {
        "lm_head": _normal(seed, TID_LM_HEAD, (cfg.vocab, cfg.hidden), WEIGHT_STD, cfg.dtype),
        "final_norm": np.ones(cfg.hidden, np.float32),
    }
    if not cfg.head_only:
        out["embed"] = _normal(seed, TID_EMBED, (cfg.vocab, cfg.hidden), WEIGHT_STD, cfg.dtype)
    return out


def layer_weights(cfg: ModelConfig, i: int, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """One decoder layer, row-major [out, in].

    Full-attention layer: w_in rows are q heads, then k heads, then v heads.
    Gated-delta-rule layer: w_in rows are q, k, v (heads x dim each), then the
    per-head alpha and beta rows.
    """
    seed = cfg.weight_seed if seed is None else seed
    base = TID_LAYER_BASE + TID_PER_LAYER * i
    H, F = cfg.hidden, cfg.ffn
    kind = cfg.layer_kinds[i]
    if kind == "attn":
        n_in, n_o = cfg.qkv_rows, cfg.n_q_heads * cfg.head_dim
    else:
        n_in, n_o = cfg.gdn_in_rows, cfg.gdn_heads * cfg.gdn_dim
    return {
        "kind": kind,
        "norm1": np.ones(H, np.float32),
        "w_in": _normal(seed, base + TIDX_IN, (n_in, H), WEIGHT_STD, cfg.dtype),
        "w_o": _normal(seed, base + TIDX_O, (H, n_o), WEIGHT_STD, cfg.dtype),
        "norm2": np.ones(H, np.float32),
        "w_gate": _normal(seed, base + TIDX_GATE, (F, H), WEIGHT_STD, cfg.dtype),
        "w_up": _normal(seed, base + TIDX_UP, (F, H), WEIGHT_STD, cfg.dtype),
        "w_down": _normal(seed, base + TIDX_DOWN, (H, F), WEIGHT_STD, cfg.dtype),
    }


def model_weights(cfg: ModelConfig, seed: Optional[int] = None) -> Dict[str, object]:
    w = dict(head_weights(cfg, seed))
    w["layers"] = [layer_weights(cfg, i, seed) for i in range(cfg.n_layers)]
    return w


def uniform_tokens(seed: int, tag: int, n: int, vocab: int) -> np.ndarray:
    return _rng(seed, 7, tag).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def prompt_tokens(cfg: ModelConfig, lane: int = 0) -> np.ndarray:
    return uniform_tokens(cfg.input_seed, 1000 + lane, cfg.prompt_len, cfg.vocab)


def kv_context(cfg: ModelConfig, attn_layer: int, lane: int, length: Optional[int] = None):
    """Synthetic committed K and V of one lane for one full-attention layer.

    Returns (K, V), each float32 [length, n_kv, head_dim], values ~ N(0, 1)
    stored at the model's precision.
    """
    length = cfg.context if length is None else length
    shape = (length, cfg.n_kv_heads, cfg.head_dim)
    r = _rng(cfg.input_seed, 11, attn_layer, lane)
    k = _to_storage(r.standard_normal(size=shape, dtype=np.float32), cfg.dtype)
    v = _to_storage(r.standard_normal(size=shape, dtype=np.float32), cfg.dtype)
    return k, v


def block_table(cfg: ModelConfig, lanes: int, blocks_per_lane: int, extra_blocks: int = 3) -> np.ndarray:
    """Randomly permuted page assignment: lane l owns blocks table[l, :]."""
    n_blocks = lanes * blocks_per_lane + extra_blocks
    perm = _rng(cfg.input_seed, 12).permutation(n_blocks).astype(np.int32)
    return perm[: lanes * blocks_per_lane].reshape(lanes, blocks_per_lane).copy(), n_blocks


def gdn_state(cfg: ModelConfig, gdn_layer: int, lane: int) -> np.ndarray:
    """Initial recurrent state [heads, dim_v, dim_k] fp32, entries ~ N(0, 1/128) (variance)."""
    shape = (cfg.gdn_heads, cfg.gdn_dim, cfg.gdn_dim)
    a = _rng(cfg.input_seed, 13, gdn_layer, lane).standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(1.0 / np.sqrt(128.0))
    return a


def drafter_rows(seed: int, tag: int, n_rows: int, vocab: int, logit_std: float = 2.0):
    """Drafter distributions q (softmax of N(0, logit_std) logits) and a draft drawn from each.

    Returns (q [n_rows, vocab] float32, drafts [n_rows] int32).  The draw uses
    numpy's generator: the drafter is an input to the verify round, not part of it.
    """
    r = _rng(seed, 17, tag)
    z = r.standard_normal(size=(n_rows, vocab), dtype=np.float32).astype(np.float64) * logit_std
    z -= z.max(axis=1, keepdims=True)
    e = np.exp(z)
    q = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    qd = q.astype(np.float64)
    qd /= qd.sum(axis=1, keepdims=True)
    u = r.random(size=n_rows)
    cdf = np.cumsum(qd, axis=1)
    d = np.minimum((cdf < u[:, None]).sum(axis=1), vocab - 1).astype(np.int32)
    return q, d


def planted_drafts(seed: int, tag: int, reference: Sequence[int], alpha, vocab: int) -> np.ndarray:
    """Drafts that equal the reference token with probability alpha[i] (i.i.d. per slot),
    otherwise a uniform token different from the reference."""
    ref = np.asarray(reference, dtype=np.int64)
    n = ref.shape[0]
    a = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (n,))
    r = _rng(seed, 19, tag)
    hit = r.random(size=n) < a
    other = r.integers(0, vocab - 1, size=n)
    other = other + (other >= ref)      # uniform over tokens != ref
    return np.where(hit, ref, other).astype(np.int32)


def hidden_states(cfg: ModelConfig, rows: int, tag: int = 0) -> np.ndarray:
    """Final hidden states [rows, hidden] ~ N(0, 1) at the model's precision (LM-head-only rounds)."""
    a = _rng(cfg.input_seed, 23, tag).standard_normal(size=(rows, cfg.hidden), dtype=np.float32)
    return _to_storage(a, cfg.dtype)
