"""Test helpers shared by the CPU and GPU tests: building oracle-side state from synth inputs."""
import numpy as np

import synth
from synth.configs import ModelConfig


def small_hybrid(**kw) -> ModelConfig:
    """A small bf16 hybrid decoder (3 gated-delta-rule layers + 1 GQA layer per 4)."""
    base = dict(name="small-hybrid", n_layers=4, hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32,
                ffn=256, vocab=512, dtype="bf16",
                layer_kinds=("gdn", "gdn", "gdn", "attn"), gdn_heads=2, gdn_dim=32,
                lanes=2, k=3, context=40, seed_index=7)
    base.update(kw)
    return ModelConfig(**base)


def small_dense(**kw) -> ModelConfig:
    base = dict(name="small-dense", n_layers=2, hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32,
                ffn=256, vocab=512, dtype="bf16", layer_kinds=("attn", "attn"),
                lanes=2, k=3, context=37, seed_index=8)
    base.update(kw)
    return ModelConfig(**base)


def oracle_cache(cfg: ModelConfig, lanes: int, context: int, blocks_per_lane: int):
    """Oracle KVCache holding `context` synthetic committed tokens per lane."""
    from oracle import KVCache
    bt, n_blocks = synth.block_table(cfg, lanes, blocks_per_lane)
    cache = KVCache(kv_len=np.full(lanes, context, np.int64), block_table=bt.astype(np.int64),
                    block=cfg.kv_block)
    for li in range(cfg.n_attn):
        pk = np.zeros((n_blocks, cfg.kv_block, cfg.n_kv_heads, cfg.head_dim), np.float32)
        pv = np.zeros_like(pk)
        cache.pool_k.append(pk)
        cache.pool_v.append(pv)
        for l in range(lanes):
            if context:
                k, v = synth.kv_context(cfg, li, l, context)
                cache.scatter(li, l, 0, k, v)
    for gi in range(cfg.n_gdn):
        cache.gdn.append(np.stack([synth.gdn_state(cfg, gi, l) for l in range(lanes)]))
    return cache
