"""Model shapes and round workloads used by tests and the benchmark.

Each entry is a decoder shape plus the round it is exercised with.  The shapes
follow the families the pages talk about (a tiny fp32 decoder, a 27B-class
dense decoder, a hybrid decoder whose recurrent layers carry a per-request
gated-delta-rule state); weights are random, never trained.
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str                      # "f32" or "bf16" (weights, KV and stored activations)
    layer_kinds: Tuple[str, ...]    # "attn" | "gdn" per layer
    gdn_heads: int = 0
    gdn_dim: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0     # 0.0 = no positional encoding
    kv_block: int = 16
    sliding_window: int = 0         # 0 = full attention; W > 0: a row sees its last W positions
    window_global_every: int = 0    # g > 0: attention layers g-1, 2g-1, ... keep full attention
    # round workload
    lanes: int = 1
    k: int = 3
    context: int = 0                # synthetic committed context per lane (0 = real prefill)
    prompt_len: int = 0
    rounds: int = 1
    modes: Tuple[str, ...] = ("greedy",)
    temperature: float = 1.0
    row_budget: int = 0
    seed_index: int = 0
    head_only: bool = False         # LM head + acceptance only (hidden states given)

    @property
    def n_attn(self) -> int:
        return sum(1 for s in self.layer_kinds if s == "attn")

    def layer_window(self, attn_index: int) -> int:
        """Window of the attention layer with this index among attention layers (0 = full)."""
        g = self.window_global_every
        if self.sliding_window <= 0 or (g > 0 and attn_index % g == g - 1):
            return 0
        return self.sliding_window

    @property
    def n_gdn(self) -> int:
        return sum(1 for s in self.layer_kinds if s == "gdn")

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads if self.n_kv_heads else 0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def gdn_in_rows(self) -> int:
        return 3 * self.gdn_heads * self.gdn_dim + 2 * self.gdn_heads

    @property
    def weight_seed(self) -> int:
        return 1000 + self.seed_index

    @property
    def input_seed(self) -> int:
        return 2000 + self.seed_index

    @property
    def philox_seed(self) -> int:
        return 3000 + self.seed_index

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


def _hybrid_kinds(n: int) -> Tuple[str, ...]:
    # three of every four layers are gated-delta-rule layers; every fourth is full GQA
    return tuple("attn" if i % 4 == 3 else "gdn" for i in range(n))


CONFIGS = {
    # tiny fp32 decoder, 1 lane, k=3, 64-token prompt, 16 greedy rounds
    "tiny-fp32": ModelConfig(
        name="tiny-fp32", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
        ffn=704, vocab=4096, dtype="f32", layer_kinds=("attn",) * 2,
        lanes=1, k=3, prompt_len=64, rounds=16, modes=("greedy",), seed_index=0),
    # LM head + acceptance only: 8 lanes x 8 rows, H 5120, V 151936
    "head-v151936": ModelConfig(
        name="head-v151936", n_layers=0, hidden=5120, n_q_heads=0, n_kv_heads=0, head_dim=0,
        ffn=0, vocab=151936, dtype="bf16", layer_kinds=(), lanes=8, k=7, context=4096,
        modes=("greedy", "sampled"), temperature=0.7, seed_index=1, head_only=True),
    # mid bf16 decoder, 8 layers, 4 lanes, k=4, context 2048 in paged KV
    "mid-bf16": ModelConfig(
        name="mid-bf16", n_layers=8, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
        ffn=5632, vocab=32768, dtype="bf16", layer_kinds=("attn",) * 8,
        lanes=4, k=4, context=2048, modes=("greedy", "sampled"), temperature=1.0,
        row_budget=8, seed_index=2),
    # 27B-class dense bf16 decoder, k=7 at 1 lane and 8 lanes, context 8192
    "dense-27b": ModelConfig(
        name="dense-27b", n_layers=64, hidden=5120, n_q_heads=40, n_kv_heads=8, head_dim=128,
        ffn=17408, vocab=151936, dtype="bf16", layer_kinds=("attn",) * 64,
        lanes=8, k=7, context=8192, modes=("greedy",), seed_index=3),
    # hybrid bf16 decoder, 48 layers (36 gated-delta-rule + 12 GQA), 4 lanes, k=3
    "hybrid-gdn": ModelConfig(
        name="hybrid-gdn", n_layers=48, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        ffn=12288, vocab=262144, dtype="bf16", layer_kinds=_hybrid_kinds(48),
        gdn_heads=16, gdn_dim=128, lanes=4, k=3, context=4096, modes=("greedy", "sampled"),
        seed_index=4),
}


def get_config(name: str, **overrides) -> ModelConfig:
    cfg = CONFIGS[name]
    if "n_layers" in overrides and "layer_kinds" not in overrides:
        n = overrides["n_layers"]
        if cfg.n_gdn:
            overrides["layer_kinds"] = _hybrid_kinds(n)
        else:
            overrides["layer_kinds"] = ("attn",) * n
    return cfg.with_(**overrides) if overrides else cfg
