"""The target decoder's forward over one verify round, and the commit.

What is computed follows "Speculative decoding" (gpillon.github.io/ignis),
section "One round, step by step", steps 1-5: every lane's columns (its anchor
plus its drafts) go through every layer once; then the state moves forward by
exactly the committed run -- attention layers keep the keys of every committed
column, recurrent layers replay only the committed prefix, and rejected
columns leave no trace.  The FreeToken tracking issue, "Per-request state",
fixes the split: verify reads the live state and stages scratch, commit rolls
the state forward to the accepted count.

Decoder (the layer list of the verify round): RMSNorm, then either GQA
attention over the lane's paged KV cache plus its own columns (causal among
them), or a gated-delta-rule recurrent layer; RMSNorm and a SwiGLU MLP; a
final RMSNorm and the LM head.  Positions: rotate-half RoPE on q and k at
absolute position kv_len + column.

Gated-delta-rule layer (Yang, Kautz & Hatamizadeh, "Gated Delta Networks"):
  alpha = sigmoid(h . w_alpha), beta = sigmoid(h . w_beta) per head,
  q = q~ / |q~| * d^-1/2, k = k~ / |k~|,
  S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,  o_t = S_t q_t.
The state is stored in float32 after every column, as the device stores it.

Precision: float64 arithmetic, one rounding to float32 per dot product or
reduction; a bf16 model's weights and KV cache hold bf16 values, so k and v
are rounded to bf16 as they are staged for the cache (see oracle.numerics).
"""
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

from .numerics import bf16, f32, store, rmsnorm, rope, sigmoid, silu

L2_EPS = 1e-6


def attend(q, keys, vals, n_ctx: int, window: int = 0) -> np.ndarray:
    """Grouped-query attention of one lane's columns (float64, exact two-pass softmax).

    q: [c, n_q, d] queries of columns 0..c-1; keys, vals: [n_ctx + c, n_kv, d]
    (committed context, then the lane's own columns).  Column j sees positions
    0 .. n_ctx + j (causal among its own columns); query head h reads kv head
    h // (n_q / n_kv); scores are scaled by 1/sqrt(d).

    Sliding-window targets (FreeToken issue, "Design": sliding-window targets; the
    Gemma 4 assistant thread): with window W > 0 column j sees only its last W
    positions, n_ctx + j - W + 1 .. n_ctx + j (itself included) -- the reading of a
    window of W positions that ends at the query.
    """
    c, nq, d = q.shape
    G = nq // keys.shape[1]
    kk = np.asarray(keys, np.float64)
    vv = np.asarray(vals, np.float64)
    out = np.zeros((c, nq, d), np.float64)
    scale = 1.0 / np.sqrt(d)
    for j in range(c):
        n_vis = n_ctx + j + 1
        lo = max(0, n_vis - window) if window > 0 else 0
        for hq in range(nq):
            g = hq // G
            s = kk[lo:n_vis, g, :] @ np.asarray(q[j, hq], np.float64) * scale
            s -= s.max()
            p = np.exp(s)
            p /= p.sum()
            out[j, hq] = p @ vv[lo:n_vis, g, :]
    return out


@dataclass
class KVCache:
    """Per-lane state that commit advances.

    kv_len[L]: committed length; the anchor of the next round sits at position kv_len.
    block_table[L, max_blocks]: token position p of lane l lives in block
        block_table[l, p // block], slot p % block.
    pool_k / pool_v: one float32 array [n_blocks, block, n_kv, d] per attention layer.
    gdn: one float32 array [L, heads, d_v, d_k] per gated-delta-rule layer.
    """
    kv_len: np.ndarray
    block_table: np.ndarray
    block: int
    pool_k: List[np.ndarray] = field(default_factory=list)
    pool_v: List[np.ndarray] = field(default_factory=list)
    gdn: List[np.ndarray] = field(default_factory=list)

    def copy(self) -> "KVCache":
        return KVCache(self.kv_len.copy(), self.block_table.copy(), self.block,
                       [a.copy() for a in self.pool_k], [a.copy() for a in self.pool_v],
                       [a.copy() for a in self.gdn])

    def gather(self, li: int, lane: int, length: int):
        """Committed K and V of `lane` for attention layer li: [length, n_kv, d] each."""
        p = np.arange(length)
        blk = self.block_table[lane, p // self.block]
        slot = p % self.block
        return self.pool_k[li][blk, slot], self.pool_v[li][blk, slot]

    def scatter(self, li: int, lane: int, start: int, k_rows, v_rows):
        p = start + np.arange(k_rows.shape[0])
        blk = self.block_table[lane, p // self.block]
        slot = p % self.block
        self.pool_k[li][blk, slot] = k_rows
        self.pool_v[li][blk, slot] = v_rows


@dataclass
class RoundResult:
    logits: np.ndarray                 # [R, V] float32
    hidden: np.ndarray                 # [R, H] final normed hidden (float32)
    row_lane: np.ndarray               # [R]
    row_col: np.ndarray                # [R]
    lane_rows: List[range]             # rows of each lane
    staged_k: List[np.ndarray]         # per attention layer [R, n_kv, d]
    staged_v: List[np.ndarray]
    gdn_staged: List[Dict[str, np.ndarray]]   # per gdn layer: k [R,h,d], v [R,h,d], alpha [R,h], beta [R,h]


class OracleModel:
    """cfg: any object with the shape attributes of a decoder config.

    weights: dict with "embed", "lm_head", "final_norm" and either "layers" (a
    list of per-layer dicts) or "layer_fn" (a callable i -> dict, so that a big
    model can be streamed layer by layer).  Arrays hold float32 values that are
    exactly representable at the model's storage precision.
    """

    def __init__(self, cfg, weights: Dict[str, object], keep_f64: bool = True):
        self.cfg = cfg
        self.w = weights
        self.dtype = cfg.dtype
        # float64 copies of resident weight matrices, made once (a streamed model keeps none)
        self._f64 = {} if keep_f64 and "layers" in weights else None

    # ------------------------------------------------------------------ helpers
    def _layer(self, i: int) -> Dict[str, np.ndarray]:
        if "layers" in self.w:
            return self.w["layers"][i]
        return self.w["layer_fn"](i)

    def _st(self, x) -> np.ndarray:
        """Storage precision of the KV cache (the model's dtype)."""
        return store(x, self.dtype)

    @staticmethod
    def _act(x) -> np.ndarray:
        """Activations are float32 values."""
        return f32(x)

    def _w64(self, w) -> np.ndarray:
        if self._f64 is None:
            return np.asarray(w, np.float64)
        key = id(w)
        hit = self._f64.get(key)
        if hit is None or hit[0] is not w:
            hit = (w, np.asarray(w, np.float64))
            self._f64[key] = hit
        return hit[1]

    def _matT(self, x, w) -> np.ndarray:
        """float32(x @ w.T) with float64 accumulation."""
        return f32(np.asarray(x, np.float64) @ self._w64(w).T)

    def lm_head(self, hidden) -> np.ndarray:
        return self._matT(hidden, self.w["lm_head"])

    # ------------------------------------------------------------------ forward
    def verify_round(self, cache: KVCache, lane_tokens: Sequence[Sequence[int]]) -> RoundResult:
        """Run every lane's columns (anchor then drafts) through the model once.

        Reads the live cache and state; writes neither.
        """
        cfg = self.cfg
        L = len(lane_tokens)
        cols = [len(t) for t in lane_tokens]
        assert all(c >= 1 for c in cols)
        lane_rows, r0 = [], 0
        for c in cols:
            lane_rows.append(range(r0, r0 + c))
            r0 += c
        R = r0
        row_lane = np.concatenate([np.full(c, l) for l, c in enumerate(cols)]).astype(np.int64)
        row_col = np.concatenate([np.arange(c) for c in cols]).astype(np.int64)
        pos = cache.kv_len[row_lane].astype(np.int64) + row_col
        tokens = np.concatenate([np.asarray(t, np.int64) for t in lane_tokens])

        x = np.asarray(self.w["embed"], np.float32)[tokens].astype(np.float32)   # [R, H]
        staged_k, staged_v, gdn_staged = [], [], []
        ia = ig = 0
        for i in range(cfg.n_layers):
            lw = self._layer(i)
            h = self._act(rmsnorm(x, lw["norm1"], cfg.rms_eps))
            if cfg.layer_kinds[i] == "attn":
                o, k, v = self._attention(h, lw, ia, cache, lane_rows, pos)
                staged_k.append(k)
                staged_v.append(v)
                ia += 1
            else:
                o, st = self._gdn(h, lw, ig, cache, lane_rows)
                gdn_staged.append(st)
                ig += 1
            x = f32(x.astype(np.float64) + self._matT(o, lw["w_o"]))
            h2 = self._act(rmsnorm(x, lw["norm2"], cfg.rms_eps))
            g = self._matT(h2, lw["w_gate"])
            u = self._matT(h2, lw["w_up"])
            a = self._act(silu(g) * u.astype(np.float64))
            x = f32(x.astype(np.float64) + self._matT(a, lw["w_down"]))
        hf = self._act(rmsnorm(x, self.w["final_norm"], cfg.rms_eps))
        logits = self.lm_head(hf)
        return RoundResult(logits, hf, row_lane, row_col, lane_rows, staged_k, staged_v, gdn_staged)

    def _attention(self, h, lw, li, cache: KVCache, lane_rows, pos):
        cfg = self.cfg
        nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        G = nq // nkv
        R = h.shape[0]
        y = self._matT(h, lw["w_in"])
        q = y[:, : nq * d].reshape(R, nq, d)
        k = y[:, nq * d: (nq + nkv) * d].reshape(R, nkv, d)
        v = y[:, (nq + nkv) * d:].reshape(R, nkv, d)
        q = self._act(rope(q, pos, cfg.rope_theta))
        k = self._st(rope(k, pos, cfg.rope_theta))     # staged for the cache
        v = self._st(v)
        o = np.zeros((R, nq, d), np.float64)
        for l, rows in enumerate(lane_rows):
            n_ctx = int(cache.kv_len[l])
            ck, cv = cache.gather(li, l, n_ctx)
            keys = np.concatenate([ck, k[rows.start:rows.stop]], axis=0)
            vals = np.concatenate([cv, v[rows.start:rows.stop]], axis=0)
            o[rows.start:rows.stop] = attend(q[rows.start:rows.stop], keys, vals, n_ctx, cfg.layer_window(li))
        return self._act(o).reshape(R, nq * d), k, v

    def _gdn_inputs(self, h, lw):
        cfg = self.cfg
        hg, dg = cfg.gdn_heads, cfg.gdn_dim
        R = h.shape[0]
        y = self._matT(h, lw["w_in"]).astype(np.float64)
        qt = y[:, : hg * dg].reshape(R, hg, dg)
        kt = y[:, hg * dg: 2 * hg * dg].reshape(R, hg, dg)
        v = f32(y[:, 2 * hg * dg: 3 * hg * dg].reshape(R, hg, dg))
        alpha = f32(sigmoid(y[:, 3 * hg * dg: 3 * hg * dg + hg]))
        beta = f32(sigmoid(y[:, 3 * hg * dg + hg: 3 * hg * dg + 2 * hg]))
        qn = f32(qt / np.sqrt((qt * qt).sum(-1, keepdims=True) + L2_EPS) / np.sqrt(dg))
        kn = f32(kt / np.sqrt((kt * kt).sum(-1, keepdims=True) + L2_EPS))
        return qn, kn, v, alpha, beta

    @staticmethod
    def gdn_step(S, k, v, alpha, beta):
        """One column of the gated delta rule on a float32 state [h, d_v, d_k]; returns float32."""
        S = S.astype(np.float64)
        a = alpha.astype(np.float64)[:, None, None]
        b = beta.astype(np.float64)[:, None, None]
        kk = k.astype(np.float64)
        Sk = np.einsum("hij,hj->hi", S, kk)                      # S_{t-1} k_t
        delta = v.astype(np.float64) - a[:, :, 0] * Sk          # v_t - alpha S k
        return f32(a * S + b * delta[:, :, None] * kk[:, None, :])

    def _gdn(self, h, lw, gi, cache: KVCache, lane_rows):
        cfg = self.cfg
        hg, dg = cfg.gdn_heads, cfg.gdn_dim
        R = h.shape[0]
        qn, kn, v, alpha, beta = self._gdn_inputs(h, lw)
        o = np.zeros((R, hg, dg), np.float64)
        for l, rows in enumerate(lane_rows):
            S = cache.gdn[gi][l]
            for r in rows:
                S = self.gdn_step(S, kn[r], v[r], alpha[r], beta[r])
                o[r] = np.einsum("hij,hj->hi", S.astype(np.float64), qn[r].astype(np.float64))
        o = f32(o).reshape(R, hg * dg)
        return o, {"q": qn, "k": kn, "v": v, "alpha": alpha, "beta": beta}

    # ------------------------------------------------------------------ commit
    def commit(self, cache: KVCache, res: RoundResult, committed: Sequence[int]) -> None:
        """Advance each lane by exactly its committed run (columns 0..c-1)."""
        for l, rows in enumerate(res.lane_rows):
            c = int(committed[l])
            assert 1 <= c <= len(rows), "committed run must lie in [1, columns]"
            start = int(cache.kv_len[l])
            sel = slice(rows.start, rows.start + c)
            for li in range(len(res.staged_k)):
                cache.scatter(li, l, start, res.staged_k[li][sel], res.staged_v[li][sel])
            for gi, st in enumerate(res.gdn_staged):
                S = cache.gdn[gi][l]
                for r in range(rows.start, rows.start + c):
                    S = self.gdn_step(S, st["k"][r], st["v"][r], st["alpha"][r], st["beta"][r])
                cache.gdn[gi][l] = S
            cache.kv_len[l] += c

    # ------------------------------------------------------------------ plain decoding
    def plain_greedy(self, cache: KVCache, anchors: Sequence[int], n_steps: int) -> np.ndarray:
        """Plain autoregressive greedy decoding: one column per lane per step.

        Returns tokens [L, n_steps]: the token chosen after each step (the first
        is the model's token after the anchor).  Mutates `cache`.
        """
        from .accept import argmax_lowest
        cur = [int(a) for a in anchors]
        out = np.zeros((len(cur), n_steps), np.int64)
        for s in range(n_steps):
            res = self.verify_round(cache, [[t] for t in cur])
            nxt = [int(argmax_lowest(res.logits[r])) for r in range(len(cur))]
            self.commit(cache, res, [1] * len(cur))
            out[:, s] = nxt
            cur = nxt
        return out

    def prefill(self, cache: KVCache, lane_prompts: Sequence[Sequence[int]], chunk: int) -> None:
        """Teacher-forced rounds: all prompt tokens but the last become committed context.

        The last prompt token is left as the lane's anchor.
        """
        L = len(lane_prompts)
        done = [0] * L
        while True:
            toks, lanes = [], []
            for l, p in enumerate(lane_prompts):
                n = len(p) - 1 - done[l]
                if n > 0:
                    toks.append(list(p[done[l]: done[l] + min(n, chunk)]))
            if not toks:
                return
            assert len(toks) == L, "prefill expects equal-length prompts"
            res = self.verify_round(cache, toks)
            self.commit(cache, res, [len(t) for t in toks])
            for l in range(L):
                done[l] += len(toks[l])
