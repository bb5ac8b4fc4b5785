"""Pins of the oracle decoder against library routines, closed forms and invariants."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import synth
from helpers import oracle_cache, small_dense, small_hybrid
from oracle import OracleModel, accept_greedy, f32, rmsnorm, rope, row_stats
from oracle.accept import argmax_lowest
from oracle.model import attend


# ---------------------------------------------------------------- element pieces
def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    g = rng.standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(1)
    d, theta = 64, 10000.0
    x = rng.standard_normal((3, 2, d))
    pos = np.array([0, 5, 8191])
    got = rope(x, pos, theta)
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = 1.0 / theta ** (np.arange(half) * 2.0 / d)
    zr = z * np.exp(1j * pos[:, None, None] * freq)
    assert np.allclose(got, np.concatenate([zr.real, zr.imag], -1), atol=1e-12)
    assert np.allclose(rope(x, np.zeros(3), theta), x)                    # position 0: identity
    assert np.allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.array_equal(rope(x, pos, 0.0), x)                            # theta 0: no encoding


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((1, 1, 32)), rng.standard_normal((1, 1, 32))
    dots = [float((rope(q, np.array([m]), 1e4) * rope(k, np.array([n]), 1e4)).sum())
            for m, n in [(10, 3), (107, 100), (7, 0)]]
    assert np.allclose(dots, dots[0], atol=1e-12)


@pytest.mark.parametrize("n_ctx,c,nq,nkv", [(0, 1, 4, 2), (0, 4, 4, 4), (37, 5, 8, 2), (130, 8, 5, 1)])
def test_attend_matches_sdpa(n_ctx, c, nq, nkv):
    rng = np.random.default_rng(n_ctx + c)
    d = 16
    q = rng.standard_normal((c, nq, d))
    keys = rng.standard_normal((n_ctx + c, nkv, d))
    vals = rng.standard_normal((n_ctx + c, nkv, d))
    got = attend(q, keys, vals, n_ctx)
    # library routine: boolean mask, kv heads repeated for the query groups
    G = nq // nkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                               # [nq, c, d]
    kt = torch.from_numpy(keys).repeat_interleave(G, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(vals).repeat_interleave(G, dim=1).permute(1, 0, 2)
    mask = torch.arange(n_ctx + c)[None, :] <= (n_ctx + torch.arange(c))[:, None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).permute(1, 0, 2).numpy()
    assert np.allclose(got, ref, atol=1e-12)


def test_attend_first_column_without_context_is_its_value():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 4, 8))
    kv = rng.standard_normal((3, 2, 8))
    vv = rng.standard_normal((3, 2, 8))
    o = attend(q, kv, vv, 0)
    assert np.array_equal(o[0], np.repeat(vv[0], 2, axis=0))


# ---------------------------------------------------------------- gated delta rule
def test_gdn_special_cases():
    rng = np.random.default_rng(4)
    h, d = 2, 8
    S = rng.standard_normal((h, d, d)).astype(np.float32)
    k = rng.standard_normal((h, d)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    v = rng.standard_normal((h, d)).astype(np.float32)
    a = np.array([0.7, 0.3], np.float32)
    # beta = 0: pure decay
    S1 = OracleModel.gdn_step(S, k, v, a, np.zeros(2, np.float32))
    assert np.array_equal(S1, f32(a.astype(np.float64)[:, None, None] * S))
    # alpha = beta = 1, |k| = 1: the delta rule overwrites the value stored under k
    S2 = OracleModel.gdn_step(S, k, v, np.ones(2, np.float32), np.ones(2, np.float32))
    assert np.allclose(np.einsum("hij,hj->hi", S2.astype(np.float64), k.astype(np.float64)), v, atol=1e-5)


def test_gdn_step_matches_product_form():
    # S_t = S_{t-1} (alpha (I - beta k k^T)) + beta v k^T  (the gated delta rule's matrix form)
    rng = np.random.default_rng(5)
    h, d = 3, 6
    S = rng.standard_normal((h, d, d)).astype(np.float32)
    k = rng.standard_normal((h, d)).astype(np.float32)
    v = rng.standard_normal((h, d)).astype(np.float32)
    a = rng.random(h).astype(np.float32)
    b = rng.random(h).astype(np.float32)
    got = OracleModel.gdn_step(S, k, v, a, b)
    for i in range(h):
        kk = k[i].astype(np.float64)[:, None]
        M = a[i] * (np.eye(d) - b[i] * kk @ kk.T)
        ref = S[i].astype(np.float64) @ M + b[i] * v[i].astype(np.float64)[:, None] @ kk.T
        assert np.allclose(got[i], ref, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- LM head statistics
def test_row_stats_bruteforce():
    rng = np.random.default_rng(6)
    z = (rng.standard_normal((6, 300)) * 3).astype(np.float32)
    z[2, 10] = z[2, 20] = z[2].max() + 1                                   # tie: lowest index wins
    nxt = np.array([5, -1, 7, 0, 299, 3])
    for T in (1.0, 0.7):
        s = row_stats(z, nxt, T)
        assert np.allclose(s["lse"], logsumexp(z.astype(np.float64) / T, axis=1), rtol=1e-14)
        assert np.array_equal(s["max"], z.max(axis=1))
        assert np.array_equal(s["argmax"], [np.argmax(r) for r in z])
        assert s["argmax"][2] == 10
        assert np.isnan(s["z_next"][1]) and s["z_next"][4] == z[4, 299]


# ---------------------------------------------------------------- whole-model invariants
def _model(cfg):
    return OracleModel(cfg, synth.model_weights(cfg))


def test_forward_matches_library_reference_tiny_fp32():
    """One round of a 2-layer fp32 decoder vs a forward written with torch's own routines."""
    cfg = synth.get_config("tiny-fp32")
    w = synth.model_weights(cfg)
    m = OracleModel(cfg, w)
    cache = oracle_cache(cfg, 1, 19, 4)
    toks = [[5, 17, 300, 4095]]
    res = m.verify_round(cache, toks)
    # reference in torch float64: rms_norm, SDPA with a causal-over-own-columns mask, silu
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    x = t(w["embed"])[torch.tensor(toks[0])]
    nq, nkv, d, H = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    pos = torch.arange(19, 23, dtype=torch.float64)
    inv = 1.0 / cfg.rope_theta ** (torch.arange(0, d // 2, dtype=torch.float64) * 2 / d)
    ang = pos[:, None] * inv
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def rope_t(a):
        z = torch.complex(a[..., : d // 2], a[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], -1)

    for i, lw in enumerate(w["layers"]):
        h = F.rms_norm(x, (H,), t(lw["norm1"]), eps=cfg.rms_eps)
        y = h @ t(lw["w_in"]).T
        q = rope_t(y[:, : nq * d].reshape(4, nq, d))
        k = rope_t(y[:, nq * d:(nq + nkv) * d].reshape(4, nkv, d))
        v = y[:, (nq + nkv) * d:].reshape(4, nkv, d)
        ck, cv = cache.gather(i, 0, 19)
        K = torch.cat([t(ck), k]).repeat_interleave(nq // nkv, 1).permute(1, 0, 2)
        Vv = torch.cat([t(cv), v]).repeat_interleave(nq // nkv, 1).permute(1, 0, 2)
        mask = torch.arange(23)[None, :] <= (19 + torch.arange(4))[:, None]
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2), K, Vv, attn_mask=mask).permute(1, 0, 2)
        x = x + o.reshape(4, nq * d) @ t(lw["w_o"]).T
        h2 = F.rms_norm(x, (H,), t(lw["norm2"]), eps=cfg.rms_eps)
        x = x + (F.silu(h2 @ t(lw["w_gate"]).T) * (h2 @ t(lw["w_up"]).T)) @ t(lw["w_down"]).T
    z = F.rms_norm(x, (H,), t(w["final_norm"]), eps=cfg.rms_eps) @ t(w["lm_head"]).T
    assert np.max(np.abs(res.logits - z.numpy())) < 1e-5


@pytest.mark.parametrize("make", [small_dense, small_hybrid])
def test_causal_over_own_columns(make):
    cfg = make()
    m = _model(cfg)
    cache = oracle_cache(cfg, 1, cfg.context, 8)
    a = m.verify_round(cache, [[3, 9, 27, 81, 100]])
    b = m.verify_round(cache, [[3, 9, 27, 500, 1]])          # drafts after column 2 differ
    assert np.array_equal(a.logits[:3], b.logits[:3])
    assert not np.array_equal(a.logits[3:], b.logits[3:])


@pytest.mark.parametrize("make", [small_dense, small_hybrid])
def test_verify_reads_but_never_writes_state(make):
    cfg = make()
    m = _model(cfg)
    cache = oracle_cache(cfg, 2, cfg.context, 8)
    before = cache.copy()
    m.verify_round(cache, [[1, 2, 3], [4, 5]])
    for x, y in zip(before.pool_k + before.pool_v + before.gdn, cache.pool_k + cache.pool_v + cache.gdn):
        assert np.array_equal(x, y)
    assert np.array_equal(before.kv_len, cache.kv_len)


@pytest.mark.parametrize("make", [small_dense, small_hybrid])
def test_commit_equals_plain_steps(make):
    """verify + commit(c) leaves the same cache and recurrent state as c plain one-column steps."""
    cfg = make()
    m = _model(cfg)
    toks = [7, 8, 9, 10]
    for c in (1, 3, 4):
        ca = oracle_cache(cfg, 1, cfg.context, 8)
        res = m.verify_round(ca, [toks])
        m.commit(ca, res, [c])
        cb = oracle_cache(cfg, 1, cfg.context, 8)
        for t in toks[:c]:
            rb = m.verify_round(cb, [[t]])
            m.commit(cb, rb, [1])
        assert ca.kv_len[0] == cb.kv_len[0] == cfg.context + c
        for x, y in zip(ca.pool_k + ca.pool_v, cb.pool_k + cb.pool_v):
            assert np.allclose(x, y, rtol=0, atol=1e-2 if cfg.dtype == "bf16" else 1e-6)
            assert np.mean(x == y) > 0.999
        for x, y in zip(ca.gdn, cb.gdn):
            assert np.allclose(x, y, rtol=1e-5, atol=1e-6)


def test_commit_compaction_and_untouched_rows():
    cfg = small_dense()
    m = _model(cfg)
    cache = oracle_cache(cfg, 2, 21, 8)
    before = cache.copy()
    res = m.verify_round(cache, [[1, 2, 3, 4], [5, 6]])
    m.commit(cache, res, [2, 1])
    for li in range(cfg.n_attn):
        for l, (rows, c) in enumerate(zip(res.lane_rows, [2, 1])):
            k, v = cache.gather(li, l, 21 + c)
            assert np.array_equal(k[21:], res.staged_k[li][rows.start:rows.start + c])
            assert np.array_equal(v[21:], res.staged_v[li][rows.start:rows.start + c])
        touched = np.zeros(cache.pool_k[li].shape[:2], bool)
        for l, c in enumerate([2, 1]):
            for p in range(21, 21 + c):
                touched[cache.block_table[l, p // 16], p % 16] = True
        assert np.array_equal(cache.pool_k[li][~touched], before.pool_k[li][~touched])
        assert np.array_equal(cache.pool_v[li][~touched], before.pool_v[li][~touched])


def test_lanes_do_not_interact():
    cfg = small_hybrid()
    m = _model(cfg)
    cache = oracle_cache(cfg, 2, cfg.context, 8)
    both = m.verify_round(cache, [[1, 2, 3], [4, 5, 6, 7]])
    c1 = cache.copy()
    c1.kv_len = c1.kv_len[1:]
    c1.block_table = c1.block_table[1:]
    c1.gdn = [g[1:] for g in c1.gdn]
    alone = m.verify_round(c1, [[4, 5, 6, 7]])
    assert np.allclose(both.logits[3:], alone.logits, atol=1e-4)
    assert [argmax_lowest(r) for r in both.logits[3:]] == [argmax_lowest(r) for r in alone.logits]


def test_speculative_greedy_equals_plain_greedy_tiny():
    """16 greedy verify rounds (k=3) commit exactly the plain greedy continuation."""
    cfg = synth.get_config("tiny-fp32")
    m = _model(cfg)
    prompt = synth.prompt_tokens(cfg)
    base = oracle_cache(cfg, 1, 0, 16)
    m.prefill(base, [prompt], chunk=16)
    assert base.kv_len[0] == 63
    ref = m.plain_greedy(base.copy(), [prompt[-1]], 16 * 4 + 4)[0]
    spec = base.copy()
    anchor, out = int(prompt[-1]), []
    rng = np.random.default_rng(20)
    for rnd in range(16):
        P = len(out)
        drafts = [int(ref[P + i]) if rng.random() < 0.7 else int(rng.integers(0, cfg.vocab))
                  for i in range(cfg.k)]
        res = m.verify_round(spec, [[anchor] + drafts])
        c, emitted = accept_greedy(res.logits, drafts)
        assert 1 <= c <= cfg.k + 1
        m.commit(spec, res, [c])
        out += emitted
        anchor = emitted[-1]
    assert out == [int(t) for t in ref[: len(out)]]
    assert spec.kv_len[0] == 63 + len(out)


def test_gdn_layer_matches_library_reference():
    """A 1-layer fp32 gated-delta-rule decoder vs torch routines (F.normalize, sigmoid,
    the rule's matrix form), over a lane's columns starting from the live state."""
    cfg = small_hybrid(n_layers=1, layer_kinds=("gdn",), dtype="f32")
    w = synth.model_weights(cfg)
    m = OracleModel(cfg, w)
    cache = oracle_cache(cfg, 1, 0, 4)
    toks = [11, 22, 33]
    res = m.verify_round(cache, [toks])
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    hg, dg, H = cfg.gdn_heads, cfg.gdn_dim, cfg.hidden
    lw = w["layers"][0]
    x = t(w["embed"])[torch.tensor(toks)]
    h = F.rms_norm(x, (H,), t(lw["norm1"]), eps=cfg.rms_eps)
    y = h @ t(lw["w_in"]).T
    q = F.normalize(y[:, :hg * dg].reshape(3, hg, dg), dim=-1) / dg ** 0.5
    k = F.normalize(y[:, hg * dg:2 * hg * dg].reshape(3, hg, dg), dim=-1)
    v = y[:, 2 * hg * dg:3 * hg * dg].reshape(3, hg, dg)
    al = torch.sigmoid(y[:, 3 * hg * dg:3 * hg * dg + hg])
    be = torch.sigmoid(y[:, 3 * hg * dg + hg:])
    S = t(cache.gdn[0][0])
    outs = []
    for j in range(3):
        S = torch.stack([S[i] @ (al[j, i] * (torch.eye(dg, dtype=torch.float64)
                                             - be[j, i] * torch.outer(k[j, i], k[j, i])))
                         + be[j, i] * torch.outer(v[j, i], k[j, i]) for i in range(hg)])
        outs.append(torch.einsum("hij,hj->hi", S, q[j]))
    o = torch.stack(outs).reshape(3, hg * dg)
    x = x + o @ t(lw["w_o"]).T
    h2 = F.rms_norm(x, (H,), t(lw["norm2"]), eps=cfg.rms_eps)
    x = x + (F.silu(h2 @ t(lw["w_gate"]).T) * (h2 @ t(lw["w_up"]).T)) @ t(lw["w_down"]).T
    z = F.rms_norm(x, (H,), t(w["final_norm"]), eps=cfg.rms_eps) @ t(w["lm_head"]).T
    assert np.max(np.abs(res.logits - z.numpy())) < 1e-4
