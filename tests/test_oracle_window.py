"""Pins of sliding-window attention in the oracle (a row sees its last W positions).

Checked against what fixes it independently: a window at least as long as what a row
can see is full attention; a window of one position returns the row's own value
vector; each row equals full attention over the context cut to its window (the
definition of the window as a truncation); per-layer windows follow the global-layer
rule; and speculative greedy decoding of a windowed model commits its plain greedy
continuation, which differs from the full-attention model's.
"""
import numpy as np

import synth
from helpers import oracle_cache
from oracle import OracleModel, accept_greedy
from oracle.model import attend


def _qkv(seed, c=5, n_ctx=40, nq=4, nkv=2, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((c, nq, d))
    k = rng.standard_normal((n_ctx + c, nkv, d))
    v = rng.standard_normal((n_ctx + c, nkv, d))
    return q, k, v, n_ctx


def test_long_window_is_full_attention():
    q, k, v, n = _qkv(1)
    full = attend(q, k, v, n)
    assert np.array_equal(attend(q, k, v, n, window=n + q.shape[0]), full)
    assert np.array_equal(attend(q, k, v, n, window=10_000), full)
    assert not np.allclose(attend(q, k, v, n, window=n), full)       # the first row loses position 0


def test_window_of_one_is_own_value():
    q, k, v, n = _qkv(2)
    out = attend(q, k, v, n, window=1)
    for j in range(q.shape[0]):
        for hq in range(q.shape[1]):
            assert np.array_equal(out[j, hq], v[n + j, hq // 2])


def test_window_is_truncated_full_attention():
    q, k, v, n = _qkv(3, c=6, n_ctx=50)
    for W in (2, 7, 16, 33):
        out = attend(q, k, v, n, window=W)
        for j in range(q.shape[0]):
            hi = n + j + 1
            lo = max(0, hi - W)
            # full attention of one column over the positions lo .. hi - 1 only
            ref = attend(q[j:j + 1], k[lo:hi], v[lo:hi], hi - lo - 1)
            assert np.allclose(out[j], ref[0], rtol=1e-12, atol=1e-12), (W, j)


def test_layer_windows():
    cfg = synth.get_config("tiny-fp32").with_(sliding_window=24, window_global_every=3)
    assert [cfg.layer_window(i) for i in range(6)] == [24, 24, 0, 24, 24, 0]
    assert cfg.with_(window_global_every=0).layer_window(2) == 24
    assert cfg.with_(sliding_window=0).layer_window(0) == 0


def test_speculative_greedy_with_window_equals_plain_greedy():
    base = synth.get_config("tiny-fp32")
    cfg = base.with_(sliding_window=24)
    w = synth.model_weights(base)
    prompt = [int(t) for t in synth.prompt_tokens(base)]
    outs = {}
    for name, c in (("window", cfg), ("full", base)):
        m = OracleModel(c, w)
        cache = oracle_cache(c, 1, 0, 24)
        m.prefill(cache, [prompt], chunk=16)
        ref = m.plain_greedy(cache.copy(), [prompt[-1]], 40)[0]
        outs[name] = [int(t) for t in ref]
        if name == "window":
            rng = np.random.default_rng(4)
            anchor, out = prompt[-1], []
            while len(out) < 30:
                P = len(out)
                drafts = [int(ref[P + i]) if rng.random() < 0.7 else int(rng.integers(0, c.vocab)) for i in range(c.k)]
                res = m.verify_round(cache, [[anchor] + drafts])
                cc, em = accept_greedy(res.logits, drafts)
                m.commit(cache, res, [cc])
                out += em
                anchor = em[-1]
            assert out == outs["window"][:len(out)]
    assert outs["window"] != outs["full"]
