"""Sliding-window targets on the GPU against the oracle.

Each case overwrites, in every windowed layer, the cache positions below the first
block spec_window_live_block allows the round to read with NaN (as if those blocks had
been released and reused): a kernel that read any of them would put NaN into the
logits.  Cases cover chunk skipping with the lane's first stage inside a chunk, a mixed
model whose every second attention layer stays global, a window shorter than the
lane's own columns, and both element types; a loop on the tiny fp32 decoder releases
blocks after every commit and must commit the windowed model's plain greedy tokens.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import Pair, log
from helpers import small_dense
from oracle.accept import argmax_lowest
from speculative_decoding_verify_round_amd import binding as B
from test_gpu_parity import _round_parity

pytestmark = pytest.mark.gpu


def _release_out_of_window(pair, kv_lens):
    cfg = pair.cfg
    for li in range(cfg.n_attn):
        W = cfg.layer_window(li)
        if W == 0:
            continue                       # a global layer keeps every block
        for l, kv in enumerate(kv_lens):
            n = B.spec_window_live_block(int(kv), W) * cfg.kv_block
            if n:
                nan = np.full((n, cfg.n_kv_heads, cfg.head_dim), np.nan, np.float32)
                pair.dc.set_kv(li, l, 0, nan, nan)
    torch.cuda.synchronize()


CASES = [
    # name, dtype, window, global_every, context, chunk
    ("bf16 W100 ctx700 chunk256", "bf16", 100, 0, 700, 256),
    ("bf16 W100 mixed ctx700", "bf16", 100, 2, 700, 256),
    ("bf16 W300 ctx1000 chunk512", "bf16", 300, 0, 1000, 512),
    ("bf16 W3 inside own columns", "bf16", 3, 0, 37, 256),
    ("bf16 window start on a chunk boundary", "bf16", 189, 0, 700, 256),
    ("bf16 W2000 longer than the context", "bf16", 2000, 0, 700, 256),
    ("bf16 W64 one stage", "bf16", 64, 0, 1000, 256),
    ("f32 W100 ctx700 chunk256", "f32", 100, 0, 700, 256),
    ("f32 W5 ctx37", "f32", 5, 0, 37, 256),
]


@pytest.mark.parametrize("name,dtype,W,every,ctx,chunk", CASES, ids=[c[0] for c in CASES])
def test_windowed_round_matches_oracle(name, dtype, W, every, ctx, chunk):
    if dtype == "bf16":
        cfg = small_dense(hidden=256, head_dim=128, ffn=512, vocab=1024, context=ctx,
                          sliding_window=W, window_global_every=every)
        tol = 3e-2
    else:
        cfg = synth.get_config("tiny-fp32").with_(sliding_window=W, window_global_every=every, context=ctx)
        tol = 1e-4
    log(f"window case {name}")
    pair = Pair(cfg, lanes=3, context=ctx, max_blocks=(ctx + 32) // 16 + 2, attn_chunk=chunk)
    _release_out_of_window(pair, [ctx] * 3)
    toks = [[5], [7, 8, 9, 10], [11, 12, 13, 14, 15, 16, 17, 18]]
    ores, rc, c, em, st, lerr, mism = _round_parity(pair, toks, logit_tol=tol)
    log(f"{name}: logit err {lerr:.2e}, mismatches {mism}")
    assert not mism
    # commit, release what slid out, and run a second round
    pair.om.commit(pair.oc, ores, list(c))
    pair.dc.commit(rc)
    torch.cuda.synchronize()
    assert list(pair.dc.kv_len.cpu().numpy()) == list(pair.oc.kv_len)
    _release_out_of_window(pair, list(pair.oc.kv_len))
    toks2 = [[int(e[-1])] + [3, 4, 5] for e in em]
    _, _, _, _, _, lerr2, mism2 = _round_parity(pair, toks2, logit_tol=tol)
    assert not mism2
    pair.close()


def test_windowed_greedy_loop_with_releases_equals_plain_greedy():
    cfg = synth.get_config("tiny-fp32").with_(sliding_window=24)
    pair = Pair(cfg, lanes=1, context=0, max_blocks=16)
    prompt = [int(t) for t in synth.prompt_tokens(cfg)]
    pair.om.prefill(pair.oc, [prompt], chunk=16)
    for c0 in range(0, 63, 16):
        c = min(16, 63 - c0)
        rc = pair.dc.round([prompt[c0:c0 + c]])
        pair.dc.verify(rc)
        pair.dc.commit(rc, torch.full((1,), c, dtype=torch.int32, device="cuda"))
        _release_out_of_window(pair, [c0 + c])
    ref = [int(t) for t in pair.om.plain_greedy(pair.oc.copy(), [prompt[-1]], 60)[0]]
    rng = np.random.default_rng(9)
    anchor, out, kv = prompt[-1], [], 63
    while len(out) < 45:
        P = len(out)
        drafts = [ref[P + i] if rng.random() < 0.7 else int(rng.integers(0, cfg.vocab)) for i in range(cfg.k)]
        rc = pair.dc.round([[anchor] + drafts])
        pair.dc.verify(rc)
        pair.dc.accept(rc)
        pair.dc.commit(rc)
        c, em, _ = pair.dc.results(rc)
        kv += int(c[0])
        _release_out_of_window(pair, [kv])
        out += em[0]
        anchor = em[0][-1]
    assert out == ref[:len(out)]
    log(f"windowed loop: {len(out)} tokens, kv_len {kv}, live block {B.spec_window_live_block(kv, 24)}")
    pair.close()
