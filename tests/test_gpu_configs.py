"""Parity at the full widths of the benchmark configs (reduced depth where the oracle must stay quick).

  * mid bf16 decoder, all 8 layers, 4 lanes x k=4, context 2048 in paged KV:
    greedy with planted drafts, sampled at T = 1.0, and the row budget 8 swept
    over 1..8 lanes;
  * 27B-class dense decoder at full width (H 5120, 40/8 heads, FFN 17408,
    V 151936), 2 of its 64 layers, context 8192, k = 7 at 1 and 8 lanes;
  * hybrid decoder at full width (H 4096, 16 recurrent heads of 128x128 state,
    32/8 GQA heads, FFN 12288, V 262144), 4 of its 48 layers (3 recurrent + 1
    attention), 4 lanes x k=3, context 4096, greedy and sampled.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import GAP_EXCUSE, Pair, log, top2_gap
from oracle import accept_greedy, accept_sampled, plan_drafts
from oracle.accept import argmax_lowest
from test_gpu_parity import _round_parity, check_committed_cache

pytestmark = pytest.mark.gpu

def _greedy_tokens(pair, anchors, steps):
    """The oracle's own plain greedy continuation (on a copy of its cache)."""
    return pair.om.plain_greedy(pair.oc.copy(), anchors, steps)


def _planted(pair, anchors, k, alpha, tag):
    ref = _greedy_tokens(pair, anchors, k)
    return [[int(a)] + [int(x) for x in synth.planted_drafts(pair.cfg.input_seed, tag + l, ref[l], alpha,
                                                               pair.cfg.vocab)]
            for l, a in enumerate(anchors)]


def _account(budget, name, rows, mism):
    for m in mism:
        assert m[-1] < GAP_EXCUSE, f"{name}: token mismatch at a row without a near-tie: {m}"
    budget.add(name, rows, len(mism))
    log(f"{name}: {rows} rows, {len(mism)} excused mismatches")


def test_mid_bf16_greedy_sampled_and_budget_sweep(mismatch_budget):
    cfg = synth.get_config("mid-bf16")
    log("mid-bf16: setup")
    pair = Pair(cfg, lanes=8, context=cfg.context, max_blocks=(cfg.context + 64) // 16 + 1)
    anchors = [int(t) for t in synth.uniform_tokens(cfg.input_seed, 5, 8, cfg.vocab)]
    # all 8 lanes x k = 4 (40 rows), greedy with drafts planted against the target's own greedy tokens
    toks = _planted(pair, anchors, cfg.k, 0.7, 100)
    ores, rc, c, em, st, lerr, mism = _round_parity(pair, toks)
    log(f"mid-bf16 greedy 8x5: logit err {lerr:.2e}, committed {list(c)}")
    _account(mismatch_budget, "mid-bf16 greedy", rc.R, mism)
    # sampled at T = 1.0
    q, d = synth.drafter_rows(cfg.input_seed, 7, rc.R, cfg.vocab)
    toks_s = [[anchors[l]] + [int(x) for x in d[l * 5 + 1:(l + 1) * 5]] for l in range(8)]
    ores, rc, c, em, st, lerr, mism = _round_parity(pair, toks_s, "sampled", 1.0, q, seed=cfg.philox_seed)
    log(f"mid-bf16 sampled: logit err {lerr:.2e}, committed {list(c)}")
    _account(mismatch_budget, "mid-bf16 sampled", rc.R, mism)
    # row budget 8 across 1..8 lanes: drafts per lane from the planner, rows never above 8
    for L in range(1, 9):
        k_l = plan_drafts(cfg.k, 8, L)
        assert L * (k_l + 1) <= 8 or k_l == 0
        toks_b = [t[: k_l + 1] for t in toks[:L]]
        sp = pair
        ores = sp.om.verify_round(_sub_cache(sp.oc, L), toks_b)
        dc = _sub_device(sp, L)
        rcb = dc.round(toks_b)
        gl = dc.debug_logits(rcb).cpu().numpy()
        err = float(np.max(np.abs(gl - ores.logits)))
        assert err <= 3e-2
        dc.verify(rcb); dc.accept(rcb)
        cb, emb, _ = dc.results(rcb)
        mism_b = []
        for l in range(L):
            rows = ores.lane_rows[l]
            oc_, oem = accept_greedy(ores.logits[rows.start:rows.stop], toks_b[l][1:])
            if (oc_, oem) != (int(cb[l]), emb[l]):
                mism_b.append((l, min(top2_gap(ores.logits[r]) for r in rows)))
        _account(mismatch_budget, f"mid-bf16 budget 8 at {L} lanes", rcb.R, mism_b)
        log(f"budget 8, {L} lanes: {k_l} drafts, {rcb.R} rows, logit err {err:.2e}")
    pair.close()


def _sub_cache(oc, L):
    c = oc.copy()
    c.kv_len = c.kv_len[:L]
    c.block_table = c.block_table[:L]
    c.gdn = [g[:L] for g in c.gdn]
    return c


def _sub_device(pair, L):
    from speculative_decoding_verify_round_amd.runtime import DeviceCache
    dc = DeviceCache(pair.dm, L, pair.dc.max_blocks, pair.dc.n_blocks, block_table=pair.bt[:L],
                     kv_len=list(pair.oc.kv_len[:L]), pools=False)
    dc.k_pool, dc.v_pool = pair.dc.k_pool, pair.dc.v_pool       # shared pools: rounds only read them
    if pair.dc.gdn is not None:
        dc.gdn = pair.dc.gdn[:L].contiguous()
    return dc


def _big(name, n_layers, lanes, context):
    cfg = synth.get_config(name, n_layers=n_layers)
    log(f"{name}: generating {n_layers}-layer weights")
    return cfg, Pair(cfg, lanes=lanes, context=context, max_blocks=(context + 32) // 16 + 1)


def test_dense_27b_full_width_two_layers(mismatch_budget):
    cfg, pair = _big("dense-27b", 2, 8, 8192)
    anchors = [int(t) for t in synth.uniform_tokens(cfg.input_seed, 5, 8, cfg.vocab)]
    log("dense-27b: planting drafts")
    toks = _planted(pair, anchors, cfg.k, [0.9, 0.8, 0.7, 0.6, 0.5, 0.45, 0.35], 200)
    log("dense-27b: 8 lanes x 8 rows")
    ores, rc, c, em, st, lerr, mism = _round_parity(pair, toks)
    log(f"dense-27b 8 lanes: logit err {lerr:.2e}, committed {list(c)}")
    _account(mismatch_budget, "dense-27b 2 layers L8", rc.R, mism)
    pair.om.commit(pair.oc, ores, list(c))
    pair.dc.commit(rc)
    torch.cuda.synchronize()
    assert list(pair.dc.kv_len.cpu().numpy()) == list(pair.oc.kv_len)
    check_committed_cache(pair, 8192)
    # one lane (8 rows) on the updated state
    dc1 = _sub_device(pair, 1)
    t1 = [[em[0][-1]] + toks[1][1:]]
    o1 = pair.om.verify_round(_sub_cache(pair.oc, 1), t1)
    z1 = dc1.debug_logits(dc1.round(t1)).cpu().numpy()
    assert np.max(np.abs(z1 - o1.logits)) <= 3e-2
    pair.close()


def test_hybrid_full_width_four_layers(mismatch_budget):
    cfg, pair = _big("hybrid-gdn", 4, 4, 4096)
    anchors = [int(t) for t in synth.uniform_tokens(cfg.input_seed, 5, 4, cfg.vocab)]
    toks = _planted(pair, anchors, cfg.k, 0.7, 300)
    ores, rc, c, em, st, lerr, mism = _round_parity(pair, toks)
    log(f"hybrid greedy: logit err {lerr:.2e}, committed {list(c)}")
    _account(mismatch_budget, "hybrid 4 layers greedy", rc.R, mism)
    q, d = synth.drafter_rows(cfg.input_seed, 8, rc.R, cfg.vocab)
    toks_s = [[anchors[l]] + [int(x) for x in d[l * 4 + 1:(l + 1) * 4]] for l in range(4)]
    ores_s, rc_s, c_s, em_s, st_s, lerr_s, mism_s = _round_parity(pair, toks_s, "sampled", 1.0, q,
                                                                  seed=cfg.philox_seed)
    log(f"hybrid sampled: logit err {lerr_s:.2e}, committed {list(c_s)}")
    _account(mismatch_budget, "hybrid 4 layers sampled", rc_s.R, mism_s)
    pair.om.commit(pair.oc, ores_s, list(c_s))
    pair.dc.commit(rc_s)
    torch.cuda.synchronize()
    for gi in range(cfg.n_gdn):   # the bar of the full-depth hybrid (test_gpu_full_depth.STATE_BAR)
        g = pair.dc.gdn[:, gi].cpu().numpy()
        o = pair.oc.gdn[gi]
        assert np.max(np.abs(g - o)) <= 2e-4 * np.max(np.abs(o))
    check_committed_cache(pair, 4096)
    pair.close()
