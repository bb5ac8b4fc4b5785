"""A verify round captured once in a HIP graph and replayed, bit for bit.

Every launch of a round goes on the caller's stream, and none of them allocates,
copies or clears memory (counters are cleared by the kernels that use them), so
verify, accept and commit can be recorded once and replayed with new tokens and new
committed counts written into the same device buffers; a sampled round's LM head is
a cooperative launch, which is recorded and replayed as such.  Each
replay is compared bit for bit with the same round run eagerly on a twin cache:
the row statistics, the committed runs and their tokens, kv_len, the paged K/V
pools and the recurrent state.  Between replays the test does eager work of its
own (the twin's round, the uploads of the next tokens and counts) and
synchronises, and every replay is checked, not only the first.

Three cases: a ragged hybrid round (gated-delta-rule and attention layers, two
lanes of 5 and 3 columns), greedy and sampled (the drafter rows and the seed fixed
at capture), and a 64-row dense round whose gate/up projection runs the balanced
launch with cut units (their completion counters must be back at zero after every
replay).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import log
from helpers import small_dense, small_hybrid
from speculative_decoding_verify_round_amd.runtime import DeviceCache, DeviceModel

pytestmark = pytest.mark.gpu


def _hybrid():
    return small_hybrid(hidden=256, head_dim=128, ffn=512, vocab=1024, gdn_heads=2, gdn_dim=128, context=45)


CASES = {
    "hybrid-ragged": (_hybrid, [5, 3], 45, 8, 256, False),
    "hybrid-ragged-sampled": (_hybrid, [5, 3], 45, 8, 256, True),
    "dense-64rows-cut-units": (lambda: small_dense(hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=5120,
                                                   vocab=2048, context=300), [16, 16, 16, 16], 300, 24, 256, False),
}


def _cache(cfg, dm, bt, nb, lanes, context, max_blocks):
    dc = DeviceCache(dm, lanes, max_blocks, nb, block_table=bt, kv_len=[context] * lanes)
    for li in range(cfg.n_attn):
        for l in range(lanes):
            k, v = synth.kv_context(cfg, li, l, context)
            dc.set_kv(li, l, 0, k, v)
    for gi in range(cfg.n_gdn):
        for l in range(lanes):
            dc.set_gdn(gi, l, synth.gdn_state(cfg, gi, l))
    return dc


def _state(dc):
    out = {"kv_len": dc.kv_len.clone(), "committed": dc.committed.clone(), "out": dc.out_tokens.clone(),
           "stats": dc.row_stats.clone().view(torch.int32)}
    if dc.k_pool is not None:
        out["k"], out["v"] = dc.k_pool.clone(), dc.v_pool.clone()
    if dc.gdn is not None:
        out["gdn"] = dc.gdn.clone()
    return out


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_equals_eager(case):
    make, cols, context, max_blocks, chunk, sampled = CASES[case]
    cfg = make()
    L, R = len(cols), sum(cols)
    kw = {}
    if sampled:
        q, _ = synth.drafter_rows(cfg.input_seed, 5, R, cfg.vocab)
        kw = dict(mode="sampled", temperature=0.9, q_probs=torch.from_numpy(q).cuda(), seed=321)
    w = synth.model_weights(cfg)
    dm = DeviceModel(cfg, w, attn_chunk=chunk)
    try:
        bt, nb = synth.block_table(cfg, L, max_blocks)
        eager = _cache(cfg, dm, bt, nb, L, context, max_blocks)
        graph = _cache(cfg, dm, bt, nb, L, context, max_blocks)
        warm = _cache(cfg, dm, bt, nb, L, context, max_blocks)
        shape = [[0] * c for c in cols]
        tok_g = torch.zeros(R, dtype=torch.int32, device="cuda")
        cnt_g = torch.ones(L, dtype=torch.int32, device="cuda")
        cnt_e = torch.ones(L, dtype=torch.int32, device="cuda")
        # every kernel of the round runs once before the capture (code objects loaded)
        rc_w = warm.round(shape, tokens_dev=torch.zeros(R, dtype=torch.int32, device="cuda"), **kw)
        warm.verify(rc_w)
        warm.accept(rc_w)
        warm.commit(rc_w)
        torch.cuda.synchronize()
        del warm

        rc_g = graph.round(shape, tokens_dev=tok_g, **kw)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            graph.verify(rc_g)
            graph.accept(rc_g)
            graph.commit(rc_g, cnt_g)
        torch.cuda.synchronize()
        assert torch.equal(graph.kv_len, eager.kv_len)     # the capture ran nothing

        rng = np.random.default_rng(41)
        for step in range(4):
            toks = rng.integers(0, cfg.vocab, R).astype(np.int32)
            cnt = np.array([rng.integers(1, c + 1) for c in cols], np.int32)
            # eager twin
            rc_e = eager.round(shape, tokens_dev=torch.from_numpy(toks).cuda(), **kw)
            eager.verify(rc_e)
            eager.accept(rc_e)
            cnt_e.copy_(torch.from_numpy(cnt))
            eager.commit(rc_e, cnt_e)
            torch.cuda.synchronize()
            want = _state(eager)
            # the same round by replay: new tokens and counts in the captured buffers
            tok_g.copy_(torch.from_numpy(toks))
            cnt_g.copy_(torch.from_numpy(cnt))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = _state(graph)
            for key, val in want.items():
                assert torch.equal(got[key], val), (case, step, key)
            log(f"{case}: replay {step} equals the eager round (counts {cnt.tolist()}, "
                f"kv_len {got['kv_len'].tolist()})")
        del g
    finally:
        dm.close()
