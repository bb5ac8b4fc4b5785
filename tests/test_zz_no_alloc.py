"""The head-only round that allocates nothing (spec_verify_head_noalloc) against
spec_verify_head + spec_accept on a caller workspace: the same committed runs, tokens and
row statistics, bit for bit, on two calls in a row (the second smaller), sampled and
greedy; the static scratch keeps the first call's contents, so the second checks that
what must start at zero does."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import log
from speculative_decoding_verify_round_amd import binding as B
from synth.configs import ModelConfig

pytestmark = pytest.mark.gpu


def _head_model():
    from speculative_decoding_verify_round_amd.runtime import DeviceModel
    cfg = ModelConfig(name="head-noalloc", n_layers=0, hidden=1024, n_q_heads=0, n_kv_heads=0, head_dim=0,
                      ffn=0, vocab=32768, dtype="bf16", layer_kinds=(), head_only=True, seed_index=21)
    return cfg, DeviceModel(cfg, synth.head_weights(cfg))


def _outputs(dc, rc, L, R):
    torch.cuda.synchronize()
    return (dc.committed[:L].clone(), dc.out_tokens[:L].clone(), dc.row_stats[:R].clone())


@pytest.mark.parametrize("mode", ["sampled", "greedy"])
def test_noalloc_head_round_equals_workspace_round(mode):
    from speculative_decoding_verify_round_amd.runtime import DeviceCache
    cfg, dm = _head_model()
    st = torch.cuda.current_stream().cuda_stream
    for L, k in ((8, 7), (3, 1)):                      # the second call is smaller
        R = L * (k + 1)
        log(f"no-alloc head round {mode}: {L} lanes x {k + 1}")
        hid = torch.from_numpy(synth.hidden_states(cfg, R, tag=L)).to("cuda", torch.bfloat16)
        q, d = synth.drafter_rows(cfg.input_seed, 50 + L, R, cfg.vocab)
        toks = [[int(l)] + [int(x) for x in d[l * (k + 1) + 1:(l + 1) * (k + 1)]] for l in range(L)]
        kw = dict(mode="sampled", temperature=0.8, q_probs=torch.from_numpy(q).cuda(), seed=77 + L) \
            if mode == "sampled" else {}
        ref = DeviceCache(dm, L, 1, 1, kv_len=[100 + l for l in range(L)])
        rc = ref.round(toks, **kw)
        ref.verify_head(rc, hid)
        ref.accept(rc)
        c_ref, t_ref, s_ref = _outputs(ref, rc, L, R)
        # the no-alloc call writes into fresh outputs; its round carries no workspace
        got = DeviceCache(dm, L, 1, 1, kv_len=[100 + l for l in range(L)])
        got.committed.fill_(-7)
        got.out_tokens.fill_(-7)
        got.row_stats.fill_(float("nan"))
        rg = got.round(toks, **kw)
        rg.r.workspace = None
        rg.r.workspace_bytes = 0
        B.spec_verify_head_noalloc(dm.handle, rg.r, hid.data_ptr(), got.committed.data_ptr(),
                                   got.out_tokens.data_ptr(), got.row_stats.data_ptr(), st)
        c, t, s = _outputs(got, rg, L, R)
        assert torch.equal(c, c_ref), (c, c_ref)
        for l in range(L):
            n = int(c_ref[l])
            assert torch.equal(t[l, :n], t_ref[l, :n]), (l, t[l], t_ref[l])
        assert torch.equal(s.view(torch.int32), s_ref.view(torch.int32))
        log(f"  committed {c.tolist()}")
    dm.close()
