"""The n-gram (copy-from-the-conversation) drafter and the multi-round loop on the GPU.

  * spec_ngram_draft gives the oracle's drafts and matched suffix length bit for bit on
    seeded histories with planted repeats, short and empty histories, k from 0 to 15 and
    suffix lengths 1..8;
  * spec_history_append appends each lane's committed run;
  * the device-side loop (draft, verify, accept, commit, append; no host round trip)
    on the tiny fp32 decoder commits exactly the oracle's plain greedy continuation of
    each lane and the same per-round runs as the oracle's n-gram loop.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import Pair, log
from oracle import round_tokens, speculative_greedy_ngram
from speculative_decoding_verify_round_amd import binding as B

pytestmark = pytest.mark.gpu


def _histories(seed, L, max_len):
    rng = np.random.default_rng(seed)
    hist = np.zeros((L, max_len), np.int32)
    lens = []
    for l in range(L):
        n = int(rng.choice([1, 2, 3, 5, 17, 64, max_len // 2, max_len]))
        vocab = int(rng.choice([3, 7, 50, 5000]))          # small vocabularies recur often
        h = rng.integers(0, vocab, n).astype(np.int32)
        if n > 40 and rng.random() < 0.5:                   # plant a copy of an earlier run
            a, b = int(rng.integers(0, n // 2)), int(rng.integers(n // 2, n - 8))
            h[b:b + 8] = h[a:a + 8]
        hist[l, :n] = h
        lens.append(n)
    return hist, np.array(lens, np.int32)


@pytest.mark.parametrize("seed,k,n_max,n_min", [(1, 7, 3, 1), (2, 0, 3, 1), (3, 15, 8, 1), (4, 4, 2, 2),
                                                 (5, 3, 8, 5), (6, 1, 1, 1)])
def test_ngram_draft_matches_oracle(seed, k, n_max, n_min):
    L, max_len = 37, 300
    hist, lens = _histories(seed, L, max_len)
    h_d = torch.from_numpy(hist).cuda()
    len_d = torch.from_numpy(lens).cuda()
    tok = torch.full((L, k + 1), -7, dtype=torch.int32, device="cuda")
    nm = torch.full((L,), -7, dtype=torch.int32, device="cuda")
    B.spec_ngram_draft(h_d.data_ptr(), len_d.data_ptr(), L, max_len, k, n_max, n_min, tok.data_ptr(), nm.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    tok, nm = tok.cpu().numpy(), nm.cpu().numpy()
    matched = 0
    for l in range(L):
        want, n = round_tokens(hist[l, :lens[l]], k, n_max, n_min)
        assert list(tok[l]) == want, (l, lens[l])
        assert int(nm[l]) == n, l
        matched += n > 0
    log(f"seed {seed}: {matched} of {L} lanes matched a suffix")


def test_ngram_draft_empty_history_gives_token_zero():
    h = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    n = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    tok = torch.full((2, 4), -1, dtype=torch.int32, device="cuda")
    nm = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    h[1, 0] = 9
    B.spec_ngram_draft(h.data_ptr(), n.data_ptr(), 2, 8, 3, 3, 1, tok.data_ptr(), nm.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert tok.cpu().tolist() == [[0, 0, 0, 0], [9, 9, 9, 9]]
    assert nm.cpu().tolist() == [0, 0]


def test_history_append():
    L, max_len, stride = 3, 10, 16
    hist = torch.zeros((L, max_len), dtype=torch.int32, device="cuda")
    lens = torch.tensor([2, 9, 0], dtype=torch.int32, device="cuda")
    committed = torch.tensor([3, 4, 1], dtype=torch.int32, device="cuda")
    out = torch.arange(L * stride, dtype=torch.int32, device="cuda").view(L, stride) + 100
    B.spec_history_append(hist.data_ptr(), lens.data_ptr(), L, max_len, committed.data_ptr(), out.data_ptr(), stride,
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    h = hist.cpu().numpy()
    assert lens.cpu().tolist() == [5, 10, 1]
    assert list(h[0, 2:5]) == [100, 101, 102]
    assert list(h[1, 9:]) == [116]                     # capped at max_len
    assert list(h[2, :1]) == [132]


def test_device_loop_tiny_fp32_equals_plain_greedy():
    """Two lanes of the tiny fp32 decoder (one prompt repeats itself), 12 rounds at k = 7
    with n-gram drafts (n 1..3), run as one sequence of device calls."""
    cfg = synth.get_config("tiny-fp32")
    pair = Pair(cfg, lanes=2, context=0, max_blocks=24)
    prompts = [synth.prompt_tokens(cfg), synth.uniform_tokens(cfg.input_seed, 91, 64, cfg.vocab)]
    prompts[1][32:] = prompts[1][:32]
    # teacher-forced prefill on both sides: 63 tokens committed, the last is the anchor
    pair.om.prefill(pair.oc, [list(map(int, p)) for p in prompts], chunk=16)
    for c0 in range(0, 63, 16):
        c = min(16, 63 - c0)
        rc = pair.dc.round([list(map(int, p[c0:c0 + c])) for p in prompts])
        pair.dc.verify(rc)
        pair.dc.commit(rc, torch.full((2,), c, dtype=torch.int32, device="cuda"))
    rounds, k = 12, 7
    ref = pair.om.plain_greedy(pair.oc.copy(), [int(p[-1]) for p in prompts], rounds * (k + 1) + 2)
    oout, ocounts = speculative_greedy_ngram(pair.om, pair.oc, [list(map(int, p)) for p in prompts], rounds, k, 3)
    max_len = 64 + rounds * (k + 1)
    hist = torch.zeros((2, max_len), dtype=torch.int32, device="cuda")
    hist[:, :64] = torch.from_numpy(np.stack(prompts).astype(np.int32)).cuda()
    hlen = torch.full((2,), 64, dtype=torch.int32, device="cuda")
    pair.dc.ngram_rounds(hist, hlen, rounds, k, 3)
    torch.cuda.synchronize()
    hl = hlen.cpu().tolist()
    h = hist.cpu().numpy()
    for l in range(2):
        got = [int(t) for t in h[l, 64:hl[l]]]
        assert got == oout[l], l
        assert got == [int(t) for t in ref[l][: len(got)]], l
    assert list(pair.dc.kv_len.cpu().numpy()) == [63 + len(o) for o in oout]
    log(f"device loop: {[len(o) for o in oout]} tokens in {rounds} rounds; committed per round {ocounts.T.tolist()}")
    pair.close()
