"""Per-row presence / frequency penalties on the GPU (the FreeToken issue's per-row
penalties in target-side verify), against the oracle's penalised rows:

  * greedy and sampled rounds on a small bf16 decoder, lanes with repeated drafts and
    non-zero counts: the row statistics (max, log-sum-exp, argmax, logit at the next
    draft) of the penalised logits, and the committed runs (a mismatch is excused only at
    an oracle near-tie);
  * a greedy loop on the tiny fp32 decoder with counts kept on the device by
    spec_counts_add commits the oracle's plain greedy tokens of the penalised model;
  * spec_counts_add counts every committed token, repeats included.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import GAP_EXCUSE, Pair, log, top2_gap
from helpers import small_dense
from oracle import accept_greedy, accept_sampled, row_stats
from oracle.accept import argmax_lowest
from oracle.penalty import add_counts, penalized_rows, penalty
from speculative_decoding_verify_round_amd import binding as B

pytestmark = pytest.mark.gpu

PRES, FREQ = 0.4, 0.25


def _counts(cfg, lanes, seed):
    rng = np.random.default_rng(seed)
    c = np.zeros((lanes, cfg.vocab), np.int32)
    for l in range(lanes):
        hot = rng.integers(0, cfg.vocab, 40)
        np.add.at(c[l], hot, 1)
        c[l, 100 + l] += 2                        # the anchors below are counted
    return c


def _penalised_round(pair, toks, counts, mode="greedy", T=1.0, q=None, seed=0):
    ores = pair.om.verify_round(pair.oc, toks)
    zs = []
    for l, rows in enumerate(ores.lane_rows):
        zs.append(penalized_rows(ores.logits[rows.start:rows.stop], toks[l], counts[l], PRES, FREQ))
    z = np.concatenate(zs)
    cd = torch.from_numpy(counts).cuda()
    qd = torch.from_numpy(q).cuda() if q is not None else None
    rc = pair.dc.round(toks, mode=mode, temperature=T, q_probs=qd, seed=seed, kv_len_host=list(pair.oc.kv_len),
                       counts=cd, presence=PRES, frequency=FREQ)
    pair.dc.verify(rc)
    pair.dc.accept(rc)
    c, em, st = pair.dc.results(rc)
    nxt = []
    for l, t in enumerate(toks):
        nxt += [int(x) for x in t[1:]] + [-1]
    ost = row_stats(z, nxt, T if mode == "sampled" else 1.0)
    mism = []
    for l, rows in enumerate(ores.lane_rows):
        lz = z[rows.start:rows.stop]
        if mode == "greedy":
            want = accept_greedy(lz, toks[l][1:])
        else:
            want = accept_sampled(lz, toks[l][1:], q[rows.start + 1:rows.stop], T, seed, l, int(pair.oc.kv_len[l]))
        if want != (int(c[l]), em[l]):
            mism.append((l, want, int(c[l]), em[l], min(top2_gap(lz[j]) for j in range(len(lz)))))
    return ores, rc, z, st, ost, c, em, mism


def test_penalised_greedy_and_sampled_rounds_small_dense():
    cfg = small_dense(hidden=256, head_dim=128, ffn=512, vocab=1024, context=37)
    pair = Pair(cfg, lanes=4, context=37, max_blocks=8)
    counts = _counts(cfg, 4, 11)
    # greedy: drafts repeat tokens of the counts and of each other; each lane has counted
    # the token its first row prefers, so the penalties move that row's choice
    toks = [[100, 7, 7, 9], [101, 101, 5], [102], [103, 200, 201, 200, 202, 200]]
    raw = pair.om.verify_round(pair.oc, toks)
    for l, rows in enumerate(raw.lane_rows):
        counts[l, argmax_lowest(raw.logits[rows.start])] += 3
    ores, rc, z, st, ost, c, em, mism = _penalised_round(pair, toks, counts)
    # the penalties change the model's choice on some rows (else the test would not test them)
    raw_am = [argmax_lowest(r) for r in ores.logits]
    assert any(a != b for a, b in zip(raw_am, ost["argmax"]))
    assert np.max(np.abs(st["max"] - ost["max"])) < 3e-2
    assert np.max(np.abs(st["lse"] - ost["lse"])) < 3e-2
    fin = ~np.isnan(ost["z_next"])
    assert np.array_equal(np.isnan(st["z_next"]), ~fin)
    assert np.max(np.abs(st["z_next"][fin] - ost["z_next"][fin])) < 3e-2
    gaps = np.array([top2_gap(r) for r in z])
    bad = [r for r in range(len(z)) if st["argmax"][r] != ost["argmax"][r] and gaps[r] >= GAP_EXCUSE]
    assert not bad, bad
    assert all(m[-1] < GAP_EXCUSE for m in mism), mism
    log(f"penalised greedy: {len(mism)} excused lane mismatches, argmax changed on "
        f"{sum(a != b for a, b in zip(raw_am, ost['argmax']))} rows")
    # sampled rounds, drafts from the drafter rows (T = 0.8)
    total, bad_lanes = 0, []
    for rnd in range(4):
        q, d = synth.drafter_rows(cfg.input_seed, 50 + rnd, 4 * 5, cfg.vocab)
        toks = [[100 + l] + [int(x) for x in d[l * 5 + 1:(l + 1) * 5]] for l in range(4)]
        _, _, _, _, _, _, _, mism = _penalised_round(pair, toks, counts, "sampled", 0.8, q, seed=99 + rnd)
        total += 4
        bad_lanes += mism
    log(f"penalised sampled: {len(bad_lanes)} of {total} lanes differ: {bad_lanes}")
    assert not bad_lanes
    pair.close()


def test_counts_add():
    counts = torch.zeros((3, 20), dtype=torch.int32, device="cuda")
    committed = torch.tensor([3, 1, 2], dtype=torch.int32, device="cuda")
    out = torch.tensor([[4, 4, 9, 1], [7, 7, 7, 7], [19, 25, 0, 0]], dtype=torch.int32, device="cuda")
    B.spec_counts_add(counts.data_ptr(), 20, 3, committed.data_ptr(), out.data_ptr(), 4,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert c[0, 4] == 2 and c[0, 9] == 1 and c[0].sum() == 3
    assert c[1, 7] == 1 and c[1].sum() == 1
    assert c[2, 19] == 1 and c[2].sum() == 1          # 25 is outside the vocabulary


def test_penalised_greedy_loop_tiny_fp32_equals_plain_penalised_greedy():
    cfg = synth.get_config("tiny-fp32")
    pair = Pair(cfg, lanes=1, context=0, max_blocks=16)
    prompt = [int(t) for t in synth.prompt_tokens(cfg)]
    pair.om.prefill(pair.oc, [prompt], chunk=16)
    for c0 in range(0, 63, 16):
        c = min(16, 63 - c0)
        rc = pair.dc.round([prompt[c0:c0 + c]])
        pair.dc.verify(rc)
        pair.dc.commit(rc, torch.full((1,), c, dtype=torch.int32, device="cuda"))
    counts0 = np.bincount(prompt, minlength=cfg.vocab).astype(np.int32)
    # the oracle's plain greedy of the penalised model
    plain, counts = pair.oc.copy(), counts0.copy()
    cur, ref = prompt[-1], []
    for _ in range(60):
        res = pair.om.verify_round(plain, [[cur]])
        nxt = argmax_lowest((res.logits[0] - penalty(counts, PRES, FREQ)).astype(np.float32))
        pair.om.commit(plain, res, [1])
        ref.append(nxt)
        counts[nxt] += 1
        cur = nxt
    # the device: drafts planted from the reference, counts kept by spec_counts_add
    cd = torch.from_numpy(counts0[None, :].copy()).cuda()
    rng = np.random.default_rng(8)
    anchor, out = prompt[-1], []
    while len(out) < 40:
        P = len(out)
        drafts = [ref[P + i] if rng.random() < 0.7 else int(rng.integers(0, cfg.vocab)) for i in range(cfg.k)]
        rc = pair.dc.round([[anchor] + drafts], counts=cd, presence=PRES, frequency=FREQ)
        pair.dc.verify(rc)
        pair.dc.accept(rc)
        pair.dc.commit(rc)
        B.spec_counts_add(cd.data_ptr(), cfg.vocab, 1, pair.dc.committed.data_ptr(), pair.dc.out_tokens.data_ptr(),
                          pair.dc.out_tokens.shape[1], torch.cuda.current_stream().cuda_stream)
        c, em, _ = pair.dc.results(rc)
        out += em[0]
        anchor = em[0][-1]
    assert out == ref[:len(out)]
    want = counts0.copy()
    add_counts(want, out)
    assert np.array_equal(cd.cpu().numpy()[0], want)
    log(f"penalised tiny loop: {len(out)} tokens")
    pair.close()


def test_penalised_sampled_rounds_tiny_fp32():
    """The fp32 LM head and residual race with penalties, sampled at T = 0.8."""
    cfg = synth.get_config("tiny-fp32").with_(context=37)
    pair = Pair(cfg, lanes=4, context=37, max_blocks=8)
    counts = _counts(cfg, 4, 12)
    bad = []
    for rnd in range(3):
        q, d = synth.drafter_rows(cfg.input_seed, 70 + rnd, 4 * 5, cfg.vocab)
        toks = [[100 + l] + [int(x) for x in d[l * 5 + 1:(l + 1) * 5]] for l in range(4)]
        _, _, _, _, _, _, _, mism = _penalised_round(pair, toks, counts, "sampled", 0.8, q, seed=7 + rnd)
        bad += mism
    log(f"penalised sampled fp32: {bad}")
    assert not bad
    pair.close()


def test_penalised_ngram_device_loop_equals_plain_penalised_greedy():
    """The n-gram drafter's device loop with penalties and device-kept counts (one lane's
    prompt repeats itself) commits the oracle's plain penalised greedy tokens.  Mild
    penalties, so that the repeating lane still keeps copied guesses."""
    pres, freq = 0.05, 0.03
    cfg = synth.get_config("tiny-fp32")
    pair = Pair(cfg, lanes=2, context=0, max_blocks=24)
    prompts = [[int(t) for t in synth.prompt_tokens(cfg)],
               [int(t) for t in synth.uniform_tokens(cfg.input_seed, 91, 64, cfg.vocab)]]
    prompts[1][32:] = prompts[1][:32]
    pair.om.prefill(pair.oc, prompts, chunk=16)
    for c0 in range(0, 63, 16):
        c = min(16, 63 - c0)
        rc = pair.dc.round([p[c0:c0 + c] for p in prompts])
        pair.dc.verify(rc)
        pair.dc.commit(rc, torch.full((2,), c, dtype=torch.int32, device="cuda"))
    counts0 = np.stack([np.bincount(p, minlength=cfg.vocab) for p in prompts]).astype(np.int32)
    rounds, k = 10, 7
    refs = []
    for l in range(2):
        one = pair.oc.copy()
        cnt, cur, ref = counts0[l].copy(), prompts[l][-1], []
        for _ in range(rounds * (k + 1)):
            res = pair.om.verify_round(one, [[cur] if i == l else [0] for i in range(2)])
            row = res.logits[res.lane_rows[l].start]
            nxt = argmax_lowest((row - penalty(cnt, pres, freq)).astype(np.float32))
            pair.om.commit(one, res, [1, 1])
            ref.append(nxt)
            cnt[nxt] += 1
            cur = nxt
        refs.append(ref)
    max_len = 64 + rounds * (k + 1)
    hist = torch.zeros((2, max_len), dtype=torch.int32, device="cuda")
    hist[:, :64] = torch.tensor(prompts, dtype=torch.int32).cuda()
    hlen = torch.full((2,), 64, dtype=torch.int32, device="cuda")
    cd = torch.from_numpy(counts0).cuda()
    pair.dc.ngram_rounds(hist, hlen, rounds, k, 3, counts=cd, presence=pres, frequency=freq)
    torch.cuda.synchronize()
    hl, h = hlen.cpu().tolist(), hist.cpu().numpy()
    for l in range(2):
        got = [int(t) for t in h[l, 64:hl[l]]]
        assert got == refs[l][:len(got)], l
        want = counts0[l].copy()
        add_counts(want, got)
        assert np.array_equal(cd.cpu().numpy()[l], want), l
    log(f"penalised n-gram loop: {[hl[l] - 64 for l in range(2)]} tokens in {rounds} rounds")
    assert hl[1] - 64 > rounds            # the repeating lane kept guesses
    pair.close()
