"""Benchmark of the verify round on one MI355X.

Workload (default): the 27B-class dense bf16 decoder (64 layers, H 5120, 40 q /
8 kv heads x 128, SwiGLU FFN 17408, vocab 151936, random N(0, 0.02) weights)
with 8 lanes x (k = 7 drafts + anchor) = 64 rows per round and 8192 tokens of
synthetic committed context per lane in paged KV.  Drafts are planted against
the model's own plain-greedy continuation with per-slot acceptance falling
linearly from 0.9 (slot 1) to 0.35 (slot 7); a miss plants a different token.

One step = one verify round through the whole hot path: the forward over all
rows, the fused LM-head statistics, acceptance and the commit, followed by the
copy of the committed run back to the host (the drafter's input).  Steps
continue decoding from where the previous one stopped.

Other workloads (`--config`):
  * head-v151936: the LM head and acceptance alone on 64 given hidden states
    (H 5120, V 151936), greedy or `--sampled T` against seeded drafter rows;
  * mid-bf16: an 8-layer bf16 decoder (H 2048, V 32768), 4 lanes x (k = 4 + 1),
    context 2048; `--evict-mall` writes a 512 MiB scratch buffer between rounds
    (outside the timed rounds) so the 256 MB last-level cache holds no weights;
  * hybrid-gdn: 48 layers, three of every four gated-delta-rule layers (16 heads
    of 128 x 128 state), H 4096, V 262144, 4 lanes x (k = 3 + 1), context 4096;
  * dense-27b with `--lanes 1`: the one-lane round (8 rows).
`--sampled T` runs the textbook rule at temperature T: each lane's drafts are
drawn from seeded drafter distributions q, and each round's anchor is the
lane's last committed token.  `--drafter ngram` takes the drafts from the
copy-from-the-conversation (n-gram prompt lookup) drafter on each lane's own
history, as a device-side loop.

Prints one JSON line: committed tokens/s as `value`, verify rows/s, the round's
HBM roofline fraction, the dominant kernel's achieved bandwidth measured with
HIP events over the timed region, a plain device copy's rate as the reachable
ceiling, and the oracle timed on host cores on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from speculative_decoding_verify_round_amd import binding as B  # noqa: E402
from speculative_decoding_verify_round_amd.runtime import DeviceCache, DeviceModel, attn_chunk_for, pack_weight  # noqa: E402

HBM_PEAK_GBS = 8000.0
# measured HBM traffic of the gate/up kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE passes,
# calibrated against a plain copy); reported only while that kernel's sources are unchanged
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_dense27b.md")
GATEUP_SOURCES = ("gemm.hip", "common.hpp")
COPY_CALIBRATION_BYTES = 512 << 20
EVICT_BYTES = 512 << 20
METRIC = "committed tokens/s & verify rows/s at lanes×(k+1); % of HBM roofline"
NGRAM_MAX = 3


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------- synthetic inputs on the GPU
def gpu_weights(cfg, seed: int):
    """Random N(0, 0.02) bf16 weights generated on the device (seeded per tensor); every
    matrix but the embedding table is packed into the library's fragment layout as it is made."""
    dev = torch.device("cuda")

    def packed(tid, shape):
        return pack_weight(normal(tid, shape))

    def normal(tid, shape, std=0.02):
        g = torch.Generator(device=dev)
        g.manual_seed(seed * 100003 + tid)
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        flat = out.view(-1)
        step = 1 << 26
        for s in range(0, flat.numel(), step):
            n = min(step, flat.numel() - s)
            flat[s:s + n] = (torch.randn(n, generator=g, device=dev) * std).to(torch.bfloat16)
        return out

    H, F = cfg.hidden, cfg.ffn
    w = {"lm_head": packed(1, (cfg.vocab, H)), "final_norm": torch.ones(H, device=dev), "layers": []}
    if not cfg.head_only:
        w["embed"] = normal(0, (cfg.vocab, H))
    for i in range(cfg.n_layers):
        base = 100 + 16 * i
        n_in = cfg.qkv_rows if cfg.layer_kinds[i] == "attn" else cfg.gdn_in_rows
        n_o = cfg.n_q_heads * cfg.head_dim if cfg.layer_kinds[i] == "attn" else cfg.gdn_heads * cfg.gdn_dim
        w["layers"].append({
            "norm1": torch.ones(H, device=dev), "norm2": torch.ones(H, device=dev),
            "w_in": packed(base, (n_in, H)), "w_o": packed(base + 1, (H, n_o)),
            "w_gate": packed(base + 2, (F, H)), "w_up": packed(base + 3, (F, H)), "w_down": packed(base + 4, (H, F)),
        })
    return w


def gateup_source_hash() -> str:
    """Hash of the code (comments and whitespace removed) the gate/up kernel is built from."""
    import hashlib, re
    h = hashlib.sha256()
    for f in GATEUP_SOURCES:
        with open(os.path.join(ROOT, "speculative_decoding_verify_round_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)     # block comments
        src = re.sub(r"//[^\n]*", " ", src)                   # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """Bytes per gate/up launch from the committed counter summary, or None when the
    summary is missing, is of another workload or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("source_hash") == gateup_source_hash() and rec.get("workload") == workload:
                        return rec
    except OSError:
        pass
    return None


def fill_pools(dc: DeviceCache, seed: int):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for pool in (dc.k_pool, dc.v_pool):
        if pool is None:
            continue
        for li in range(pool.shape[0]):
            flat = pool[li].view(-1)
            step = 1 << 26
            for s in range(0, flat.numel(), step):
                n = min(step, flat.numel() - s)
                flat[s:s + n] = torch.randn(n, generator=g, device="cuda").to(pool.dtype)
    if dc.gdn is not None:
        dc.gdn.normal_(0.0, 1.0 / np.sqrt(128.0), generator=g)


def copy_ceiling():
    """A plain device-to-device copy of 512 MiB, best of five: read + written bytes per second."""
    src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return {"gbs": round(2 * COPY_CALIBRATION_BYTES / (best * 1e-3) / 1e9, 1), "bytes": 2 * COPY_CALIBRATION_BYTES,
            "kind": "device-to-device copy of 512 MiB (read + write), best of 6, HIP events"}


# ---------------------------------------------------------------------------- algorithmic bytes
def layer_weight_bytes(cfg, i):
    H, F = cfg.hidden, cfg.ffn
    if cfg.layer_kinds[i] == "attn":
        mix = cfg.qkv_rows * H + H * cfg.n_q_heads * cfg.head_dim
    else:
        mix = cfg.gdn_in_rows * H + H * cfg.gdn_heads * cfg.gdn_dim
    return (mix + 3 * F * H) * 2


def round_bytes(cfg, lanes, k, context, committed_mean, sampled=False, rejecting=0.0):
    """Bytes a round must move: weights once, KV once per lane, staging, compaction, the
    recurrent state (verify read, commit read + write), embeddings; sampled rounds add the
    drafter's q rows the draws read."""
    ab = 2
    H, V = cfg.hidden, cfg.vocab
    R = lanes * (k + 1)
    weights = sum(layer_weight_bytes(cfg, i) for i in range(cfg.n_layers)) + V * H * ab
    kv_row = 2 * cfg.n_kv_heads * cfg.head_dim * ab
    seen = [min(context, cfg.layer_window(i) + k) if cfg.layer_window(i) else context for i in range(cfg.n_attn)]
    kv = lanes * kv_row * sum(seen)
    staging = R * kv_row * cfg.n_attn
    compaction = lanes * committed_mean * kv_row * cfg.n_attn * 2
    gdn = 3 * lanes * cfg.n_gdn * cfg.gdn_heads * cfg.gdn_dim ** 2 * 4
    embed = 0 if cfg.head_only else R * H * ab
    q = rejecting * V * 4 if sampled else 0
    return weights + kv + staging + compaction + gdn + embed + q


def gate_up_bytes(cfg, R):
    """Gate and up weights once, the float32 input rows (two bf16 planes) and the float32
    SwiGLU output rows (two bf16 planes)."""
    return 2 * cfg.ffn * cfg.hidden * 2 + R * cfg.hidden * 4 + R * cfg.ffn * 4


def lm_head_bytes(cfg, R):
    """The head's weights once and its input rows (exact bf16 rows of a head-only round,
    two bf16 planes of float32 rows after a decoder)."""
    return cfg.vocab * cfg.hidden * 2 + R * cfg.hidden * (2 if cfg.head_only else 4)


# ---------------------------------------------------------------------------- CPU baseline (oracle)
def _threads():
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = cores
    return cores, threads


def cpu_baseline_head(cfg, lanes, k, tokens_per_round, sampled, temperature):
    """The oracle's whole head-only round: the LM head on all rows, then acceptance."""
    from oracle import OracleModel, accept_greedy, accept_sampled
    cores, threads = _threads()
    R = lanes * (k + 1)
    w = synth.head_weights(cfg)
    om = OracleModel(cfg, w)
    hid = synth.hidden_states(cfg, R)
    q, d = synth.drafter_rows(cfg.input_seed, 99, R, cfg.vocab)
    t0 = time.perf_counter()
    z = om.lm_head(hid)
    for l in range(lanes):
        rows = slice(l * (k + 1), (l + 1) * (k + 1))
        drafts = [int(x) for x in d[l * (k + 1) + 1:(l + 1) * (k + 1)]]
        if sampled:
            accept_sampled(z[rows], drafts, q[l * (k + 1) + 1:(l + 1) * (k + 1)], temperature, cfg.philox_seed, l,
                           cfg.context)
        else:
            accept_greedy(z[rows], drafts)
    t = time.perf_counter() - t0
    return {"value": lanes * tokens_per_round / t, "unit": "tokens/s", "cores": cores, "threads": threads,
            "kind": "oracle",
            "sample": f"one whole round: LM head {cfg.vocab} x {cfg.hidden} on {R} rows + acceptance of {lanes} "
                      f"lanes, {t:.2f} s"}


def cpu_baseline_decoder(cfg, lanes, k, context, tokens_per_round):
    """The oracle on a bounded sample of the same round: one decoder layer of each kind and
    the LM head for all rows, at full width and context, extrapolated to the model's depth
    (a whole round of the 64-layer model takes minutes on the host)."""
    from oracle import KVCache, OracleModel
    cores, threads = _threads()
    kinds = sorted(set(cfg.layer_kinds))
    per_kind = {}
    t_head = None
    for kind in kinds:
        one = cfg.with_(n_layers=1, layer_kinds=(kind,), sliding_window=0)
        log(f"cpu baseline: generating a 1-layer {kind} sample")
        w = synth.model_weights(one)
        om = OracleModel(one, w, keep_f64=False)          # streamed weights, as a deep oracle runs
        blocks = (context + 16) // 16 + 1
        bt, nb = synth.block_table(one, lanes, blocks)
        oc = KVCache(kv_len=np.full(lanes, context, np.int64), block_table=bt.astype(np.int64), block=16)
        if kind == "attn":
            oc.pool_k.append(np.zeros((nb, 16, one.n_kv_heads, one.head_dim), np.float32))
            oc.pool_v.append(np.zeros_like(oc.pool_k[0]))
            for l in range(lanes):
                kk, vv = synth.kv_context(one, 0, l, context)
                oc.scatter(0, l, 0, kk, vv)
        else:
            oc.gdn.append(np.stack([synth.gdn_state(one, 0, l) for l in range(lanes)]))
        toks = [[int(t) for t in synth.uniform_tokens(one.input_seed, 40 + l, k + 1, one.vocab)]
                for l in range(lanes)]
        log(f"cpu baseline: timing one {kind} layer + LM head")
        t0 = time.perf_counter()
        res = om.verify_round(oc, toks)
        t_all = time.perf_counter() - t0
        t0 = time.perf_counter()
        om.lm_head(res.hidden)
        t_h = time.perf_counter() - t0
        per_kind[kind] = max(t_all - t_h, 1e-9)
        t_head = t_h if t_head is None else min(t_head, t_h)
    n_kind = {kd: sum(1 for x in cfg.layer_kinds if x == kd) for kd in kinds}
    t_round = sum(n_kind[kd] * per_kind[kd] for kd in kinds) + t_head
    tok_s = lanes * tokens_per_round / t_round
    parts = ", ".join(f"{per_kind[kd]:.2f} s per {kd} layer x {n_kind[kd]}" for kd in kinds)
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "threads": threads, "kind": "oracle",
            "sample": f"extrapolated: 1 layer of each kind + LM head timed at {lanes} lanes x {k + 1} rows, context "
                      f"{context}; {parts}, {t_head:.2f} s LM head -> a {t_round:.1f} s round"}


# ---------------------------------------------------------------------------- profiling helpers
def _profile_class(dm, cls, every):
    B.spec_profile_enable(dm.handle, cls, every)


def _collect(dm):
    ms, n = B.spec_profile_collect(dm.handle)
    B.spec_profile_enable(dm.handle, B.SPEC_K_NONE, 1)
    return ms / max(n, 1), n


def _roofline(name, nbytes, avg_ms, launches, traffic=None):
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "avg_launch_ms": round(avg_ms, 5),
            "launches": launches, "bytes_per_launch": nbytes}


def _base_result(cfg, args, L, k, R, ctx, mode, committed_total, elapsed, steps, extra_workload=""):
    ms_step = elapsed / steps * 1e3
    return {
        "metric": METRIC, "value": round(committed_total / elapsed, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload_name(cfg, L, k, R, ctx, mode) + extra_workload,
                   "lanes": L, "k": k, "rows": R, "context": ctx, "mode": mode,
                   **({"attn_chunk": args.chunk_used} if getattr(args, "chunk_used", 0) else {})},
        "verify_rows_per_s": round(R * steps / elapsed, 1),
    }


def workload_name(cfg, L, k, R, ctx, mode):
    if cfg.head_only:
        return (f"{cfg.name}: LM head {cfg.vocab} x {cfg.hidden} bf16 + acceptance on {R} given hidden states, "
                f"{L} lanes x (k={k} + 1), {mode}")
    kinds = (f"{cfg.n_layers}-layer dense bf16 decoder" if not cfg.n_gdn else
             f"{cfg.n_layers}-layer hybrid bf16 decoder ({cfg.n_gdn} gated-delta-rule, {cfg.n_attn} GQA)")
    return (f"{cfg.name}: {kinds} H{cfg.hidden}, {cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}, "
            f"FFN {cfg.ffn}, vocab {cfg.vocab}; {L} lanes x (k={k} + 1) = {R} rows, context {ctx}, {mode}")


# ---------------------------------------------------------------------------- LM head + acceptance only
def run_head(args, cfg):
    L, k = args.lanes, args.k
    R = L * (k + 1)
    steps, warm = args.steps, args.warmup
    sampled = args.sampled > 0
    log(f"{cfg.name}: weights on the device")
    w = gpu_weights(cfg, cfg.weight_seed)
    dm = DeviceModel(cfg, w, prepacked=True)
    del w
    dc = DeviceCache(dm, L, 1, 1, kv_len=[cfg.context] * L)
    g = torch.Generator(device="cuda").manual_seed(cfg.input_seed)
    hid = torch.randn((R, cfg.hidden), generator=g, device="cuda").to(torch.bfloat16)
    # the drafter: seeded softmax rows q (logits N(0, 2)), each draft drawn from its row
    qd = torch.softmax(2.0 * torch.randn((R, cfg.vocab), generator=g, device="cuda"), dim=-1)
    drafts = torch.multinomial(qd, 1, generator=g).view(-1).to(torch.int32)
    toks = drafts.clone()
    toks[0::k + 1] = torch.arange(L, dtype=torch.int32, device="cuda")    # anchors (unused by a head-only round)
    kw = dict(mode="sampled", temperature=args.sampled, q_probs=qd) if sampled else {}
    rc = dc.round([[0] * (k + 1)] * L, tokens_dev=toks, seed=cfg.philox_seed, **kw)
    committed_log = []
    com_host = torch.empty(L, dtype=torch.int32).pin_memory()

    def step(i):
        rc.r.seed = cfg.philox_seed + i
        dc.verify_head(rc, hid)
        dc.accept(rc, stats=False)
        com_host.copy_(dc.committed)        # the per-round device -> host crossing (blocking)
        committed_log.append(com_host.numpy().copy())

    log(f"warmup {warm} steps")
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    committed_log.clear()
    _profile_class(dm, B.SPEC_K_LM_HEAD, 1)
    log(f"timed {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warm + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    head_ms, head_n = _collect(dm)
    committed = np.array(committed_log)
    mode = f"sampled T {args.sampled}" if sampled else "greedy"
    res = _base_result(cfg, args, L, k, R, cfg.context, mode, int(committed.sum()), elapsed, steps,
                       ", drafts drawn from seeded drafter rows q = softmax(N(0, 2) logits)")
    tpr = float(committed.mean())
    rejecting = float((committed <= k).mean()) * L
    rb = round_bytes(cfg, L, k, 0, tpr, sampled, rejecting)
    res["tokens_per_round"] = round(tpr, 3)
    res["round_roofline_frac"] = round(rb / (elapsed / steps) / 1e9 / HBM_PEAK_GBS, 4)
    res["roofline"] = _roofline("LM head" + (" (sampled: cooperative, decisions and draws on chip)" if sampled
                                             else " (greedy statistics)"), lm_head_bytes(cfg, R), head_ms, head_n)
    res["copy_ceiling"] = copy_ceiling()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_head(cfg, L, k, tpr, sampled, args.sampled)
    dm.close()
    return res


# ---------------------------------------------------------------------------- decoder rounds
def run_decoder(args, cfg):
    L, k, ctx = args.lanes, args.k, args.context
    R = L * (k + 1)
    steps, warm = args.steps, args.warmup
    sampled = args.sampled > 0
    total_rounds = steps + warm
    ref_len = total_rounds * (k + 1) + 2
    max_blocks = (ctx + ref_len + 32) // 16 + 1
    log(f"{cfg.name}: weights on the device")
    w = gpu_weights(cfg, cfg.weight_seed)
    # split-KV chunk by workgroup count (at context 8192: 1024 for 8 lanes, 512 for one lane;
    # measured 15.4 against 15.9 ms a round at 8 lanes, 10.2 against 10.7 ms at one lane)
    chunk = args.attn_chunk or attn_chunk_for(cfg.n_kv_heads, L, ctx, args.window)
    args.chunk_used = chunk
    dm = DeviceModel(cfg, w, prepacked=True, attn_chunk=chunk)
    del w
    bt, nb = synth.block_table(cfg, L, max_blocks)
    dc = DeviceCache(dm, L, max_blocks, nb, block_table=bt, kv_len=[ctx] * L)
    log("KV context and recurrent state")
    fill_pools(dc, cfg.input_seed)
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda") if args.evict_mall else None
    if args.copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    anchors = [int(t) for t in synth.uniform_tokens(cfg.input_seed, 5, L, cfg.vocab)]
    pen, counts0 = {}, None
    if args.penalties:
        pres, freq = (float(x) for x in args.penalties.split(","))
        # each lane's counts: a seeded history as long as the context, then its anchor
        hist = np.stack([np.append(synth.uniform_tokens(cfg.input_seed, 300 + l, ctx, cfg.vocab), anchors[l])
                         for l in range(L)])
        counts0 = torch.from_numpy(np.stack([np.bincount(h, minlength=cfg.vocab) for h in hist]).astype(np.int32))
        counts0 = counts0.cuda()
        pen = {"counts": counts0.clone(), "presence": pres, "frequency": freq}

    def add_counts():
        if pen:
            B.spec_counts_add(pen["counts"].data_ptr(), cfg.vocab, L, dc.committed.data_ptr(),
                              dc.out_tokens.data_ptr(), dc.out_tokens.shape[1], torch.cuda.current_stream().cuda_stream)

    # reference plain-greedy continuation (one row per lane per round); also the plain-round timing
    n_plain = ref_len if (not sampled and args.drafter == "planted") else 2 + max(1, args.plain_steps)
    log(f"reference continuation: {n_plain} plain rounds")
    ref = np.zeros((L, n_plain + 1), np.int64)
    ref[:, 0] = anchors
    cur = torch.tensor(anchors, dtype=torch.int32, device="cuda")
    plain_times = []
    for s in range(n_plain):
        rc = dc.round([[0]] * L, tokens_dev=cur, **pen)
        if evict is not None:
            evict.fill_(s & 255)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dc.verify(rc)
        dc.accept(rc, stats=False)
        dc.commit(rc)
        add_counts()
        nxt = dc.out_tokens[:, 0].clone()
        torch.cuda.synchronize()
        plain_times.append(time.perf_counter() - t0)
        ref[:, s + 1] = nxt.cpu().numpy()
        cur = nxt
    plain_ms = float(np.median(plain_times[2:2 + max(1, args.plain_steps)]) * 1e3)
    dc.set_kv_len([ctx] * L)
    if pen:
        pen["counts"].copy_(counts0)
    if cfg.n_gdn:
        fill_pools(dc, cfg.input_seed)      # the plain rounds advanced the recurrent state: start again

    if args.drafter == "ngram":
        return run_ngram(args, cfg, dm, dc, anchors, plain_ms)

    # planted drafts (greedy): slot i matches the reference with probability alpha_i
    alpha = np.linspace(0.9, 0.35, k) if k else np.zeros(0)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.input_seed, 77])))
    pos = np.zeros(L, np.int64)          # tokens committed so far per lane (ref[l, pos] is the anchor)
    planted_hits = []                    # per step: [L] leading planted hits (the expected kept drafts)

    def draw_plant():
        # one step's planted decisions, drawn lane by lane and slot by slot: a miss (and the
        # offset of its planted token) depends on the draw alone, not on where the lane stands,
        # so a step's draw is taken while the previous round still runs on the device
        miss = np.zeros((L, k), bool)
        off = np.zeros((L, k), np.int64)
        for l in range(L):
            for i in range(k):
                if rng.random() >= alpha[i]:
                    miss[l, i] = True
                    off[l, i] = int(rng.integers(0, cfg.vocab - 1))
        # leading planted hits per lane: the drafts a correct round keeps
        lead = np.where(miss.any(axis=1), miss.argmax(axis=1), k)
        return miss, off, lead

    lane_ix = np.arange(L)[:, None]
    slot_ix = np.arange(1, k + 1)[None, :]

    qsets = None
    if sampled:
        # the drafter: seeded softmax rows q (logits N(0, 2)), each draft drawn from its
        # row; a pool of four (q, drafts) sets made before the timed steps, used in turn
        gq = torch.Generator(device="cuda").manual_seed(cfg.input_seed + 5)
        qsets = []
        for _ in range(4):
            qd = torch.softmax(2.0 * torch.randn((R, cfg.vocab), generator=gq, device="cuda"), dim=-1)
            dr = torch.multinomial(qd, 1, generator=gq).view(L, k + 1)[:, 1:].cpu().numpy()
            qsets.append((qd, dr))
    n_step = [0]
    tok_host = torch.empty(R, dtype=torch.int32).pin_memory()
    tok_dev = torch.empty(R, dtype=torch.int32, device="cuda")
    com_host = torch.empty(L, dtype=torch.int32).pin_memory()
    out_host = torch.empty(tuple(dc.out_tokens.shape), dtype=dc.out_tokens.dtype).pin_memory()
    tok_np, com_np, out_np = tok_host.numpy(), com_host.numpy(), out_host.numpy()
    committed_log = []
    anchor = np.array(anchors, np.int64)
    ev_pairs = []
    # the round descriptor is the same every step (the tokens are rewritten in place);
    # sampled steps change only the drafter rows and the seed
    rc = dc.round([[0] * (k + 1)] * L, tokens_dev=tok_dev, **pen,
                  **({"mode": "sampled", "temperature": args.sampled, "q_probs": qsets[0][0]} if sampled else {}))
    plant = [None if sampled else draw_plant()]

    def step(timed):
        if sampled:
            qd, dr = qsets[n_step[0] % len(qsets)]
            toks = np.concatenate([anchor[:, None], dr.astype(np.int64)], axis=1)
            rc.q = qd
            rc.r.q_probs = qd.data_ptr()
            rc.r.seed = 1000 + n_step[0]
            lead = None
        else:
            miss, off, lead = plant[0]
            cur = ref[lane_ix, pos[:, None] + slot_ix]
            toks = np.concatenate([ref[lane_ix[:, 0], pos][:, None],
                                   np.where(miss, (cur + 1 + off) % cfg.vocab, cur)], axis=1)
        tok_np[:] = toks.reshape(-1)
        tok_dev.copy_(tok_host, non_blocking=True)
        n_step[0] += 1
        if evict is not None:
            evict.fill_(n_step[0] & 255)    # outside the round's events: the cache holds no weights
        a = b = None
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
        dc.verify(rc)
        dc.accept(rc, stats=False)
        dc.commit(rc)
        add_counts()
        if timed:
            b.record()
            ev_pairs.append((a, b))
        if not sampled:
            plant[0] = draw_plant()         # the next step's draw, while this round runs
        # the per-round device -> host crossing (the drafter's input), a blocking copy into
        # pinned memory that also waits for the round
        com_host.copy_(dc.committed)
        if sampled:
            out_host.copy_(dc.out_tokens)
        c = com_np.astype(np.int64)
        if sampled:
            anchor[:] = out_np[np.arange(L), c - 1]
        pos[:] += c
        committed_log.append(c)
        planted_hits.append(lead)

    log(f"warmup {warm} steps")
    for _ in range(warm):
        step(False)
    torch.cuda.synchronize()
    committed_log.clear()
    planted_hits.clear()
    # every 8th gate/up launch carries a pair of HIP events (8 per round at 64 layers): an
    # event pair around every launch would add its queue gap to every launch of the round
    every = max(1, cfg.n_layers // 8)
    _profile_class(dm, B.SPEC_K_GATE_UP, every)
    log(f"timed {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(evict is not None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gu_avg_ms, gu_n = _collect(dm)
    timing = "wall clock over the timed steps"
    if evict is not None:      # the rounds alone: the eviction writes between them are not timed
        elapsed = sum(a.elapsed_time(b) for a, b in ev_pairs) * 1e-3
        timing = "HIP events around each round (the 512 MiB eviction write between rounds excluded)"

    committed = np.array(committed_log)               # [steps, L]
    mode = f"sampled T {args.sampled}" if sampled else "greedy"
    extra = ""
    if sampled:
        extra = ", drafts drawn from seeded drafter rows q = softmax(N(0, 2) logits), anchors = each lane's last " \
                "committed token"
    else:
        extra = ", drafts planted at slot acceptance 0.9..0.35"
    if pen:
        extra += f", presence/frequency penalties {pen['presence']}/{pen['frequency']} per row"
    if cfg.sliding_window:
        extra += (f", sliding window {cfg.sliding_window}" + (
            f" (every {cfg.window_global_every}th attention layer global)" if cfg.window_global_every
            else " on every attention layer"))
    if evict is not None:
        extra += ", 512 MiB written between rounds (last-level cache evicted)"
    res = _base_result(cfg, args, L, k, R, ctx, mode, int(committed.sum()), elapsed, steps, extra)
    ms_step = elapsed / steps * 1e3
    tpr = float(committed.mean())
    rejecting = float((committed <= k).mean()) * L
    res["tokens_per_round"] = round(tpr, 3)
    res["timing"] = timing
    if not sampled:
        res["textbook_tokens_per_round"] = round(1.0 + float(np.sum(np.cumprod(alpha))), 3)
        # the planted draw itself: the kept drafts it implies, and whether each lane kept exactly them
        leads = np.array(planted_hits)
        res["planted_tokens_per_round"] = round(float((leads + 1).mean()), 3)
        mism = int(np.sum(committed != leads + 1))
        res["self_check"] = {"rounds": steps, "lanes": L,
                             "committed_equals_planted_prefix_plus_one": mism == 0, "mismatched": mism,
                             "what": "each lane's committed run = the planted drafts up to the first miss + the "
                                     "reference token (the 64-row verify rows equal the plain one-row rounds)"}
        res["drafter"] = (f"planted α 0.9..0.35 · depth {k}, no gate · acceptance "
                          f"{(committed - 1).sum()}/{committed.size * k} guesses · greedy · {L} streams")
    else:
        res["drafter"] = (f"seeded random drafter rows q, drafts d ~ q · depth {k} · acceptance "
                          f"{(committed - 1).sum()}/{committed.size * k} guesses · sampled T {args.sampled} · "
                          f"{L} streams")
    res["plain_round_ms"] = round(plain_ms, 3)
    res["verify_over_plain"] = round(ms_step / plain_ms, 3)
    rb = round_bytes(cfg, L, k, ctx + int(pos.mean()), tpr, sampled, rejecting)
    res["round_bytes"] = int(rb)
    res["round_roofline_frac"] = round(rb / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    tr = measured_traffic(res["config"]["workload"].split(":")[0] + f" L{L}") if not sampled and not pen else None
    res["roofline"] = _roofline("gate/up projection (SwiGLU epilogue)", gate_up_bytes(cfg, R), gu_avg_ms, gu_n,
                                int(tr["fetch_bytes"] + tr["write_bytes"]) if tr else None)
    if cfg.n_gdn and args.gdn_profile:
        res["gdn_verify"] = gdn_timing(dm, dc, cfg, L, k, R)
    res["copy_ceiling"] = copy_ceiling()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decoder(cfg, L, k, ctx, tpr)
    dm.close()
    return res


def gdn_timing(dm, dc, cfg, L, k, R):
    """The recurrent verify kernel alone, HIP events around each of its launches over a few
    rounds: state bytes read per launch (L heads x d^2 x 4) and the inputs."""
    toks = torch.zeros(R, dtype=torch.int32, device="cuda")
    rc = dc.round([[0] * (k + 1)] * L, tokens_dev=toks)
    _profile_class(dm, B.SPEC_K_GDN, 1)
    for _ in range(3):
        dc.verify(rc)
    torch.cuda.synchronize()
    ms, n = _collect(dm)
    state = L * cfg.gdn_heads * cfg.gdn_dim ** 2 * 4
    return {"avg_launch_ms": round(ms, 5), "launches": n, "state_bytes_per_launch": state,
            "state_gbs": round(state / (ms * 1e-3) / 1e9, 1)}


def run_ngram(args, cfg, dm, dc, anchors, plain_ms):
    """Greedy rounds with drafts from the n-gram drafter on each lane's own history, as one
    sequence of device calls per timed region (no host round trip between rounds)."""
    L, k, ctx = args.lanes, args.k, args.context
    R = L * (k + 1)
    steps, warm = args.steps, args.warmup
    dc.set_kv_len([ctx] * L)
    max_len = ctx + 1 + (steps + warm) * (k + 1) + 8
    hist = torch.zeros((L, max_len), dtype=torch.int32, device="cuda")
    for l in range(L):
        hist[l, :ctx] = torch.from_numpy(synth.uniform_tokens(cfg.input_seed, 300 + l, ctx, cfg.vocab)).cuda()
        hist[l, ctx] = anchors[l]
    hlen = torch.full((L,), ctx + 1, dtype=torch.int32, device="cuda")
    log(f"n-gram loop: warmup {warm} rounds")
    dc.ngram_rounds(hist, hlen, warm, k, NGRAM_MAX)
    torch.cuda.synchronize()
    h0 = hlen.clone()
    _profile_class(dm, B.SPEC_K_GATE_UP, max(1, cfg.n_layers // 8))
    log(f"n-gram loop: timed {steps} rounds")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dc.ngram_rounds(hist, hlen, steps, k, NGRAM_MAX)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gu_avg_ms, gu_n = _collect(dm)
    committed = int((hlen - h0).sum())
    tpr = committed / (steps * L)
    res = _base_result(cfg, args, L, k, R, ctx, "greedy", committed, elapsed, steps,
                       f", drafts from the n-gram drafter (n {NGRAM_MAX}..1) on each lane's own history, "
                       f"device-side loop")
    ms_step = elapsed / steps * 1e3
    res["tokens_per_round"] = round(tpr, 3)
    res["drafter"] = (f"n-gram prompt lookup (n {NGRAM_MAX}..1) on each lane's history: {ctx} uniform random context "
                      f"tokens + the generated text; k = {k} guesses every round (the anchor as filler where no "
                      f"suffix recurs); {committed - steps * L}/{steps * L * k} guesses kept")
    res["plain_round_ms"] = round(plain_ms, 3)
    res["verify_over_plain"] = round(ms_step / plain_ms, 3)
    rb = round_bytes(cfg, L, k, ctx, tpr)
    res["round_roofline_frac"] = round(rb / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    res["roofline"] = _roofline("gate/up projection (SwiGLU epilogue)", gate_up_bytes(cfg, R), gu_avg_ms, gu_n)
    res["copy_ceiling"] = copy_ceiling()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decoder(cfg, L, k, ctx, tpr)
    dm.close()
    return res


# ---------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="dense-27b", choices=("dense-27b", "head-v151936", "mid-bf16", "hybrid-gdn"))
    ap.add_argument("--lanes", type=int, default=0, help="default: the config's lanes")
    ap.add_argument("--k", type=int, default=-1, help="default: the config's drafts per lane")
    ap.add_argument("--context", type=int, default=-1, help="default: the config's context")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--plain-steps", type=int, default=10, help="plain one-row rounds timed for comparison")
    ap.add_argument("--drafter", choices=("planted", "ngram"), default="planted",
                    help="planted drafts (default) or the n-gram drafter on each lane's own history")
    ap.add_argument("--penalties", default=None, metavar="PRESENCE,FREQUENCY",
                    help="per-row presence and frequency penalties on every round (plain ones too), with "
                         "each lane's counts kept on the device; the lanes' histories are seeded tokens")
    ap.add_argument("--sampled", type=float, default=0.0, metavar="T",
                    help="sampled verify at temperature T (textbook rule) against seeded drafter rows")
    ap.add_argument("--evict-mall", action="store_true",
                    help="write 512 MiB between rounds (untimed) so the last-level cache holds no weights")
    ap.add_argument("--gdn-profile", action="store_true", help="hybrid: also time the recurrent verify kernel")
    ap.add_argument("--attn-chunk", type=int, default=0,
                    help="positions per split-KV chunk (default 1024 at >= 4K context, else 512)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window target: attention layers see their last W positions")
    ap.add_argument("--window-global-every", type=int, default=0,
                    help="with --window, every g-th attention layer keeps full attention")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of 512 MiB (the reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; the verify round does not shard "
                                   "(--gpus must be 1)"}))
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs one process on one GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    cfg = synth.get_config(args.config)
    if args.window:
        cfg = cfg.with_(sliding_window=args.window, window_global_every=args.window_global_every)
    args.lanes = args.lanes or cfg.lanes
    args.k = cfg.k if args.k < 0 else args.k
    args.context = cfg.context if args.context < 0 else args.context
    if args.drafter == "ngram" and (args.sampled > 0 or args.penalties):
        print("--drafter ngram runs greedy rounds without penalties", file=sys.stderr)
        sys.exit(2)
    if cfg.head_only:
        if args.drafter != "planted" or args.penalties or args.window or args.evict_mall:
            print("the head-only workload takes --sampled only", file=sys.stderr)
            sys.exit(2)
        result = run_head(args, cfg)
    else:
        result = run_decoder(args, cfg)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
