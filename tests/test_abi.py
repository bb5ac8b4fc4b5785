"""The C-ABI library: exports, the host-side planner and host-side validation (no GPU needed).

Every call below returns before anything is enqueued, so no device work runs.
"""
import ctypes as C
import os
import re

import pytest

from oracle import plan_drafts
from speculative_decoding_verify_round_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "spec_verify.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_library_exports_every_header_function():
    lib = B.load_library()
    names = header_functions()
    assert names == sorted(B.HEADER_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert B.spec_status_string(s) != "unknown status"
    assert B.spec_status_string(-99) == "unknown status"


def test_planner_matches_oracle_exhaustively():
    for k in range(0, 17):
        for budget in range(0, 65):
            for lanes in range(1, 65):
                assert B.spec_plan_drafts(k, budget, lanes) == plan_drafts(k, budget, lanes)
    assert B.spec_plan_drafts(3, 8, 0) == B.SPEC_E_INVAL
    assert B.spec_plan_drafts(-1, 8, 1) == B.SPEC_E_INVAL
    assert B.spec_plan_drafts(3, -1, 1) == B.SPEC_E_INVAL


FAKE = 0x1000   # never dereferenced: every call here fails validation before any launch


def make_desc(**kw):
    d = B.SpecModelDesc()
    d.n_layers = kw.get("n_layers", 2)
    d.hidden, d.head_dim = kw.get("hidden", 256), kw.get("head_dim", 128)
    d.n_q_heads, d.n_kv_heads = kw.get("q_heads", 4), kw.get("kv_heads", 2)
    d.ffn, d.vocab = kw.get("ffn", 512), kw.get("vocab", 1024)
    d.dtype = kw.get("dtype", B.SPEC_BF16)
    kinds = kw.get("kinds", [B.SPEC_LAYER_ATTN] * d.n_layers)
    arr = (C.c_int32 * max(1, len(kinds)))(*kinds)
    d.layer_kind = C.cast(arr, C.POINTER(C.c_int32))
    d.gdn_heads, d.gdn_dim = kw.get("gdn_heads", 0), kw.get("gdn_dim", 0)
    d.rms_eps, d.rope_theta, d.kv_block, d.attn_chunk = 1e-6, 1e4, kw.get("kv_block", 16), kw.get("chunk", 0)
    d.embed, d.lm_head, d.final_norm = FAKE, kw.get("lm_head", FAKE), FAKE
    lw = (B.SpecLayerWeights * max(1, d.n_layers))()
    for i in range(d.n_layers):
        lw[i] = B.SpecLayerWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    d.layers = C.cast(lw, C.POINTER(B.SpecLayerWeights))
    d.sliding_window, d.window_global_every = kw.get("sliding_window", 0), kw.get("window_global_every", 0)
    d._keep = (arr, lw)
    return d


def create_status(**kw):
    h = C.c_void_p()
    st = B.load_library().spec_model_create(C.byref(make_desc(**kw)), C.byref(h))
    if st == 0:
        B.spec_model_destroy(h)
    return st


def test_model_create_validation():
    assert create_status() == B.SPEC_OK
    assert create_status(vocab=1000) == B.SPEC_E_INVAL             # vocab not a multiple of 16
    assert create_status(dtype=7) == B.SPEC_E_INVAL
    assert create_status(kv_block=32) == B.SPEC_E_UNSUPPORTED
    assert create_status(lm_head=None) == B.SPEC_E_INVAL
    assert create_status(hidden=200) == B.SPEC_E_UNSUPPORTED        # bf16 hidden must be a multiple of 256
    assert create_status(hidden=8448) == B.SPEC_E_UNSUPPORTED       # row kernels hold at most 8192 per row
    assert create_status(head_dim=64) == B.SPEC_E_UNSUPPORTED       # bf16 attention runs head_dim 128
    assert create_status(dtype=B.SPEC_F32, hidden=200, head_dim=64, ffn=100) == B.SPEC_OK
    assert create_status(kinds=[0, 5]) == B.SPEC_E_INVAL
    assert create_status(kinds=[1, 0], gdn_heads=2, gdn_dim=64) == B.SPEC_E_UNSUPPORTED
    assert create_status(kinds=[1, 0], gdn_heads=2, gdn_dim=128) == B.SPEC_OK
    assert create_status(chunk=300) == B.SPEC_E_UNSUPPORTED
    assert create_status(n_layers=0, kinds=[]) == B.SPEC_OK      # LM head only


@pytest.fixture
def model():
    h = C.c_void_p()
    desc = make_desc(kinds=[B.SPEC_LAYER_GDN, B.SPEC_LAYER_ATTN], gdn_heads=2, gdn_dim=128)
    assert B.load_library().spec_model_create(C.byref(desc), C.byref(h)) == 0
    yield h
    B.spec_model_destroy(h)


def test_workspace_bytes(model):
    lib = B.load_library()
    a = lib.spec_workspace_bytes(model, 1, 4, 8)
    b = lib.spec_workspace_bytes(model, 8, 8, 600)
    assert 0 < a < b
    assert lib.spec_workspace_bytes(model, 0, 4, 8) == B.SPEC_E_INVAL
    assert lib.spec_workspace_bytes(model, 1, 17, 8) == B.SPEC_E_INVAL
    assert lib.spec_workspace_bytes(None, 1, 4, 8) == B.SPEC_E_INVAL


def make_round(model, **kw):
    lanes = kw.get("lanes", 2)
    cols = kw.get("cols", [4] * lanes)
    colsa = (C.c_int32 * max(1, len(cols)))(*cols)
    r = B.SpecRound()
    r.lanes = lanes
    r.cols_host = C.cast(colsa, C.POINTER(C.c_int32))
    r.tokens = kw.get("tokens", FAKE)
    r.kv_len = FAKE
    kvh = kw.get("kv_len_host")
    kva = (C.c_int32 * lanes)(*kvh) if kvh else None
    r.kv_len_host = C.cast(kva, C.POINTER(C.c_int32)) if kva else None
    r.block_table, r.max_blocks, r.k_pool, r.v_pool, r.n_blocks = FAKE, kw.get("max_blocks", 4), FAKE, FAKE, 16
    r.gdn_state = kw.get("gdn_state", FAKE)
    r.mode = kw.get("mode", B.SPEC_GREEDY)
    r.temperature = kw.get("temperature", 1.0)
    r.q_probs = kw.get("q_probs", None)
    r.seed = 1
    r.workspace = kw.get("workspace", 0x100000)
    r.workspace_bytes = kw.get("workspace_bytes", 1 << 40)
    r._keep = (colsa, kva)
    return r


def verify_status(model, **kw):
    return B.load_library().spec_verify_round(model, C.byref(make_round(model, **kw)), None)


def test_round_validation_errors(model):
    assert verify_status(model, lanes=0, cols=[]) == B.SPEC_E_INVAL
    assert verify_status(model, cols=[4, 0]) == B.SPEC_E_INVAL
    assert verify_status(model, cols=[4, 17]) == B.SPEC_E_INVAL
    assert verify_status(model, lanes=5, cols=[16] * 5) == B.SPEC_E_INVAL       # 80 rows > 64
    assert verify_status(model, tokens=None) == B.SPEC_E_INVAL
    assert verify_status(model, mode=B.SPEC_SAMPLED) == B.SPEC_E_INVAL           # no q_probs
    assert verify_status(model, mode=B.SPEC_SAMPLED, q_probs=FAKE, temperature=0.0) == B.SPEC_E_INVAL
    assert verify_status(model, mode=3) == B.SPEC_E_INVAL
    assert verify_status(model, kv_len_host=[61, 0]) == B.SPEC_E_RANGE           # 61 + 4 > 4 blocks * 16
    assert verify_status(model, kv_len_host=[-1, 0]) == B.SPEC_E_INVAL
    assert verify_status(model, gdn_state=None) == B.SPEC_E_UNSUPPORTED          # recurrent state refused
    assert verify_status(model, workspace_bytes=16) == B.SPEC_E_WORKSPACE
    assert verify_status(model, workspace=None) == B.SPEC_E_WORKSPACE
    assert verify_status(model, workspace=0x100010) == B.SPEC_E_WORKSPACE        # misaligned


def test_query_rows_per_lane_limit():
    # a chunk partial holds 64 query rows: cols x (q heads per kv head) above 64 is refused
    h = C.c_void_p()
    desc = make_desc(dtype=B.SPEC_F32, head_dim=8, q_heads=32, kv_heads=2)   # 16 q heads per kv head
    assert B.load_library().spec_model_create(C.byref(desc), C.byref(h)) == 0
    try:
        assert verify_status(h, cols=[5, 1]) == B.SPEC_E_UNSUPPORTED            # 80 query rows
    finally:
        B.spec_model_destroy(h)


def test_other_calls_validate(model):
    lib = B.load_library()
    r = make_round(model, lanes=0, cols=[])
    assert lib.spec_accept(model, C.byref(r), FAKE, FAKE, None, None) == B.SPEC_E_INVAL
    assert lib.spec_commit(model, C.byref(r), FAKE, None) == B.SPEC_E_INVAL
    assert lib.spec_debug_logits(model, C.byref(r), FAKE, None) == B.SPEC_E_INVAL
    r = make_round(model)
    assert lib.spec_accept(model, C.byref(r), None, FAKE, None, None) == B.SPEC_E_INVAL
    assert lib.spec_commit(model, C.byref(r), None, None) == B.SPEC_E_INVAL
    assert lib.spec_verify_head(model, C.byref(r), None, None) == B.SPEC_E_INVAL
    assert lib.spec_debug_gemm(model, FAKE, FAKE, FAKE, 0, 16, 256, None, 0, None) == B.SPEC_E_INVAL
    assert lib.spec_debug_gemm(model, FAKE, FAKE, FAKE, 8, 16, 100, None, 0, None) == B.SPEC_E_UNSUPPORTED
    assert lib.spec_profile_enable(model, 99, 1) == B.SPEC_E_INVAL
    assert lib.spec_debug_barrier_spin(model, -1) == B.SPEC_E_INVAL
    assert lib.spec_debug_barrier_spin(None, 5) == B.SPEC_E_INVAL
    assert lib.spec_debug_barrier_spin(model, 0) == B.SPEC_OK
    assert lib.spec_profile_enable(model, B.SPEC_K_GATE_UP, 0) == B.SPEC_E_INVAL


def test_pack_weight_sizes_and_validation():
    """Packed size = 16 ceil(N / 16) K bf16 elements; bad shapes are refused before any HIP call."""
    lib = B.load_library()
    assert lib.spec_packed_weight_bytes(16, 256) == 16 * 256 * 2
    assert lib.spec_packed_weight_bytes(17, 256) == 32 * 256 * 2
    assert lib.spec_packed_weight_bytes(151936, 5120) == 151936 * 5120 * 2
    assert lib.spec_packed_weight_bytes(0, 256) == B.SPEC_E_INVAL
    assert lib.spec_packed_weight_bytes(16, 300) == B.SPEC_E_INVAL
    assert lib.spec_pack_weight(None, FAKE, 16, 256, None) == B.SPEC_E_INVAL
    assert lib.spec_pack_weight(FAKE, FAKE, 16, 256, None) == B.SPEC_E_INVAL      # in place
    assert lib.spec_pack_weight(FAKE, FAKE + 64, 16, 100, None) == B.SPEC_E_INVAL


def test_ngram_calls_validate():
    """The drafter and history calls refuse bad sizes and null buffers before any HIP call."""
    lib = B.load_library()
    bad = [
        (None, FAKE, 2, 64, 3, 3, 1, FAKE, FAKE, None),
        (FAKE, FAKE, 0, 64, 3, 3, 1, FAKE, FAKE, None),              # lanes
        (FAKE, FAKE, B.SPEC_MAX_LANES + 1, 64, 3, 3, 1, FAKE, FAKE, None),
        (FAKE, FAKE, 2, 0, 3, 3, 1, FAKE, FAKE, None),               # max_len
        (FAKE, FAKE, 2, 64, -1, 3, 1, FAKE, FAKE, None),             # k
        (FAKE, FAKE, 2, 64, B.SPEC_MAX_COLS, 3, 1, FAKE, FAKE, None),
        (FAKE, FAKE, 2, 64, 3, 3, 0, FAKE, FAKE, None),              # n_min
        (FAKE, FAKE, 2, 64, 3, 2, 3, FAKE, FAKE, None),              # n_max < n_min
        (FAKE, FAKE, 2, 64, 3, B.SPEC_MAX_NGRAM + 1, 1, FAKE, FAKE, None),
        (FAKE, FAKE, 2, 64, 3, 3, 1, None, FAKE, None),
    ]
    for args in bad:
        assert lib.spec_ngram_draft(*args) == B.SPEC_E_INVAL, args
    assert lib.spec_history_append(None, FAKE, 2, 64, FAKE, FAKE, 16, None) == B.SPEC_E_INVAL
    assert lib.spec_history_append(FAKE, FAKE, 0, 64, FAKE, FAKE, 16, None) == B.SPEC_E_INVAL
    assert lib.spec_history_append(FAKE, FAKE, 2, 0, FAKE, FAKE, 16, None) == B.SPEC_E_INVAL
    assert lib.spec_history_append(FAKE, FAKE, 2, 64, FAKE, FAKE, 0, None) == B.SPEC_E_INVAL
    assert lib.spec_history_append(FAKE, FAKE, 2, 64, None, FAKE, 16, None) == B.SPEC_E_INVAL


def test_penalty_fields_validate(model):
    """Non-finite penalties or a misaligned counts buffer are refused; counts_add refuses bad sizes."""
    lib = B.load_library()
    for pres, freq in ((float("nan"), 0.1), (0.1, float("inf"))):
        r = make_round(model)
        r.counts, r.presence_penalty, r.frequency_penalty = FAKE, pres, freq
        assert lib.spec_verify_round(model, C.byref(r), None) == B.SPEC_E_INVAL
        assert lib.spec_accept(model, C.byref(r), FAKE, FAKE, None, None) == B.SPEC_E_INVAL
    r = make_round(model)
    r.counts, r.presence_penalty, r.frequency_penalty = FAKE + 4, 0.1, 0.1     # not 16-byte aligned
    assert lib.spec_verify_round(model, C.byref(r), None) == B.SPEC_E_INVAL
    assert lib.spec_counts_add(None, 100, 2, FAKE, FAKE, 16, None) == B.SPEC_E_INVAL
    assert lib.spec_counts_add(FAKE, 0, 2, FAKE, FAKE, 16, None) == B.SPEC_E_INVAL
    assert lib.spec_counts_add(FAKE, 100, 0, FAKE, FAKE, 16, None) == B.SPEC_E_INVAL
    assert lib.spec_counts_add(FAKE, 100, 2, FAKE, FAKE, 0, None) == B.SPEC_E_INVAL


def test_window_fields_and_live_block():
    """Negative window settings are refused; the first block a windowed round reads is the
    64-position stage holding the lowest window start, kv_len - W + 1."""
    assert create_status(sliding_window=-1) == B.SPEC_E_INVAL
    assert create_status(window_global_every=-2) == B.SPEC_E_INVAL
    lib = B.load_library()
    assert lib.spec_window_live_block(-1, 8) == B.SPEC_E_INVAL
    assert lib.spec_window_live_block(10, -1) == B.SPEC_E_INVAL
    assert lib.spec_window_live_block(5000, 0) == 0
    for kv, W in ((0, 16), (100, 200), (300, 100), (700, 100), (8192, 1024), (64, 1), (63, 1)):
        lo = max(0, kv - W + 1)
        assert lib.spec_window_live_block(kv, W) == (lo // 64) * 4, (kv, W)


def test_noalloc_head_validates_before_any_device_call():
    """The no-allocation head round refuses bad arguments, and a round larger than the static
    scratch, before it looks up the scratch or enqueues anything."""
    lib = B.load_library()
    h = C.c_void_p()
    desc = make_desc(n_layers=0, kinds=[], vocab=1 << 20)      # greedy LM-head partials of 16.8 MB
    assert lib.spec_model_create(C.byref(desc), C.byref(h)) == 0
    try:
        r = make_round(h, lanes=8, cols=[8] * 8, workspace=None, workspace_bytes=0)
        assert lib.spec_verify_head_noalloc(h, C.byref(r), FAKE, FAKE, FAKE, None, None) == B.SPEC_E_SCRATCH
        assert lib.spec_verify_head_noalloc(h, C.byref(r), None, FAKE, FAKE, None, None) == B.SPEC_E_INVAL
        assert lib.spec_verify_head_noalloc(h, C.byref(r), FAKE, None, FAKE, None, None) == B.SPEC_E_INVAL
        r = make_round(h, lanes=0, cols=[])
        assert lib.spec_verify_head_noalloc(h, C.byref(r), FAKE, FAKE, FAKE, None, None) == B.SPEC_E_INVAL
        r = make_round(h, mode=B.SPEC_SAMPLED)                   # sampled without q
        assert lib.spec_verify_head_noalloc(h, C.byref(r), FAKE, FAKE, FAKE, None, None) == B.SPEC_E_INVAL
    finally:
        B.spec_model_destroy(h)
