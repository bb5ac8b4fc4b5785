"""ctypes binding of libspecverify.so: the C calls under the same names.

Argument marshalling only: every step of the verify round runs in the HIP
kernels behind these calls.  Structures mirror include/spec_verify.h.
The library is never built or replaced here; build it with
`python -m speculative_decoding_verify_round_amd.build`.
"""
import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_MAX_ROWS = 64
SPEC_MAX_COLS = 16
SPEC_MAX_LANES = 64
SPEC_KV_BLOCK = 16

SPEC_OK, SPEC_E_INVAL, SPEC_E_RANGE, SPEC_E_UNSUPPORTED, SPEC_E_WORKSPACE, SPEC_E_HIP, SPEC_E_SCRATCH = (
    0, -1, -2, -3, -4, -5, -6)
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_LAYER_ATTN, SPEC_LAYER_GDN = 0, 1
SPEC_GREEDY, SPEC_SAMPLED = 0, 1
(SPEC_K_NONE, SPEC_K_PROJ_IN, SPEC_K_ATTN, SPEC_K_PROJ_O, SPEC_K_GATE_UP, SPEC_K_DOWN, SPEC_K_LM_HEAD,
 SPEC_K_GDN) = (-1, 0, 1, 2, 3, 4, 5, 6)

HEADER_SYMBOLS = (
    "spec_status_string", "spec_plan_drafts", "spec_model_create", "spec_model_destroy",
    "spec_workspace_bytes", "spec_verify_round", "spec_verify_head", "spec_accept", "spec_commit",
    "spec_debug_logits", "spec_debug_gemm", "spec_packed_weight_bytes", "spec_pack_weight",
    "spec_profile_enable", "spec_profile_collect", "spec_debug_barrier_spin", "spec_ngram_draft",
    "spec_history_append",
    "spec_backoff_init", "spec_backoff_call", "spec_backoff_pass", "spec_counts_add",
    "spec_window_live_block", "spec_verify_head_noalloc",
)
SPEC_MAX_NGRAM = 8


class SpecBackoff(C.Structure):
    """Mirror of spec_backoff (one request's miss back-off state)."""
    _fields_ = [("miss_run", C.c_int32), ("wait_len", C.c_int32), ("wait_left", C.c_int32), ("may_guess", C.c_int32)]


class SpecError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {spec_status_string(status)} ({status})")
        self.status = status


class SpecLayerWeights(C.Structure):
    _fields_ = [("norm1", C.c_void_p), ("w_in", C.c_void_p), ("w_o", C.c_void_p), ("norm2", C.c_void_p),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p)]


class SpecModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("hidden", C.c_int), ("n_q_heads", C.c_int), ("n_kv_heads", C.c_int),
                ("head_dim", C.c_int), ("ffn", C.c_int), ("vocab", C.c_int), ("dtype", C.c_int),
                ("layer_kind", C.POINTER(C.c_int32)), ("gdn_heads", C.c_int), ("gdn_dim", C.c_int),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("kv_block", C.c_int),
                ("attn_chunk", C.c_int), ("embed", C.c_void_p), ("lm_head", C.c_void_p),
                ("final_norm", C.c_void_p), ("layers", C.POINTER(SpecLayerWeights)),
                ("sliding_window", C.c_int), ("window_global_every", C.c_int)]


class SpecRound(C.Structure):
    _fields_ = [("lanes", C.c_int), ("cols_host", C.POINTER(C.c_int32)), ("tokens", C.c_void_p),
                ("kv_len", C.c_void_p), ("kv_len_host", C.POINTER(C.c_int32)), ("block_table", C.c_void_p),
                ("max_blocks", C.c_int), ("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("n_blocks", C.c_int),
                ("gdn_state", C.c_void_p), ("mode", C.c_int), ("temperature", C.c_float),
                ("q_probs", C.c_void_p), ("seed", C.c_uint64), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("counts", C.c_void_p), ("presence_penalty", C.c_float),
                ("frequency_penalty", C.c_float)]


class SpecRowStat(C.Structure):
    _fields_ = [("max_logit", C.c_float), ("lse", C.c_float), ("argmax", C.c_int32), ("z_next", C.c_float)]


_lib = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load the built library; raises if it is missing (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m speculative_decoding_verify_round_amd.build`")
        lib = C.CDLL(path)
        lib.spec_status_string.restype = C.c_char_p
        lib.spec_status_string.argtypes = [C.c_int]
        lib.spec_plan_drafts.restype = C.c_int
        lib.spec_plan_drafts.argtypes = [C.c_int, C.c_int, C.c_int]
        lib.spec_model_create.restype = C.c_int
        lib.spec_model_create.argtypes = [C.POINTER(SpecModelDesc), C.POINTER(C.c_void_p)]
        lib.spec_model_destroy.restype = None
        lib.spec_model_destroy.argtypes = [C.c_void_p]
        lib.spec_workspace_bytes.restype = C.c_int64
        lib.spec_workspace_bytes.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int]
        for name in ("spec_verify_round",):
            getattr(lib, name).restype = C.c_int
            getattr(lib, name).argtypes = [C.c_void_p, C.POINTER(SpecRound), C.c_void_p]
        lib.spec_verify_head.restype = C.c_int
        lib.spec_verify_head.argtypes = [C.c_void_p, C.POINTER(SpecRound), C.c_void_p, C.c_void_p]
        lib.spec_verify_head_noalloc.restype = C.c_int
        lib.spec_verify_head_noalloc.argtypes = [C.c_void_p, C.POINTER(SpecRound), C.c_void_p, C.c_void_p, C.c_void_p,
                                                 C.c_void_p, C.c_void_p]
        lib.spec_accept.restype = C.c_int
        lib.spec_accept.argtypes = [C.c_void_p, C.POINTER(SpecRound), C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p]
        lib.spec_commit.restype = C.c_int
        lib.spec_commit.argtypes = [C.c_void_p, C.POINTER(SpecRound), C.c_void_p, C.c_void_p]
        lib.spec_debug_logits.restype = C.c_int
        lib.spec_debug_logits.argtypes = [C.c_void_p, C.POINTER(SpecRound), C.c_void_p, C.c_void_p]
        lib.spec_debug_gemm.restype = C.c_int
        lib.spec_debug_gemm.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                        C.c_void_p, C.c_size_t, C.c_void_p]
        lib.spec_packed_weight_bytes.restype = C.c_int64
        lib.spec_packed_weight_bytes.argtypes = [C.c_int, C.c_int]
        lib.spec_pack_weight.restype = C.c_int
        lib.spec_pack_weight.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        lib.spec_profile_enable.restype = C.c_int
        lib.spec_profile_enable.argtypes = [C.c_void_p, C.c_int, C.c_int]
        lib.spec_debug_barrier_spin.restype = C.c_int
        lib.spec_debug_barrier_spin.argtypes = [C.c_void_p, C.c_int]
        lib.spec_profile_collect.restype = C.c_int
        lib.spec_profile_collect.argtypes = [C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_int)]
        lib.spec_ngram_draft.restype = C.c_int
        lib.spec_ngram_draft.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                         C.c_void_p, C.c_void_p, C.c_void_p]
        lib.spec_backoff_init.restype = C.c_int
        lib.spec_backoff_init.argtypes = [C.c_void_p, C.c_int]
        lib.spec_backoff_call.restype = C.c_int
        lib.spec_backoff_call.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p]
        lib.spec_backoff_pass.restype = C.c_int
        lib.spec_backoff_pass.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_int]
        lib.spec_window_live_block.restype = C.c_int
        lib.spec_window_live_block.argtypes = [C.c_int, C.c_int]
        lib.spec_counts_add.restype = C.c_int
        lib.spec_counts_add.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p]
        lib.spec_history_append.restype = C.c_int
        lib.spec_history_append.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_int,
                                            C.c_void_p]
        _lib = lib
    return _lib


def _check(status: int, where: str) -> int:
    if status < 0:
        raise SpecError(status, where)
    return status


# ---------------------------------------------------------------------- the C calls
def spec_status_string(status: int) -> str:
    return load_library().spec_status_string(int(status)).decode()


def spec_plan_drafts(k: int, row_budget: int, lanes: int) -> int:
    """Returns the draft count, or a negative status (no exception) as the C call does."""
    return load_library().spec_plan_drafts(int(k), int(row_budget), int(lanes))


def spec_model_create(desc: SpecModelDesc) -> C.c_void_p:
    h = C.c_void_p()
    _check(load_library().spec_model_create(C.byref(desc), C.byref(h)), "spec_model_create")
    return h


def spec_model_destroy(model) -> None:
    load_library().spec_model_destroy(model)


def spec_workspace_bytes(model, max_lanes: int, max_cols: int, max_blocks: int) -> int:
    return _check(load_library().spec_workspace_bytes(model, max_lanes, max_cols, max_blocks),
                  "spec_workspace_bytes")


def spec_verify_round(model, rnd: SpecRound, stream: int) -> None:
    _check(load_library().spec_verify_round(model, C.byref(rnd), C.c_void_p(stream)), "spec_verify_round")


def spec_verify_head(model, rnd: SpecRound, hidden_ptr: int, stream: int) -> None:
    _check(load_library().spec_verify_head(model, C.byref(rnd), C.c_void_p(hidden_ptr), C.c_void_p(stream)),
           "spec_verify_head")


def spec_verify_head_noalloc(model, rnd: SpecRound, hidden_ptr: int, committed_ptr: int, out_tokens_ptr: int,
                             row_stats_ptr, stream: int) -> None:
    _check(load_library().spec_verify_head_noalloc(model, C.byref(rnd), C.c_void_p(hidden_ptr),
                                                   C.c_void_p(committed_ptr), C.c_void_p(out_tokens_ptr),
                                                   C.c_void_p(row_stats_ptr or 0), C.c_void_p(stream)),
           "spec_verify_head_noalloc")


def spec_accept(model, rnd: SpecRound, committed_ptr: int, out_tokens_ptr: int, row_stats_ptr, stream: int) -> None:
    _check(load_library().spec_accept(model, C.byref(rnd), C.c_void_p(committed_ptr), C.c_void_p(out_tokens_ptr),
                                      C.c_void_p(row_stats_ptr or 0), C.c_void_p(stream)), "spec_accept")


def spec_commit(model, rnd: SpecRound, committed_ptr: int, stream: int) -> None:
    _check(load_library().spec_commit(model, C.byref(rnd), C.c_void_p(committed_ptr), C.c_void_p(stream)),
           "spec_commit")


def spec_debug_logits(model, rnd: SpecRound, logits_ptr: int, stream: int) -> None:
    _check(load_library().spec_debug_logits(model, C.byref(rnd), C.c_void_p(logits_ptr), C.c_void_p(stream)),
           "spec_debug_logits")


def spec_debug_gemm(model, x_ptr: int, w_ptr: int, y_ptr: int, R: int, N: int, K: int, ws_ptr: int,
                    ws_bytes: int, stream: int) -> None:
    _check(load_library().spec_debug_gemm(model, C.c_void_p(x_ptr), C.c_void_p(w_ptr), C.c_void_p(y_ptr), R, N, K,
                                          C.c_void_p(ws_ptr), ws_bytes, C.c_void_p(stream)), "spec_debug_gemm")


def spec_packed_weight_bytes(N: int, K: int) -> int:
    return _check(load_library().spec_packed_weight_bytes(int(N), int(K)), "spec_packed_weight_bytes")


def spec_pack_weight(src_ptr: int, dst_ptr: int, N: int, K: int, stream: int) -> None:
    _check(load_library().spec_pack_weight(C.c_void_p(src_ptr), C.c_void_p(dst_ptr), int(N), int(K),
                                           C.c_void_p(stream)), "spec_pack_weight")


def spec_debug_barrier_spin(model, polls: int) -> None:
    _check(load_library().spec_debug_barrier_spin(model, int(polls)), "spec_debug_barrier_spin")


def spec_profile_enable(model, kernel_class: int, every: int = 1) -> None:
    _check(load_library().spec_profile_enable(model, kernel_class, every), "spec_profile_enable")


def spec_profile_collect(model):
    t = C.c_double()
    n = C.c_int()
    _check(load_library().spec_profile_collect(model, C.byref(t), C.byref(n)), "spec_profile_collect")
    return t.value, n.value


def spec_ngram_draft(history_ptr: int, hist_len_ptr: int, lanes: int, max_len: int, k: int, n_max: int, n_min: int,
                     tokens_ptr: int, n_match_ptr: int, stream: int) -> None:
    _check(load_library().spec_ngram_draft(C.c_void_p(history_ptr), C.c_void_p(hist_len_ptr), lanes, max_len, k,
                                           n_max, n_min, C.c_void_p(tokens_ptr), C.c_void_p(n_match_ptr),
                                           C.c_void_p(stream)), "spec_ngram_draft")


def spec_history_append(history_ptr: int, hist_len_ptr: int, lanes: int, max_len: int, committed_ptr: int,
                        out_tokens_ptr: int, out_stride: int, stream: int) -> None:
    _check(load_library().spec_history_append(C.c_void_p(history_ptr), C.c_void_p(hist_len_ptr), lanes, max_len,
                                              C.c_void_p(committed_ptr), C.c_void_p(out_tokens_ptr), out_stride,
                                              C.c_void_p(stream)), "spec_history_append")


def spec_backoff_init(states, n: int) -> None:
    _check(load_library().spec_backoff_init(states, n), "spec_backoff_init")


def spec_backoff_call(states, n: int, k: int, row_budget: int, drafts) -> bool:
    return bool(_check(load_library().spec_backoff_call(states, n, k, row_budget, drafts), "spec_backoff_call"))


def spec_backoff_pass(states, n: int, kept, speculates: bool) -> None:
    _check(load_library().spec_backoff_pass(states, n, kept, int(speculates)), "spec_backoff_pass")


def spec_window_live_block(kv_len: int, window: int) -> int:
    r = load_library().spec_window_live_block(kv_len, window)
    if r < 0:
        _check(r, "spec_window_live_block")
    return r


def spec_counts_add(counts_ptr: int, vocab: int, lanes: int, committed_ptr: int, out_tokens_ptr: int,
                    out_stride: int, stream: int) -> None:
    _check(load_library().spec_counts_add(C.c_void_p(counts_ptr), vocab, lanes, C.c_void_p(committed_ptr),
                                          C.c_void_p(out_tokens_ptr), out_stride, C.c_void_p(stream)),
           "spec_counts_add")
