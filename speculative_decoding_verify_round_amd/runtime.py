"""Device buffers for the C ABI, held in torch tensors (plumbing only).

DeviceModel uploads weights and owns the spec_model handle; DeviceCache owns
the paged KV pools, the block table, kv_len, the recurrent state and the
workspace of a set of lanes; RoundCall packs one spec_round.  Every step of
the verify round itself runs in the HIP library.
"""
import ctypes as C
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import binding as B


def _dev(device):
    return torch.device(device)


def _upload(a, dtype, device):
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=dtype).contiguous()


def pack_weight(w: torch.Tensor, stream: Optional[int] = None) -> torch.Tensor:
    """A row-major bf16 device matrix [N][K] in the library's fragment layout (spec_pack_weight)."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.is_cuda
    w = w.contiguous()
    N, K = w.shape
    n = B.spec_packed_weight_bytes(N, K) // 2
    out = torch.empty(n, dtype=torch.bfloat16, device=w.device)
    st = torch.cuda.current_stream(w.device).cuda_stream if stream is None else stream
    B.spec_pack_weight(w.data_ptr(), out.data_ptr(), N, K, st)
    return out


def attn_chunk_for(n_kv_heads: int, lanes: int, context: int, window: int = 0) -> int:
    """Split-KV chunk (positions) for a model that serves `lanes` lanes at about `context`
    positions: 1024 when the (lane, kv head, chunk) triples at that size give at least half
    as many workgroups as the card has CUs (128), else 512; 512 with a sliding window (a
    window of W positions spans only about W / chunk + 1 chunks) or below 4096 positions.
    The chunk grid is fixed per model, and results depend on it only through the fixed
    order of the merge."""
    wide = lanes * n_kv_heads * ((context + 1023) // 1024) >= 128
    return 1024 if wide and not window and context >= 4096 else 512


class DeviceModel:
    """Weights on the device plus the library's model handle.

    cfg: a decoder config (shape attributes); weights: dict with "embed",
    "lm_head", "final_norm" and "layers" (list of dicts with norm1, w_in, w_o,
    norm2, w_gate, w_up, w_down), numpy or torch, matrices row-major [out][in].
    """

    def __init__(self, cfg, weights: Dict[str, object], device="cuda", attn_chunk: int = 0,
                 prepacked: bool = False):
        B.load_library()
        self.cfg = cfg
        self.device = _dev(device)
        self.tdtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.t: Dict[str, torch.Tensor] = {}
        up = lambda a: _upload(a, self.tdtype, self.device)
        f32 = lambda a: _upload(a, torch.float32, self.device)
        # bf16 matrices go to the device in the fragment layout the projections read
        # (prepacked: the caller already holds them packed, as flat bf16 device tensors)
        mat = (lambda a: pack_weight(up(a))) if cfg.dtype == "bf16" and not prepacked else up
        self.t["lm_head"] = mat(weights["lm_head"])
        if "embed" in weights:
            self.t["embed"] = up(weights["embed"])
        self.t["final_norm"] = f32(weights["final_norm"])
        self.layers: List[Dict[str, torch.Tensor]] = []
        lw_arr = (B.SpecLayerWeights * max(1, cfg.n_layers))()
        for i in range(cfg.n_layers):
            lw = weights["layers"][i]
            d = {"norm1": f32(lw["norm1"]), "norm2": f32(lw["norm2"])}
            for k in ("w_in", "w_o", "w_gate", "w_up", "w_down"):
                d[k] = mat(lw[k])
            self.layers.append(d)
            lw_arr[i] = B.SpecLayerWeights(d["norm1"].data_ptr(), d["w_in"].data_ptr(), d["w_o"].data_ptr(),
                                           d["norm2"].data_ptr(), d["w_gate"].data_ptr(), d["w_up"].data_ptr(),
                                           d["w_down"].data_ptr())
        self._lw = lw_arr
        kinds = [B.SPEC_LAYER_ATTN if k == "attn" else B.SPEC_LAYER_GDN for k in cfg.layer_kinds]
        self._kinds = (C.c_int32 * max(1, len(kinds)))(*kinds)
        desc = B.SpecModelDesc()
        desc.n_layers = cfg.n_layers
        desc.hidden = cfg.hidden
        desc.n_q_heads, desc.n_kv_heads, desc.head_dim = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        desc.ffn, desc.vocab = cfg.ffn, cfg.vocab
        desc.dtype = B.SPEC_BF16 if cfg.dtype == "bf16" else B.SPEC_F32
        desc.layer_kind = C.cast(self._kinds, C.POINTER(C.c_int32))
        desc.gdn_heads, desc.gdn_dim = cfg.gdn_heads, cfg.gdn_dim
        desc.rms_eps, desc.rope_theta = cfg.rms_eps, cfg.rope_theta
        desc.kv_block = cfg.kv_block
        desc.attn_chunk = attn_chunk
        desc.sliding_window = cfg.sliding_window
        desc.window_global_every = cfg.window_global_every
        desc.embed = self.t["embed"].data_ptr() if "embed" in self.t else None
        desc.lm_head = self.t["lm_head"].data_ptr()
        desc.final_norm = self.t["final_norm"].data_ptr()
        desc.layers = C.cast(self._lw, C.POINTER(B.SpecLayerWeights))
        self.desc = desc
        self.handle = B.spec_model_create(desc)

    def close(self):
        if self.handle:
            B.spec_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class RoundCall:
    """One spec_round plus the host arrays and device tensors it points at."""

    def __init__(self, cache: "DeviceCache", lane_tokens: Sequence[Sequence[int]], mode: str = "greedy",
                 temperature: float = 1.0, q_probs: Optional[torch.Tensor] = None, seed: int = 0,
                 kv_len_host: Optional[Sequence[int]] = None, tokens_dev: Optional[torch.Tensor] = None,
                 counts: Optional[torch.Tensor] = None, presence: float = 0.0, frequency: float = 0.0):
        self.cache = cache
        self.L = len(lane_tokens)
        self.cols = [len(t) for t in lane_tokens]
        self.R = sum(self.cols)
        self._cols = (C.c_int32 * self.L)(*self.cols)
        if tokens_dev is None:
            flat = np.concatenate([np.asarray(t, np.int32) for t in lane_tokens])
            tokens_dev = torch.from_numpy(flat).to(cache.device)
        self.tokens = tokens_dev
        self._kvh = None
        if kv_len_host is not None:
            self._kvh = (C.c_int32 * self.L)(*[int(v) for v in kv_len_host])
        self.q = q_probs
        r = B.SpecRound()
        r.lanes = self.L
        r.cols_host = C.cast(self._cols, C.POINTER(C.c_int32))
        r.tokens = self.tokens.data_ptr()
        r.kv_len = cache.kv_len.data_ptr()
        r.kv_len_host = C.cast(self._kvh, C.POINTER(C.c_int32)) if self._kvh is not None else None
        r.block_table = cache.block_table.data_ptr() if cache.block_table is not None else None
        r.max_blocks = cache.max_blocks
        r.k_pool = cache.k_pool.data_ptr() if cache.k_pool is not None else None
        r.v_pool = cache.v_pool.data_ptr() if cache.v_pool is not None else None
        r.n_blocks = cache.n_blocks
        r.gdn_state = cache.gdn.data_ptr() if cache.gdn is not None else None
        r.mode = B.SPEC_SAMPLED if mode == "sampled" else B.SPEC_GREEDY
        r.temperature = float(temperature)
        r.q_probs = q_probs.data_ptr() if q_probs is not None else None
        r.seed = int(seed)
        r.workspace = cache.workspace.data_ptr()
        r.workspace_bytes = cache.workspace.numel()
        self.counts = counts            # device int32 [lanes][vocab] or None: per-row penalties
        r.counts = counts.data_ptr() if counts is not None else None
        r.presence_penalty = float(presence)
        r.frequency_penalty = float(frequency)
        self.r = r


class DeviceCache:
    """Per-lane device state: paged KV pools, block table, kv_len, recurrent state, workspace."""

    def __init__(self, model: DeviceModel, lanes: int, max_blocks: int, n_blocks: int,
                 block_table: Optional[np.ndarray] = None, kv_len: Optional[Sequence[int]] = None,
                 max_cols: int = B.SPEC_MAX_COLS, pools: bool = True):
        cfg = model.cfg
        self.model = model
        self.device = model.device
        self.lanes, self.max_blocks, self.n_blocks = lanes, max_blocks, n_blocks
        dev = self.device
        self.kv_len = torch.tensor(list(kv_len) if kv_len is not None else [0] * lanes, dtype=torch.int32,
                                   device=dev)
        self.block_table = None
        self.k_pool = self.v_pool = None
        if cfg.n_attn:
            bt = block_table if block_table is not None else np.arange(lanes * max_blocks).reshape(lanes, max_blocks)
            self.block_table = torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to(dev)
        if cfg.n_attn and pools:
            shape_k = (cfg.n_attn, n_blocks, cfg.n_kv_heads, B.SPEC_KV_BLOCK, cfg.head_dim)
            shape_v = (cfg.n_attn, n_blocks, cfg.n_kv_heads, cfg.head_dim, B.SPEC_KV_BLOCK)
            self.k_pool = torch.zeros(shape_k, dtype=model.tdtype, device=dev)
            self.v_pool = torch.zeros(shape_v, dtype=model.tdtype, device=dev)
        self.gdn = None
        if cfg.n_gdn and pools:
            self.gdn = torch.zeros((lanes, cfg.n_gdn, cfg.gdn_heads, cfg.gdn_dim, cfg.gdn_dim), dtype=torch.float32,
                                   device=dev)
        nbytes = B.spec_workspace_bytes(model.handle, lanes, max_cols, max(1, max_blocks))
        self.workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device=dev)
        off = (-self.workspace.data_ptr()) % 256
        self.workspace = self.workspace[off:off + nbytes]
        self.committed = torch.zeros(lanes, dtype=torch.int32, device=dev)
        self.out_tokens = torch.zeros((lanes, B.SPEC_MAX_COLS), dtype=torch.int32, device=dev)
        self.row_stats = torch.zeros((B.SPEC_MAX_ROWS, 4), dtype=torch.float32, device=dev)

    # -------------------------------------------------------------- state loading / reading
    def _positions(self, lane: int, start: int, n: int):
        p = np.arange(start, start + n)
        bt = self.block_table[lane].cpu().numpy()
        return torch.from_numpy(bt[p // 16].astype(np.int64)), torch.from_numpy((p % 16).astype(np.int64))

    def set_kv(self, attn_layer: int, lane: int, start: int, K, V) -> None:
        """Write logical K, V rows [n, n_kv, d] of one lane at positions start .. start + n - 1."""
        K = _upload(K, self.model.tdtype, self.device)
        V = _upload(V, self.model.tdtype, self.device)
        blk, slot = self._positions(lane, start, K.shape[0])
        blk, slot = blk.to(self.device), slot.to(self.device)
        self.k_pool[attn_layer][blk, :, slot, :] = K
        self.v_pool[attn_layer][blk, :, :, slot] = V

    def get_kv(self, attn_layer: int, lane: int, start: int, n: int):
        blk, slot = self._positions(lane, start, n)
        blk, slot = blk.to(self.device), slot.to(self.device)
        K = self.k_pool[attn_layer][blk, :, slot, :]
        V = self.v_pool[attn_layer][blk, :, :, slot]
        return K.float().cpu().numpy(), V.float().cpu().numpy()

    def set_gdn(self, gdn_layer: int, lane: int, S) -> None:
        self.gdn[lane, gdn_layer] = _upload(S, torch.float32, self.device)

    def set_kv_len(self, values: Sequence[int]) -> None:
        self.kv_len.copy_(torch.tensor(list(values), dtype=torch.int32))

    # -------------------------------------------------------------- calls
    def round(self, lane_tokens, **kw) -> RoundCall:
        return RoundCall(self, lane_tokens, **kw)

    def verify(self, rc: RoundCall, stream: Optional[int] = None) -> None:
        B.spec_verify_round(self.model.handle, rc.r, _stream(stream))

    def verify_head(self, rc: RoundCall, hidden: torch.Tensor, stream: Optional[int] = None) -> None:
        B.spec_verify_head(self.model.handle, rc.r, hidden.data_ptr(), _stream(stream))

    def accept(self, rc: RoundCall, stats: bool = True, stream: Optional[int] = None) -> None:
        B.spec_accept(self.model.handle, rc.r, self.committed.data_ptr(), self.out_tokens.data_ptr(),
                      self.row_stats.data_ptr() if stats else 0, _stream(stream))

    def commit(self, rc: RoundCall, committed: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> None:
        c = self.committed if committed is None else committed
        B.spec_commit(self.model.handle, rc.r, c.data_ptr(), _stream(stream))

    def debug_logits(self, rc: RoundCall, stream: Optional[int] = None) -> torch.Tensor:
        out = torch.empty((rc.R, self.model.cfg.vocab), dtype=torch.float32, device=self.device)
        B.spec_debug_logits(self.model.handle, rc.r, out.data_ptr(), _stream(stream))
        return out

    def ngram_rounds(self, history: torch.Tensor, hist_len: torch.Tensor, rounds: int, k: int, n_max: int,
                     n_min: int = 1, stream: Optional[int] = None, counts: Optional[torch.Tensor] = None,
                     presence: float = 0.0, frequency: float = 0.0):
        """`rounds` greedy verify rounds on every lane, drafts from the lane's own history by the
        n-gram drafter, k + 1 columns per lane, each round's committed run appended to the
        history: device work only, no host round trip between rounds.  history: device int32
        [lanes][max_len] ending with each lane's anchor; hist_len: device int32 [lanes].
        With counts (device int32 [lanes][vocab], each lane's tokens up to its anchor) every
        round applies the per-row penalties and adds its committed runs to the counts.
        Returns the device tensors of the last round (tokens [lanes][k + 1], n_match [lanes])."""
        L, max_len = history.shape
        s = _stream(stream)
        tokens = torch.empty((L, k + 1), dtype=torch.int32, device=self.device)
        n_match = torch.empty(L, dtype=torch.int32, device=self.device)
        rc = self.round([[0] * (k + 1)] * L, tokens_dev=tokens.view(-1), counts=counts, presence=presence,
                        frequency=frequency)
        for _ in range(rounds):
            B.spec_ngram_draft(history.data_ptr(), hist_len.data_ptr(), L, max_len, k, n_max, n_min,
                               tokens.data_ptr(), n_match.data_ptr(), s)
            self.verify(rc, s)
            self.accept(rc, stats=False, stream=s)
            self.commit(rc, stream=s)
            if counts is not None:
                B.spec_counts_add(counts.data_ptr(), self.model.cfg.vocab, L, self.committed.data_ptr(),
                                  self.out_tokens.data_ptr(), self.out_tokens.shape[1], s)
            B.spec_history_append(history.data_ptr(), hist_len.data_ptr(), L, max_len, self.committed.data_ptr(),
                                  self.out_tokens.data_ptr(), self.out_tokens.shape[1], s)
        return tokens, n_match

    def results(self, rc: RoundCall):
        """Host copies of committed[L], the committed tokens per lane, and the row stats."""
        torch.cuda.synchronize(self.device)
        c = self.committed[: rc.L].cpu().numpy().astype(np.int64)
        toks = self.out_tokens[: rc.L].cpu().numpy()
        rs = self.row_stats[: rc.R].cpu()
        stats = {
            "max": rs[:, 0].numpy().copy(),
            "lse": rs[:, 1].numpy().copy(),
            "argmax": rs[:, 2].contiguous().view(torch.int32).numpy().astype(np.int64),
            "z_next": rs[:, 3].numpy().copy(),
        }
        return c, [list(map(int, toks[l, : c[l]])) for l in range(rc.L)], stats


def _stream(stream: Optional[int]) -> int:
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream
