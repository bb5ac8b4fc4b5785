"""Shared setup of GPU parity tests: the same synth inputs feed the oracle and the HIP path.

Nothing here computes any step of the verify round: the oracle side calls
oracle/, the device side calls the C ABI through the binding.
"""
import os
import sys
import time

import numpy as np
import torch

import synth
from oracle import OracleModel, KVCache
from oracle.accept import argmax_lowest
from speculative_decoding_verify_round_amd.runtime import DeviceCache, DeviceModel

GAP_EXCUSE = 5e-2          # oracle top-2 logit gap under which a token mismatch is excused


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


class Pair:
    """Oracle model + cache and device model + cache built from the same seeded inputs."""

    def __init__(self, cfg, lanes, context, max_blocks, weights=None, attn_chunk=0):
        self.cfg = cfg
        self.lanes = lanes
        w = weights if weights is not None else synth.model_weights(cfg)
        self.weights = w
        self.om = OracleModel(cfg, w)
        bt, n_blocks = synth.block_table(cfg, lanes, max_blocks)
        self.bt, self.n_blocks = bt, n_blocks
        self.oc = KVCache(kv_len=np.full(lanes, context, np.int64), block_table=bt.astype(np.int64),
                          block=cfg.kv_block)
        self.dm = DeviceModel(cfg, w, attn_chunk=attn_chunk)
        self.dc = DeviceCache(self.dm, lanes, max_blocks, n_blocks, block_table=bt, kv_len=[context] * lanes)
        for li in range(cfg.n_attn):
            self.oc.pool_k.append(np.zeros((n_blocks, cfg.kv_block, cfg.n_kv_heads, cfg.head_dim), np.float32))
            self.oc.pool_v.append(np.zeros_like(self.oc.pool_k[-1]))
            for l in range(lanes):
                if context:
                    k, v = synth.kv_context(cfg, li, l, context)
                    self.oc.scatter(li, l, 0, k, v)
                    self.dc.set_kv(li, l, 0, k, v)
        for gi in range(cfg.n_gdn):
            S = np.stack([synth.gdn_state(cfg, gi, l) for l in range(lanes)])
            self.oc.gdn.append(S)
            for l in range(lanes):
                self.dc.set_gdn(gi, l, S[l])
        torch.cuda.synchronize()

    def close(self):
        self.dm.close()


def top2_gap(z):
    z = np.sort(np.asarray(z, np.float64))
    return z[-1] - z[-2]


def compare_rows(oracle_logits, gpu_stats, tol):
    """Per-row checks of the LM-head statistics; returns (mismatch_rows, max_err_max)."""
    R = oracle_logits.shape[0]
    mism = []
    for r in range(R):
        z = oracle_logits[r]
        if argmax_lowest(z) != gpu_stats["argmax"][r]:
            mism.append((r, top2_gap(z)))
    err_max = float(np.max(np.abs(oracle_logits.max(axis=1) - gpu_stats["max"])))
    assert err_max <= tol, err_max
    return mism, err_max
