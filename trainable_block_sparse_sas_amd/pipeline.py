"""Buffers and call sequences of the two SAS hot paths on one GPU.

Training (full or sparse scope):  sas_score_blocks_lse (pool + score + the gate
  normaliser) -> sas_topk_select_gated (sparse scope only; also the selection's
  log gates; sas_topk_select where C > 1024 or K > 64) -> sas_gated_attn_fwd_ctx
  (LSE_s and the log gates given; saves the selection lists and log gates) ->
  sas_gated_attn_bwd_ctx.
Decode:  sas_score_blocks (group-summed scores from pooled keys kept beside the
  cache) -> sas_topk_select -> sas_sparse_decode.

Every buffer is allocated once, up front, with torch; `run` only enqueues the
library calls on the current stream.
"""
from __future__ import annotations

import torch

from . import binding as sas


class TrainStep:
    def __init__(self, B, Hq, Hkv, N, D, block, topk, dtype, device="cuda", scale=None):
        self.B, self.Hq, self.Hkv, self.N, self.D, self.block = B, Hq, Hkv, N, D, block
        self.topk = topk  # None: full scope
        self.scale = D ** -0.5 if scale is None else scale
        self.C = N // block
        C, dev = self.C, device
        self.dtype = dtype
        sdt = sas.SAS_BF16 if dtype == torch.bfloat16 else sas.SAS_F32
        self.kbar = torch.empty((B, Hkv, C, D), dtype=dtype, device=dev)
        # the calls write only each row's history columns: the others keep
        # these fills (-inf scores, zero ds), as in the dense form
        self.scores = torch.full((B, Hq, N, C), float("-inf"), dtype=torch.float32, device=dev)
        self.idx = None if topk is None else torch.empty((B, Hkv, N, topk), dtype=torch.int32, device=dev)
        self.o = torch.empty((B, Hq, N, D), dtype=dtype, device=dev)
        self.lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        self.lse_s = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        self.dq = torch.empty((B, Hq, N, D), dtype=dtype, device=dev)
        self.dk = torch.empty((B, Hkv, N, D), dtype=dtype, device=dev)
        self.dv = torch.empty((B, Hkv, N, D), dtype=dtype, device=dev)
        self.ds = torch.zeros((B, Hq, N, C), dtype=torch.float32, device=dev)
        tk = -1 if topk is None else topk
        # one scratch buffer for both calls: they run in stream order and a
        # workspace carries nothing from one call to the next
        n_ws = max(sas.sas_workspace_bytes(op, B, Hq, Hkv, N, D, block, tk, sdt)
                   for op in (sas.SAS_OP_FWD, sas.SAS_OP_BWD))
        self.ws = torch.empty(n_ws, dtype=torch.uint8, device=dev) if n_ws else None
        self.ws_fwd = self.ws_bwd = self.ws
        # the forward's saved context for the backward (selection lists and
        # log gates); valid after a forward on the step's own scores
        n_ctx = sas.sas_workspace_bytes(sas.SAS_OP_CTX, B, Hq, Hkv, N, D, block, tk, sdt)
        self.ctx = torch.empty(n_ctx, dtype=torch.uint8, device=dev) if n_ctx else None
        self._ctx_valid = False
        # the selection's log gates from the gated Top-K (its range only)
        G = Hq // Hkv
        gated = topk is not None and 0 < topk <= 64 and C <= 1024 and G in (1, 2, 4, 8)
        self.gates = torch.empty((B, Hkv, N, topk, G), dtype=torch.float32, device=dev) if gated else None

    def select(self, q, k):
        # scores and, in the same kernel, the gate normaliser LSE_s
        sas.sas_score_blocks_lse(q, k, self.kbar, self.scores, self.lse_s, self.block, self.scale)
        if self.gates is not None:
            sas.sas_topk_select_gated(self.scores, self.lse_s, self.idx, self.gates, self.block)
        elif self.idx is not None:
            sas.sas_topk_select(self.scores, self.idx, None, self.Hq // self.Hkv, self.block)

    def forward(self, q, k, v, scores=None, idx=None):
        own = scores is None and idx is None  # the step's own scores and selection
        idx = self.idx if idx is None else idx
        if own:  # LSE_s from select(); the saved context filled for the backward
            sas.sas_gated_attn_fwd_ctx(q, k, v, self.scores, idx, self.lse_s, self.o, self.lse, self.block,
                                       self.scale, self.ctx, self.ws_fwd, gates=self.gates)
        else:
            sas.sas_gated_attn_fwd(q, k, v, self.scores if scores is None else scores, idx, self.o, self.lse,
                                   self.lse_s, self.block, self.scale, self.ws_fwd)
        self._ctx_valid = own

    def backward(self, q, k, v, do, scores=None, idx=None):
        if scores is None and idx is None and self._ctx_valid:
            sas.sas_gated_attn_bwd_ctx(q, k, v, self.o, do, self.scores, self.idx, self.lse, self.lse_s,
                                       self.ctx, self.dq, self.dk, self.dv, self.ds, self.block, self.scale,
                                       self.ws_bwd)
            return
        scores = self.scores if scores is None else scores
        idx = self.idx if idx is None else idx
        sas.sas_gated_attn_bwd(q, k, v, self.o, do, scores, idx, self.lse, self.lse_s, self.dq,
                               self.dk, self.dv, self.ds, self.block, self.scale, self.ws_bwd)

    def run(self, q, k, v, do):
        self.select(q, k)
        self.forward(q, k, v)
        self.backward(q, k, v, do)


class DecodeStep:
    def __init__(self, B, Hq, Hkv, L, D, block, topk, dtype, device="cuda", scale=None):
        self.B, self.Hq, self.Hkv, self.L, self.D, self.block = B, Hq, Hkv, L, D, block
        self.topk = topk  # None: dense decode
        self.scale = D ** -0.5 if scale is None else scale
        self.C = L // block
        dev = device
        sdt = sas.SAS_BF16 if dtype == torch.bfloat16 else sas.SAS_F32
        self.kbar = torch.empty((B, Hkv, self.C, D), dtype=dtype, device=dev)
        self.u = torch.empty((B, Hkv, self.C), dtype=torch.float32, device=dev)
        self.idx = None if topk is None else torch.empty((B, Hkv, topk), dtype=torch.int32, device=dev)
        self.o = torch.empty((B, Hq, D), dtype=dtype, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        tk = -1 if topk is None else topk
        self.ws = sas.workspace(sas.SAS_OP_DECODE, B, Hq, Hkv, L, D, block, tk, sdt, dev)
        self.q_dummy = None

    def pool(self, k_cache):
        """Pooled keys of every complete cached block (kept beside the cache)."""
        q0 = torch.zeros((self.B, self.Hq, self.D), dtype=k_cache.dtype, device=k_cache.device)
        lens = torch.zeros((self.B,), dtype=torch.int32, device=k_cache.device)
        sas.sas_score_blocks(q0, k_cache, self.kbar, self.u.new_empty((self.B, self.Hq, self.C)),
                             lens, self.block, self.scale, L=self.L)

    def select(self, q, cache_len, kbar=None):
        kbar = self.kbar if kbar is None else kbar
        sas.sas_score_blocks(q, None, kbar, self.u, cache_len, self.block, self.scale,
                             group_sum=True, L=self.L)
        sas.sas_topk_select(self.u, self.idx, cache_len, 1, self.block)

    def attend(self, q, k_cache, v_cache, cache_len, idx=None):
        idx = self.idx if idx is None else idx
        sas.sas_sparse_decode(q, k_cache, v_cache, cache_len, idx, self.o, self.lse, self.block,
                              self.scale, self.ws)

    def run(self, q, k_cache, v_cache, cache_len):
        if self.topk is not None:
            self.select(q, cache_len)
        self.attend(q, k_cache, v_cache, cache_len)
