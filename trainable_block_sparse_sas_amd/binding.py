"""ctypes binding of libsas (C ABI in include/sas.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, reads their shapes, passes raw device pointers and the current
HIP stream to the library call of the same name, and raises SasError on a
non-zero status.  No computation happens here and there is no fallback: if
libsas.so is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SAS_LIB", os.path.join(_HERE, "libsas.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libsas.so not found at {LIB_PATH}; build it with "
                      f"`python -m trainable_block_sparse_sas_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

SAS_OK, SAS_EINVAL, SAS_EUNSUPPORTED, SAS_EHIP, SAS_EWORKSPACE = 0, -1, -2, -3, -4
SAS_F32, SAS_BF16 = 0, 1
SAS_OP_SCORE, SAS_OP_TOPK, SAS_OP_FWD, SAS_OP_BWD, SAS_OP_DECODE, SAS_OP_SELECTOR_BWD = 1, 2, 3, 4, 5, 6
SAS_OP_PAGED_DECODE = 7
SAS_OP_FWD_GATE, SAS_OP_BWD_GATE = 8, 9
SAS_OP_DECODE_STEP = 10
SAS_OP_PREFILL = 11
SAS_OP_CTX = 12
SAS_GATE_SOFTMAX, SAS_GATE_SIGMOID, SAS_GATE_RAW, SAS_GATE_OUTER, SAS_GATE_STE = 0, 1, 2, 3, 4

EXPORTED = ("sas_score_blocks", "sas_score_blocks_lse", "sas_topk_select", "sas_topk_select_gated", "sas_gated_attn_fwd",
            "sas_gated_attn_fwd_lse", "sas_gated_attn_fwd_ctx", "sas_gated_attn_bwd", "sas_gated_attn_bwd_ctx",
            "sas_gated_attn_fwd_gate", "sas_gated_attn_bwd_gate", "sas_sparse_decode", "sas_selector_bwd", "sas_pool_pages", "sas_paged_decode",
            "sas_sparse_decode_noalloc", "sas_decode_step", "sas_prefill_paged", "sas_workspace_bytes", "sas_last_error", "sas_abi_version",
            "sas_profile_enable", "sas_profile_read")

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib.sas_score_blocks.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
_lib.sas_score_blocks_lse.argtypes = [_vp] * 5 + [_i] * 6 + [_f, _i, _vp]
_lib.sas_topk_select.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
_lib.sas_topk_select_gated.argtypes = [_vp] * 4 + [_i] * 7 + [_vp]
_lib.sas_gated_attn_fwd.argtypes = [_vp] * 8 + [_i] * 7 + [_f, _i, _vp, _sz, _vp]
_lib.sas_gated_attn_fwd_lse.argtypes = [_vp] * 8 + [_i] * 7 + [_f, _i, _vp, _sz, _vp]
_lib.sas_gated_attn_bwd.argtypes = [_vp] * 13 + [_i] * 7 + [_f, _i, _vp, _sz, _vp]
_lib.sas_gated_attn_fwd_ctx.argtypes = [_vp] * 9 + [_i] * 7 + [_f, _i, _vp, _sz, _vp, _sz, _vp]
_lib.sas_gated_attn_bwd_ctx.argtypes = [_vp] * 10 + [_sz] + [_vp] * 4 + [_i] * 7 + [_f, _i, _vp, _sz, _vp]
_lib.sas_gated_attn_fwd_gate.argtypes = [_vp] * 8 + [_i] * 7 + [_f, _i, _i, _vp, _sz, _vp]
_lib.sas_gated_attn_bwd_gate.argtypes = [_vp] * 13 + [_i] * 7 + [_f, _i, _i, _vp, _sz, _vp]
_lib.sas_sparse_decode.argtypes = [_vp] * 7 + [_i] * 7 + [_f, _i, _vp, _sz, _vp]
_lib.sas_sparse_decode_noalloc.argtypes = [_vp] * 7 + [_i] * 7 + [_f, _i, _vp]
_lib.sas_decode_step.argtypes = [_vp] * 5 + [_i, _vp, _vp, _vp] + [_i] * 6 + [_f, _i, _vp, _sz, _vp]
_lib.sas_prefill_paged.argtypes = [_vp] * 10 + [_i] * 7 + [_f, _i, _vp, _sz, _vp]
_lib.sas_selector_bwd.argtypes = [_vp] * 6 + [_i] * 6 + [_f, _i, _i, _vp, _sz, _vp]
_lib.sas_pool_pages.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
_lib.sas_paged_decode.argtypes = [_vp] * 5 + [_i, _vp, _i, _vp, _vp, _vp] + [_i] * 5 + [_f, _i, _vp, _sz, _vp]
_lib.sas_workspace_bytes.argtypes = [_i] * 9
_lib.sas_workspace_bytes.restype = _sz
_lib.sas_last_error.restype = ctypes.c_char_p
_lib.sas_abi_version.restype = _i
_lib.sas_profile_enable.argtypes = [_i]
_lib.sas_profile_enable.restype = _i
_lib.sas_profile_read.argtypes = [_i, ctypes.c_char_p, _i, ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(_i)]
_lib.sas_profile_read.restype = _i
for _name in ("sas_score_blocks", "sas_score_blocks_lse", "sas_topk_select", "sas_topk_select_gated", "sas_gated_attn_fwd",
              "sas_gated_attn_fwd_lse", "sas_gated_attn_fwd_ctx", "sas_gated_attn_bwd", "sas_gated_attn_bwd_ctx",
              "sas_gated_attn_fwd_gate", "sas_gated_attn_bwd_gate", "sas_sparse_decode", "sas_selector_bwd", "sas_pool_pages", "sas_paged_decode",
              "sas_sparse_decode_noalloc", "sas_decode_step", "sas_prefill_paged"):
    getattr(_lib, _name).restype = _i


class SasError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"[{code}] {message}")
        self.code = code


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libsas tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_EMPTY_IDX = {}


def _idx_ptr(idx: Optional[torch.Tensor]):
    """idx pointer: NULL only for full scope.  A zero-width index tensor (topk 0)
    has no storage, so a one-element placeholder on its device stands in."""
    if idx is None:
        return None
    if idx.numel() == 0:
        dev = idx.device
        if dev not in _EMPTY_IDX:
            _EMPTY_IDX[dev] = torch.full((1,), -1, dtype=torch.int32, device=dev)
        return ctypes.c_void_p(_EMPTY_IDX[dev].data_ptr())
    return _p(idx)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SAS_F32
    if t.dtype == torch.bfloat16:
        return SAS_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(code: int):
    if code != SAS_OK:
        raise SasError(code, _lib.sas_last_error().decode())


def sas_abi_version() -> int:
    return _lib.sas_abi_version()


def sas_profile_enable(on: bool = True) -> None:
    _check(_lib.sas_profile_enable(int(bool(on))))


def sas_profile_read(max_entries: int = 64) -> dict:
    """{kernel name: (total ms, launches)} since the last read (waits for them)."""
    nb = 48
    names = ctypes.create_string_buffer(max_entries * nb)
    ms = (ctypes.c_double * max_entries)()
    counts = (_i * max_entries)()
    n = _lib.sas_profile_read(max_entries, names, nb, ms, counts)
    if n < 0:
        raise SasError(n, "sas_profile_read failed")
    out = {}
    for i in range(min(n, max_entries)):
        out[names.raw[i * nb:(i + 1) * nb].split(b"\0", 1)[0].decode()] = (ms[i], counts[i])
    return out


def sas_last_error() -> str:
    return _lib.sas_last_error().decode()


def sas_workspace_bytes(op: int, B: int, Hq: int, Hkv: int, n_or_lmax: int, D: int, block: int,
                        topk: int, dtype: int) -> int:
    return int(_lib.sas_workspace_bytes(op, B, Hq, Hkv, n_or_lmax, D, block, topk, dtype))


def workspace(op, B, Hq, Hkv, n_or_lmax, D, block, topk, dtype, device="cuda"):
    """A byte tensor of the size sas_workspace_bytes asks for (None if 0)."""
    n = sas_workspace_bytes(op, B, Hq, Hkv, n_or_lmax, D, block, topk, dtype)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def sas_score_blocks(q, k, kbar, scores, cache_len, block, scale, group_sum=False, L=None,
                     stream=None):
    """Training: q [B,Hq,N,D], k [B,Hkv,N,D] or None, kbar [B,Hkv,C,D], scores fp32.
    Decode (cache_len given): q [B,Hq,D], k the cache or None, L = cache capacity
    (taken from k when given; required otherwise, since the pooled keys alone
    do not fix a capacity that is not a multiple of the block)."""
    B, Hq, D = q.shape[0], q.shape[1], q.shape[-1]
    Hkv = kbar.shape[1]
    if cache_len is None:
        Nq = q.shape[2]
        L = Nq
    else:
        Nq = 1
        if L is None:
            if k is None:
                raise ValueError("sas_score_blocks: decode mode without k needs the cache capacity L")
            L = k.shape[2]
    _check(_lib.sas_score_blocks(_p(q), _p(k), _p(kbar), _p(scores), _p(cache_len), B, Hq, Hkv,
                                 Nq, L, D, block, scale, int(bool(group_sum)), _dt(q),
                                 _stream(stream)))


def sas_score_blocks_lse(q, k, kbar, scores, lse_s, block, scale, stream=None):
    """Training scores (q [B,Hq,N,D], k [B,Hkv,N,D] or None, kbar [B,Hkv,C,D],
    scores fp32 [B,Hq,N,C]) and the gate normaliser lse_s fp32 [B,Hq,N]."""
    B, Hq, N, D = q.shape
    Hkv = kbar.shape[1]
    _check(_lib.sas_score_blocks_lse(_p(q), _p(k), _p(kbar), _p(scores), _p(lse_s), B, Hq, Hkv, N, D,
                                     block, scale, _dt(q), _stream(stream)))


def sas_topk_select(scores, idx, cache_len, heads_per_row, block, workspace=None, stream=None):
    """scores fp32 [B, Hkv*hpr, Nq, C] (decode: [B, Hkv*hpr, C]); idx int32 [B,Hkv,Nq,K] / [B,Hkv,K]."""
    if cache_len is None:
        B, H, Nq, C = scores.shape
    else:
        B, H, C = scores.shape
        Nq = 1
    Hkv = H // heads_per_row
    topk = idx.shape[-1]
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_topk_select(_p(scores), _p(idx), _p(cache_len), B, Hkv, heads_per_row, Nq, C,
                                block, topk, _p(workspace), wsb, _stream(stream)))


def sas_topk_select_gated(scores, lse_s, idx, gates, block, stream=None):
    """Training Top-K (scores fp32 [B, Hkv*hpr, N, C], idx int32 [B, Hkv, N, K]) that also writes
    gates fp32 [B, Hkv, N, K, hpr]: the selection's base-2 log gates by slot (ascending block)."""
    B, H, Nq, C = scores.shape
    Hkv, topk, hpr = idx.shape[1], idx.shape[-1], gates.shape[-1]
    _check(_lib.sas_topk_select_gated(_p(scores), _p(lse_s), _p(idx), _p(gates), B, Hkv, hpr, Nq, C, block,
                                      topk, _stream(stream)))


def sas_gated_attn_fwd(q, k, v, scores, idx, o, lse, lse_s, block, scale, workspace=None,
                       stream=None):
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_gated_attn_fwd(_p(q), _p(k), _p(v), _p(scores), _idx_ptr(idx), _p(o), _p(lse),
                                   _p(lse_s), B, Hq, Hkv, N, D, block, topk, scale, _dt(q),
                                   _p(workspace), wsb, _stream(stream)))


def sas_gated_attn_fwd_lse(q, k, v, scores, idx, lse_s, o, lse, block, scale, workspace=None,
                           stream=None):
    """The forward with LSE_s given (lse_s is an input, e.g. from sas_score_blocks_lse)."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_gated_attn_fwd_lse(_p(q), _p(k), _p(v), _p(scores), _idx_ptr(idx), _p(lse_s), _p(o),
                                       _p(lse), B, Hq, Hkv, N, D, block, topk, scale, _dt(q),
                                       _p(workspace), wsb, _stream(stream)))


def sas_gated_attn_fwd_ctx(q, k, v, scores, idx, lse_s, o, lse, block, scale, ctx, workspace=None,
                           stream=None, gates=None):
    """The training forward with LSE_s given that also fills the saved context `ctx`
    (a byte tensor of sas_workspace_bytes(SAS_OP_CTX, ...) bytes, or None if that is 0);
    gates: None, or sas_topk_select_gated's log gates for these scores, LSE_s and idx."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    cb = 0 if ctx is None else ctx.numel()
    _check(_lib.sas_gated_attn_fwd_ctx(_p(q), _p(k), _p(v), _p(scores), _idx_ptr(idx), _p(lse_s), _p(gates),
                                       _p(o), _p(lse), B, Hq, Hkv, N, D, block, topk, scale, _dt(q), _p(ctx), cb,
                                       _p(workspace), wsb, _stream(stream)))


def sas_gated_attn_bwd_ctx(q, k, v, o, dout, scores, idx, lse, lse_s, ctx, dq, dk, dv, ds, block, scale,
                           workspace=None, stream=None):
    """The backward reading the saved context the forward filled."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    cb = 0 if ctx is None else ctx.numel()
    _check(_lib.sas_gated_attn_bwd_ctx(_p(q), _p(k), _p(v), _p(o), _p(dout), _p(scores), _idx_ptr(idx),
                                       _p(lse), _p(lse_s), _p(ctx), cb, _p(dq), _p(dk), _p(dv), _p(ds), B, Hq,
                                       Hkv, N, D, block, topk, scale, _dt(q), _p(workspace), wsb,
                                       _stream(stream)))


def sas_gated_attn_bwd(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, block, scale,
                       workspace=None, stream=None):
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_gated_attn_bwd(_p(q), _p(k), _p(v), _p(o), _p(dout), _p(scores), _idx_ptr(idx),
                                   _p(lse), _p(lse_s), _p(dq), _p(dk), _p(dv), _p(ds), B, Hq, Hkv,
                                   N, D, block, topk, scale, _dt(q), _p(workspace), wsb,
                                   _stream(stream)))


def sas_gated_attn_fwd_gate(q, k, v, scores, idx, o, lse, lse_s, block, scale, gate, workspace=None,
                            stream=None):
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_gated_attn_fwd_gate(_p(q), _p(k), _p(v), _p(scores), _idx_ptr(idx), _p(o), _p(lse),
                                        _p(lse_s), B, Hq, Hkv, N, D, block, topk, scale, _dt(q), gate,
                                        _p(workspace), wsb, _stream(stream)))


def sas_gated_attn_bwd_gate(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, block, scale,
                            gate, workspace=None, stream=None):
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_gated_attn_bwd_gate(_p(q), _p(k), _p(v), _p(o), _p(dout), _p(scores), _idx_ptr(idx),
                                        _p(lse), _p(lse_s), _p(dq), _p(dk), _p(dv), _p(ds), B, Hq, Hkv,
                                        N, D, block, topk, scale, _dt(q), gate, _p(workspace), wsb,
                                        _stream(stream)))


def sas_sparse_decode(q, k_cache, v_cache, cache_len, idx, o, lse, block, scale, workspace=None,
                      stream=None):
    B, Hq, D = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    topk = idx.shape[-1] if idx is not None else 0
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_sparse_decode(_p(q), _p(k_cache), _p(v_cache), _p(cache_len), _idx_ptr(idx), _p(o),
                                  _p(lse), B, Hq, Hkv, L, D, block, topk, scale, _dt(q),
                                  _p(workspace), wsb, _stream(stream)))


def sas_sparse_decode_noalloc(q, k_cache, v_cache, cache_len, idx, o, lse, block, scale, stream=None):
    """sas_sparse_decode with the library's fixed per-GPU scratch instead of a workspace."""
    B, Hq, D = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    topk = idx.shape[-1] if idx is not None else 0
    _check(_lib.sas_sparse_decode_noalloc(_p(q), _p(k_cache), _p(v_cache), _p(cache_len), _idx_ptr(idx), _p(o),
                                          _p(lse), B, Hq, Hkv, L, D, block, topk, scale, _dt(q),
                                          _stream(stream)))


def sas_selector_bwd(q, kbar, ds, dq, dk, block, scale, dkbar=None, accumulate=False, workspace=None,
                     stream=None):
    """q [B,Hq,N,D], kbar [B,Hkv,C,D], ds fp32 [B,Hq,N,C] -> dq [B,Hq,N,D], dk [B,Hkv,N,D]
    (written, or added to with accumulate=True), optional dkbar fp32 [B,Hkv,C,D]."""
    B, Hq, N, D = q.shape
    Hkv = kbar.shape[1]
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_selector_bwd(_p(q), _p(kbar), _p(ds), _p(dq), _p(dk), _p(dkbar), B, Hq, Hkv, N, D,
                                 block, scale, 1 if accumulate else 0, _dt(q), _p(workspace), wsb,
                                 _stream(stream)))


def sas_pool_pages(k_pages, kbar_pages, pages, block, stream=None):
    """k_pages [P,Hkv,block,D] -> kbar_pages [P,Hkv,D] rows of the int32 page list `pages`."""
    Hkv, D = k_pages.shape[1], k_pages.shape[3]
    _check(_lib.sas_pool_pages(_p(k_pages), _p(kbar_pages), _p(pages), pages.numel(), Hkv, D, block, _dt(k_pages),
                               _stream(stream)))


def sas_paged_decode(q, k_pages, v_pages, kbar_pages, block_table, cache_len, topk, o, lse, block, scale,
                     idx_out=None, workspace=None, stream=None):
    """q [B,Hq,D]; pages [P,Hkv,block,D]; kbar_pages [P,Hkv,D]; block_table int32 [B,max_blocks]."""
    B, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_paged_decode(_p(q), _p(k_pages), _p(v_pages), _p(kbar_pages), _p(block_table),
                                 block_table.shape[1], _p(cache_len), topk, _p(o), _p(lse), _p(idx_out), B, Hq,
                                 Hkv, D, block, scale, _dt(q), _p(workspace), wsb, _stream(stream)))


def sas_decode_step(q, kbar, k_cache, v_cache, cache_len, topk, o, lse, block, scale, idx_out=None, workspace=None,
                    stream=None):
    """q [B,Hq,D]; kbar [B,Hkv,C,D]; caches [B,Hkv,L_max,D]; cache_len int32 [B]: scores, Top-K and sparse
    attention in one call."""
    B, Hq, D = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_decode_step(_p(q), _p(kbar), _p(k_cache), _p(v_cache), _p(cache_len), topk, _p(o), _p(lse),
                                _p(idx_out), B, Hq, Hkv, L, D, block, scale, _dt(q), _p(workspace), wsb,
                                _stream(stream)))


def sas_prefill_paged(q, k, v, seq_len, o, lse, k_pages, v_pages, kbar_pages, block_table, block, scale,
                      workspace=None, stream=None):
    """q [B,Hq,N,D]; k, v [B,Hkv,N,D]; seq_len int32 [B]; pages [P,Hkv,block,D]; kbar_pages [P,Hkv,D];
    block_table int32 [B,max_blocks]: dense causal attention of the prompts, and their pages filled."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    wsb = 0 if workspace is None else workspace.numel()
    _check(_lib.sas_prefill_paged(_p(q), _p(k), _p(v), _p(seq_len), _p(o), _p(lse), _p(k_pages), _p(v_pages),
                                  _p(kbar_pages), _p(block_table), block_table.shape[1], B, Hq, Hkv, N, D, block,
                                  scale, _dt(q), _p(workspace), wsb, _stream(stream)))
