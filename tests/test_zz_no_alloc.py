"""sas_sparse_decode_noalloc (the allocation-free decode call) against
sas_sparse_decode with a caller workspace: the same kernels run, so the two
must agree bit for bit.  Two calls in a row, the second on a smaller input,
so the second reuses the scratch the first left behind."""
import ctypes

import pytest
import torch

from trainable_block_sparse_sas_amd.inputs import Workload, decode_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from trainable_block_sparse_sas_amd import binding as sas

DEV = "cuda"


def _noalloc_c_abi(q, kc, vc, lens, idx, o, lse, block, scale):
    """The call through the C ABI itself (ctypes, raw device pointers)."""
    B, Hq, D = q.shape
    Hkv, L = kc.shape[1], kc.shape[2]
    topk = idx.shape[-1] if idx is not None else 0
    vp = ctypes.c_void_p
    st = sas._lib.sas_sparse_decode_noalloc(
        vp(q.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()), vp(lens.data_ptr()),
        None if idx is None else vp(idx.data_ptr()), vp(o.data_ptr()), vp(lse.data_ptr()),
        B, Hq, Hkv, L, D, block, topk, ctypes.c_float(scale),
        sas.SAS_BF16 if q.dtype == torch.bfloat16 else sas.SAS_F32,
        vp(torch.cuda.current_stream().cuda_stream))
    assert st == sas.SAS_OK, sas.sas_last_error()


def _reference(q, kc, vc, lens, idx, block, scale):
    B, Hq, D = q.shape
    Hkv, L = kc.shape[1], kc.shape[2]
    o = torch.empty((B, Hq, D), dtype=q.dtype, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    tk = -1 if idx is None else idx.shape[-1]
    ws = sas.workspace(sas.SAS_OP_DECODE, B, Hq, Hkv, L, D, block, tk,
                       sas.SAS_BF16 if q.dtype == torch.bfloat16 else sas.SAS_F32)
    sas.sas_sparse_decode(q, kc, vc, lens, idx, o, lse, block, scale, ws)
    return o, lse


def _case(dts, B, Hq, Hkv, D, L, block, topk, lens, seed):
    w = Workload("noalloc", "decode", dts, B, Hq, Hkv, D, L, block, topk, index=seed)
    q, kc, vc, _ = decode_inputs(w, device=DEV)
    lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = None
    if topk is not None:
        g = torch.Generator(device="cpu").manual_seed(seed)
        idx = torch.randint(-1, L // block, (B, Hkv, topk), generator=g, dtype=torch.int32).to(DEV)
    return q, kc, vc, lens, idx, w.scale


def _check(q, kc, vc, lens, idx, block, scale):
    o_ref, lse_ref = _reference(q, kc, vc, lens, idx, block, scale)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    _noalloc_c_abi(q, kc, vc, lens, idx, o, lse, block, scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                       o_ref.view(torch.int16) if o.dtype == torch.bfloat16 else o_ref.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))


@pytest.mark.parametrize("dts,topk", [("bf16", 6), ("bf16", None), ("f32", 3)], ids=["bf16-sparse", "bf16-dense",
                                                                                     "f32-sparse"])
def test_noalloc_decode_matches_workspace_call(dts, topk):
    # first call: 4 sequences (one idle, one over-long), 8192-token cache
    big = _case(dts, 4, 8, 2, 128, 8192, 64, topk, [8192, 5000, 0, 9000], 31)
    _check(*big[:5], 64, big[5])
    # second call, smaller: 2 sequences, 1000-token cache, block 32, the scratch
    # still holds the first call's partials
    small = _case(dts, 2, 10, 2, 64, 1000, 32, None if topk is None else 2, [1000, 77], 32)
    _check(*small[:5], 32, small[5])
