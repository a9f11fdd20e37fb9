"""Run-to-run determinism of every bf16 entry point.

Each call runs twice on identical inputs, with every output overwritten by NaN
in between, and the two results must agree bit for bit.  The kernels use no
global-memory and no floating-point atomics; the only atomics are integer LDS
counters and bit sets (Top-K histograms, selection bitmasks, running maxima of
non-negative integers), whose results do not depend on the order in which the
lanes arrive, so every sum is formed in a fixed order.
Small shapes cover every entry point; the benchmark shapes cover the training
step and the decode step as bench.py times them.
"""
import numpy as np
import pytest
import torch

from trainable_block_sparse_sas_amd.inputs import WORKLOADS, Workload, decode_inputs, training_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from trainable_block_sparse_sas_amd import binding as sas
    from trainable_block_sparse_sas_amd.pipeline import DecodeStep, TrainStep

DEV = "cuda"


def _twice(run, outs, partial=(), fill=float("nan")):
    """run() writes `outs` (and `partial`, outputs it writes only in part, such
    as the rows of a page pool that a prompt reaches); the two runs must agree
    bit for bit.  `outs` are overwritten with `fill` (NaN; integer outputs -7)
    between the runs; a call that leaves part of an output to the caller's fill
    (scores beyond the history: -inf; ds there: 0) is given that fill."""
    run()
    torch.cuda.synchronize()
    first = [o.clone() for o in list(outs) + list(partial)]
    for o in outs:
        if o.is_floating_point():
            o.fill_(fill)
        else:
            o.fill_(-7)
    run()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(first, list(outs) + list(partial))):
        assert a.dtype == b.dtype and a.shape == b.shape
        # compare the bit patterns (NaN-safe; -0.0 and +0.0 differ)
        if a.is_floating_point():
            a = a.view(torch.int16 if a.element_size() == 2 else torch.int32)
            b = b.view(torch.int16 if b.element_size() == 2 else torch.int32)
        assert torch.equal(a, b), f"output {i} differs between two identical runs"


@pytest.mark.parametrize("topk", [None, 3], ids=["full", "sparse"])
def test_training_entry_points_deterministic(topk):
    w = Workload("det", "train", "bf16", 1, 8, 2, 128, 4672, 64, topk, index=21)
    q, k, v, do = training_inputs(w, device=DEV)
    step = TrainStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, topk, torch.bfloat16)
    sel_outs = [step.kbar, step.lse_s] + ([] if topk is None else [step.idx])
    # the gate normaliser LSE_s; the gated Top-K's log gates (slots from the
    # row's candidate count on are not written)
    _twice(lambda: step.select(q, k), sel_outs, partial=[] if step.gates is None else [step.gates])
    _twice(lambda: step.select(q, k), [step.scores], fill=float("-inf"))  # history columns
    grads = [step.dq, step.dk, step.dv, step.ds]
    # LSE_s computed, lists built by each call
    _twice(lambda: step.forward(q, k, v, step.scores), [step.o, step.lse, step.lse_s])
    _twice(lambda: step.backward(q, k, v, do, step.scores), grads)
    # LSE_s given and the saved context (written in part: the list capacity)
    ctx = [] if step.ctx is None else [step.ctx]
    _twice(lambda: step.forward(q, k, v), [step.o, step.lse], partial=ctx)
    _twice(lambda: step.backward(q, k, v, do), grads[:3])
    _twice(lambda: step.backward(q, k, v, do), [step.ds], fill=0.0)  # history columns
    # the gate variants
    B, Hq, Hkv, N, D, C = w.B, w.Hq, w.Hkv, w.N, w.D, w.C
    tk = -1 if topk is None else topk
    wsf = sas.workspace(sas.SAS_OP_FWD_GATE, B, Hq, Hkv, N, D, w.block, tk, sas.SAS_BF16, DEV)
    wsb = sas.workspace(sas.SAS_OP_BWD_GATE, B, Hq, Hkv, N, D, w.block, tk, sas.SAS_BF16, DEV)
    for gate in (sas.SAS_GATE_SIGMOID, sas.SAS_GATE_RAW, sas.SAS_GATE_OUTER, sas.SAS_GATE_STE):
        o, lse, lse_s = torch.empty_like(q), torch.empty_like(step.lse), torch.empty_like(step.lse_s)
        _twice(lambda: sas.sas_gated_attn_fwd_gate(q, k, v, step.scores, step.idx, o, lse, lse_s, w.block,
                                                   w.scale, gate, wsf), [o, lse, lse_s])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ds = torch.empty((B, Hq, N, C), dtype=torch.float32, device=DEV)
        _twice(lambda: sas.sas_gated_attn_bwd_gate(q, k, v, o, do, step.scores, step.idx, lse, lse_s, dq, dk, dv,
                                                   ds, w.block, w.scale, gate, wsb), [dq, dk, dv, ds])
    # the selector backward, on the softmax gate's ds
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dkbar = torch.empty((B, Hkv, C, D), dtype=torch.float32, device=DEV)
    wss = sas.workspace(sas.SAS_OP_SELECTOR_BWD, B, Hq, Hkv, N, D, w.block, -1, sas.SAS_BF16, DEV)
    _twice(lambda: sas.sas_selector_bwd(q, step.kbar, step.ds, dq, dk, w.block, w.scale, dkbar=dkbar,
                                        workspace=wss), [dq, dk, dkbar])


def test_decode_entry_points_deterministic():
    B, Hq, Hkv, D, L, block, topk = 4, 8, 2, 128, 4096, 64, 5
    w = Workload("det-dec", "decode", "bf16", B, Hq, Hkv, D, L, block, topk, index=22)
    q, kc, vc, _ = decode_inputs(w, device=DEV)
    lens = torch.tensor([L, L - 100, 70, 0], dtype=torch.int32, device=DEV)
    step = DecodeStep(B, Hq, Hkv, L, D, block, topk, torch.bfloat16)
    step.pool(kc)
    _twice(lambda: step.select(q, lens), [step.u, step.idx])
    _twice(lambda: step.attend(q, kc, vc, lens), [step.o, step.lse])
    dense = DecodeStep(B, Hq, Hkv, L, D, block, None, torch.bfloat16)
    _twice(lambda: dense.attend(q, kc, vc, lens), [dense.o, dense.lse])
    # paged: the cache's blocks as pages in order
    C = L // block
    kp = kc.reshape(B, Hkv, C, block, D).permute(0, 2, 1, 3, 4).reshape(B * C, Hkv, block, D).contiguous()
    vp = vc.reshape(B, Hkv, C, block, D).permute(0, 2, 1, 3, 4).reshape(B * C, Hkv, block, D).contiguous()
    table = torch.arange(B * C, dtype=torch.int32, device=DEV).reshape(B, C)
    kbp = torch.empty((B * C, Hkv, D), dtype=torch.bfloat16, device=DEV)
    _twice(lambda: sas.sas_pool_pages(kp, kbp, table.reshape(-1).contiguous(), block), [kbp])
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=DEV)
    ws = sas.workspace(sas.SAS_OP_PAGED_DECODE, B, Hq, Hkv, L, D, block, topk, sas.SAS_BF16)
    _twice(lambda: sas.sas_paged_decode(q, kp, vp, kbp, table, lens, topk, o, lse, block, w.scale, idx_out=idx,
                                        workspace=ws), [o, lse, idx])
    # the dense prefill into pages
    N = 640
    qp, kq, vq = (torch.randn((B, h, N, D), generator=torch.Generator(device=DEV).manual_seed(5 + h), device=DEV)
                  .to(torch.bfloat16) for h in (Hq, Hkv, Hkv))
    seq = torch.tensor([N, 600, 130, 1], dtype=torch.int32, device=DEV)
    tab2 = torch.arange(B * 10, dtype=torch.int32, device=DEV).reshape(B, 10)
    kp2 = torch.zeros((B * 10, Hkv, block, D), dtype=torch.bfloat16, device=DEV)
    vp2, kb2 = torch.zeros_like(kp2), torch.zeros((B * 10, Hkv, D), dtype=torch.bfloat16, device=DEV)
    op = torch.empty_like(qp)
    lp = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    wsp = sas.workspace(sas.SAS_OP_PREFILL, B, Hq, Hkv, N, D, block, 0, sas.SAS_BF16)
    _twice(lambda: sas.sas_prefill_paged(qp, kq, vq, seq, op, lp, kp2, vp2, kb2, tab2, block, w.scale, wsp),
           [op, lp], partial=[kp2, vp2, kb2])
    # the one-call step on the contiguous cache
    wsd = sas.workspace(sas.SAS_OP_DECODE_STEP, B, Hq, Hkv, L, D, block, topk, sas.SAS_BF16)
    _twice(lambda: sas.sas_decode_step(q, step.kbar, kc, vc, lens, topk, o, lse, block, w.scale, idx_out=idx,
                                       workspace=wsd), [o, lse, idx])


@pytest.mark.slow
def test_benchmark_shapes_deterministic():
    """The 32K sparse training step and the 512K decode step, as bench.py runs them."""
    w = WORKLOADS[2]
    q, k, v, do = training_inputs(w, device=DEV)
    step = TrainStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk, w.torch_dtype)
    # scores and ds: the step writes their history columns only (the rest
    # keeps the step's -inf and zero fills), so they are not refilled
    _twice(lambda: step.run(q, k, v, do),
           [step.kbar, step.idx, step.o, step.lse, step.lse_s, step.dq, step.dk, step.dv],
           partial=[step.scores, step.ds] + ([] if step.gates is None else [step.gates]))
    del step, q, k, v, do
    torch.cuda.empty_cache()
    w = WORKLOADS[4]
    q, kc, vc, lens = decode_inputs(w, device=DEV)
    d = DecodeStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk, w.torch_dtype)
    d.pool(kc)
    torch.cuda.synchronize()
    _twice(lambda: d.run(q, kc, vc, lens), [d.u, d.idx, d.o, d.lse])
    ws = sas.workspace(sas.SAS_OP_DECODE_STEP, w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk, sas.SAS_BF16)
    _twice(lambda: sas.sas_decode_step(q, d.kbar, kc, vc, lens, w.topk, d.o, d.lse, w.block, w.scale, idx_out=d.idx,
                                       workspace=ws), [d.o, d.lse, d.idx])
