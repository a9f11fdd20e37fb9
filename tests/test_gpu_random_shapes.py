"""GPU parity over seeded random small shapes (beside the fixed cases).

Each case draws its shape from a fixed seed (numpy default_rng): ragged token
counts, every group size the kernels specialise, D 64 and 128, blocks 16 to
128, Top-K from 0 to past the history, bf16 and fp32; decode lengths that are
idle, ragged, full or over the capacity.  The oracle's scores and indices feed
the attention calls, as in the fixed training cases; decode runs the whole
step (sas_decode_step) and is held to the oracle on the scores it selected on;
the gate variants (sigmoid, raw logit, outer, straight-through) and the
selector backward run on random shapes too.
Tolerances are those of the fixed cases (tests/gpu_util.py).
"""
import numpy as np
import pytest
import torch

from oracle import sas_oracle as orc
from tests.gpu_util import kbar_close, max_abs, normwise, to64, tolerances
from trainable_block_sparse_sas_amd.inputs import Workload, decode_inputs, training_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from trainable_block_sparse_sas_amd import binding as sas
    from trainable_block_sparse_sas_amd.pipeline import TrainStep

DEV = "cuda"


def _train_shape(i):
    r = np.random.default_rng(7000 + i)
    dts = "bf16" if r.random() < 0.75 else "f32"
    block = 64 if r.random() < 0.7 else int(r.choice([16, 32]))
    Hkv = int(r.choice([1, 2]))
    G = int(r.choice([1, 2, 4, 8]))
    D = int(r.choice([64, 128]))
    N = int(r.integers(block, 900))
    C = N // block
    topk = None if r.random() < 0.3 else int(r.integers(0, C + 3))
    B = int(r.choice([1, 2]))
    return dts, B, Hkv * G, Hkv, D, N, block, topk


def _train_shape_many(i):
    """Longer rows selecting most of their history (long selection lists,
    many P V slots per row)."""
    r = np.random.default_rng(7500 + i)
    Hkv = int(r.choice([1, 2]))
    G = int(r.choice([1, 2, 4, 8]))
    D = int(r.choice([64, 128]))
    N = int(r.integers(1000, 3000))
    C = N // 64
    topk = int(r.integers(C // 2, C + 3))
    return "bf16", 1, Hkv * G, Hkv, D, N, 64, topk


TRAIN_IDS = list(range(20)) + list(range(100, 108))


@pytest.mark.parametrize("i", TRAIN_IDS, ids=[f"train{i}" for i in TRAIN_IDS])
def test_training_random_shape(i):
    dts, B, Hq, Hkv, D, N, block, topk = _train_shape(i) if i < 100 else _train_shape_many(i)
    print(f"case train{i}: {dts} B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} block{block} topk{topk}", flush=True)
    dt = torch.float32 if dts == "f32" else torch.bfloat16
    w = Workload(f"rand{i}", "train", dts, B, Hq, Hkv, D, N, block, topk, index=20 + i)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    G, scale, tol = Hq // Hkv, w.scale, tolerances(dt)
    q64, k64 = to64(q), to64(k)
    kbar = orc.pool_block_keys(k64, block)
    kbar_r = to64(torch.tensor(kbar).to(dt))
    pos = np.broadcast_to(np.arange(N), (B, N))
    s32 = orc.block_scores(q64, kbar_r, block, scale, pos).astype(np.float32)
    idx = None if topk is None else orc.topk_select(s32, G, pos // block, topk)
    step = TrainStep(B, Hq, Hkv, N, D, block, topk, dt)
    step.select(q, k)
    torch.cuda.synchronize()
    if dt == torch.float32:
        normwise(to64(step.kbar), kbar, 1e-6, "kbar")
    else:
        kbar_close(to64(step.kbar), kbar_r)
    scores = torch.tensor(s32).to(DEV)
    idx_t = None
    if topk is not None:
        sas.sas_topk_select(scores, step.idx, None, G, block)
        torch.cuda.synchronize()
        assert np.array_equal(step.idx.cpu().numpy(), idx), "topk"
        idx_t = torch.tensor(idx).to(DEV)
    step.forward(q, k, v, scores, idx_t)
    step.backward(q, k, v, do, scores, idx_t)
    torch.cuda.synchronize()
    s64 = s32.astype(np.float64)
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(q64, k64, to64(v), s64, idx, block, scale)
    if tol["o_abs"] is not None:
        max_abs(to64(step.o), o_ref, tol["o_abs"], "o")
    else:
        normwise(to64(step.o), o_ref, tol["o_rel"], "o")
    normwise(to64(step.lse), lse_ref, tol["lse"], "lse")
    normwise(to64(step.lse_s), lses_ref, tol["lse"], "lse_s")
    dq, dk, dv, ds = orc.gated_attention_backward(q64, k64, to64(v), to64(do), s64, idx, block, scale)
    normwise(to64(step.dq), dq, tol["grad"], "dq")
    normwise(to64(step.dk), dk, tol["grad"], "dk")
    normwise(to64(step.dv), dv, tol["grad"], "dv")
    normwise(to64(step.ds), ds, tol["ds"], "ds")


def _decode_shape(i):
    r = np.random.default_rng(8000 + i)
    dts = "bf16" if r.random() < 0.8 else "f32"
    block = int(r.choice([16, 32, 64, 64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 5, 8]))
    D = int(r.choice([64, 128]))
    C = int(r.integers(1, 160))
    L = C * block + int(r.integers(0, block))
    B = int(r.integers(1, 5))
    lens = [int(x) for x in r.integers(-1, L + 2 * block, size=B)]
    lens[0] = L  # one full cache
    if B >= 2:
        lens[1] = L + int(r.integers(1, 3 * block))  # over the capacity: counts as L
    if B >= 3:
        lens[2] = 0  # idle
    topk = int(r.integers(0, min(C + 3, 70)))
    return dts, B, Hkv * G, Hkv, D, L, block, topk, lens


DECODE_IDS = list(range(16))


@pytest.mark.parametrize("i", DECODE_IDS, ids=[f"decode{i}" for i in DECODE_IDS])
def test_decode_step_random_shape(i):
    dts, B, Hq, Hkv, D, L, block, topk, lens_l = _decode_shape(i)
    print(f"case decode{i}: {dts} B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} block{block} topk{topk} lens{lens_l}",
          flush=True)
    dt = torch.float32 if dts == "f32" else torch.bfloat16
    w = Workload(f"drand{i}", "decode", dts, B, Hq, Hkv, D, L, block, topk, index=40 + i)
    q, kc, vc, _ = decode_inputs(w, device="cpu")
    lens = torch.tensor(lens_l, dtype=torch.int32)
    C = L // block
    kbar_r = to64(torch.tensor(orc.pool_block_keys(to64(kc), block)).to(dt))
    o = torch.full((B, Hq, D), float("nan"), dtype=dt, device=DEV)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((B, Hkv, max(topk, 1)), -7, dtype=torch.int32, device=DEV)
    ws = sas.workspace(sas.SAS_OP_DECODE_STEP, B, Hq, Hkv, L, D, block, topk,
                       sas.SAS_BF16 if dt == torch.bfloat16 else sas.SAS_F32)
    sas.sas_decode_step(q.to(DEV), torch.tensor(kbar_r).to(dt).to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV),
                        topk, o, lse, block, w.scale, idx_out=idx[..., :topk] if topk > 0 else None, workspace=ws)
    torch.cuda.synchronize()
    u_ref = orc.decode_scores(to64(q), kbar_r, lens.numpy(), L, block, w.scale, True)
    u_gpu = ws[: B * Hkv * C * 4].view(torch.float32).reshape(B, Hkv, C).cpu().numpy()
    normwise(u_gpu.astype(np.float64), u_ref.astype(np.float64), 1e-5, "u")
    assert np.array_equal(np.isneginf(u_gpu), np.isneginf(u_ref))
    c = orc.decode_candidates(lens.numpy(), L, block)
    idx_ref = np.zeros((B, Hkv, 0), dtype=np.int64)
    if topk > 0:
        idx_ref = orc.topk_select(u_gpu[:, :, None, :], 1, c[:, None], topk)[:, :, 0, :]
        assert np.array_equal(idx.cpu().numpy()[..., :topk], idx_ref), "Top-K on the step's own scores"
    o_ref, lse_ref = orc.sparse_decode(to64(q), to64(kc), to64(vc), lens.numpy(), idx_ref, block, w.scale)
    active = lens.numpy() > 0
    tol = tolerances(dt)
    if tol["o_abs"] is not None:
        max_abs(to64(o)[active], o_ref[active], tol["o_abs"], "o")
    else:
        normwise(to64(o)[active], o_ref[active], tol["o_rel"], "o")
    normwise(to64(lse)[active], lse_ref[active], 1e-4, "lse")
    assert torch.all(o[~torch.tensor(active)] == 0)


GATES = ["sigmoid", "raw", "outer"]
GATE_IDS = list(range(12))


@pytest.mark.parametrize("i", GATE_IDS, ids=[f"gate{i}" for i in GATE_IDS])
def test_gate_variant_random_shape(i):
    """sas_gated_attn_fwd_gate / _bwd_gate with the sigmoid, raw-logit and outer
    gates on random shapes, against the oracle's gate variants."""
    dts, B, Hq, Hkv, D, N, block, topk = _train_shape(100 + i)
    gate = GATES[i % 3]
    print(f"case gate{i}: {gate} {dts} B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} block{block} topk{topk}", flush=True)
    dt = torch.float32 if dts == "f32" else torch.bfloat16
    w = Workload(f"grand{i}", "train", dts, B, Hq, Hkv, D, N, block, topk, index=60 + i)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    G, scale, tol, C = Hq // Hkv, w.scale, tolerances(dt), N // block
    q64, k64, v64 = to64(q), to64(k), to64(v)
    kbar_r = to64(torch.tensor(orc.pool_block_keys(k64, block)).to(dt))
    pos = np.broadcast_to(np.arange(N), (B, N))
    s32 = orc.block_scores(q64, kbar_r, block, scale, pos).astype(np.float32)
    idx = None if topk is None else orc.topk_select(s32, G, pos // block, topk)
    scores = torch.tensor(s32).to(DEV)
    idx_t = None if idx is None else torch.tensor(idx).to(DEV)
    g = {"sigmoid": sas.SAS_GATE_SIGMOID, "raw": sas.SAS_GATE_RAW, "outer": sas.SAS_GATE_OUTER}[gate]
    tk = -1 if topk is None else topk
    sdt = sas.SAS_F32 if dt == torch.float32 else sas.SAS_BF16
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    lse_s = torch.full((B, Hq, N), 7.0, dtype=torch.float32, device=DEV)
    wsf = sas.workspace(sas.SAS_OP_FWD_GATE, B, Hq, Hkv, N, D, block, tk, sdt, DEV)
    sas.sas_gated_attn_fwd_gate(q, k, v, scores, idx_t, o, lse, lse_s, block, scale, g, wsf)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty((B, Hq, N, C), dtype=torch.float32, device=DEV)
    wsb = sas.workspace(sas.SAS_OP_BWD_GATE, B, Hq, Hkv, N, D, block, tk, sdt, DEV)
    sas.sas_gated_attn_bwd_gate(q, k, v, o, do, scores, idx_t, lse, lse_s if gate == "outer" else None, dq, dk,
                                dv, ds, block, scale, g, wsb)
    torch.cuda.synchronize()
    s64 = s32.astype(np.float64)
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(q64, k64, v64, s64, idx, block, scale, gate=gate)
    if tol["o_abs"] is not None:
        max_abs(to64(o), o_ref, tol["o_abs"], "o")
    else:
        normwise(to64(o), o_ref, tol["o_rel"], "o")
    normwise(to64(lse), lse_ref, tol["lse"], "lse")
    if gate == "outer":
        normwise(to64(lse_s), lses_ref, tol["lse"], "lse_s")
    else:
        assert torch.count_nonzero(lse_s).item() == 0, "lse_s"
    r_dq, r_dk, r_dv, r_ds = orc.gated_attention_backward(q64, k64, v64, to64(do), s64, idx, block, scale,
                                                          gate=gate)
    normwise(to64(dq), r_dq, tol["grad"], "dq")
    normwise(to64(dk), r_dk, tol["grad"], "dk")
    normwise(to64(dv), r_dv, tol["grad"], "dv")
    normwise(to64(ds), r_ds, tol["ds"], "ds")


SEL_IDS = list(range(6))


@pytest.mark.parametrize("i", SEL_IDS, ids=[f"selector{i}" for i in SEL_IDS])
def test_selector_backward_random_shape(i):
    """sas_selector_bwd on random shapes (ragged tails, every group size, both
    dtypes) against the oracle on the pooled keys as the GPU holds them."""
    dts, B, Hq, Hkv, D, N, block, _ = _train_shape(200 + i)
    print(f"case selector{i}: {dts} B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} block{block}", flush=True)
    dt = torch.float32 if dts == "f32" else torch.bfloat16
    C = N // block
    g = torch.Generator().manual_seed(9000 + i)
    q = torch.randn((B, Hq, N, D), generator=g).to(dt)
    k = torch.randn((B, Hkv, N, D), generator=g).to(dt)
    ds = torch.randn((B, Hq, N, C), generator=g)
    kbar = torch.tensor(orc.pool_block_keys(to64(k), block)).to(dt)
    scale = D ** -0.5
    dq_ref, dkbar_ref, dk_ref = orc.selector_backward(to64(q), to64(k), ds.numpy(), block, scale, kbar=to64(kbar))
    ws = sas.workspace(sas.SAS_OP_SELECTOR_BWD, B, Hq, Hkv, N, D, block, -1,
                       sas.SAS_BF16 if dt == torch.bfloat16 else sas.SAS_F32)
    dq = torch.full((B, Hq, N, D), float("nan"), dtype=dt, device=DEV)
    dk = torch.full((B, Hkv, N, D), float("nan"), dtype=dt, device=DEV)
    dkbar = torch.empty((B, Hkv, C, D), dtype=torch.float32, device=DEV)
    sas.sas_selector_bwd(q.to(DEV), kbar.to(DEV), ds.to(DEV), dq, dk, block, scale, dkbar=dkbar, workspace=ws)
    torch.cuda.synchronize()
    tol = 1e-5 if dt == torch.float32 else 2e-2
    normwise(to64(dq), dq_ref, tol, "dq")
    normwise(to64(dkbar), dkbar_ref, tol, "dkbar")
    normwise(to64(dk), dk_ref, tol, "dk")
    assert torch.all(dk[:, :, C * block:] == 0)


STE_IDS = list(range(6))


@pytest.mark.parametrize("i", STE_IDS, ids=[f"ste{i}" for i in STE_IDS])
def test_ste_gate_random_shape(i):
    """The hard gate with a straight-through estimator on random shapes (both
    scopes), against the oracle's reading of it."""
    dts, B, Hq, Hkv, D, N, block, topk = _train_shape(300 + i)
    N = min(N, 600)  # the oracle's STE visits every history block of every row
    print(f"case ste{i}: {dts} B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} block{block} topk{topk}", flush=True)
    dt = torch.float32 if dts == "f32" else torch.bfloat16
    if topk is not None:
        topk = min(topk, N // block + 2)
    w = Workload(f"srand{i}", "train", dts, B, Hq, Hkv, D, N, block, topk, index=80 + i)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    G, scale, tol, C = Hq // Hkv, w.scale, tolerances(dt), N // block
    q64, k64, v64 = to64(q), to64(k), to64(v)
    kbar_r = to64(torch.tensor(orc.pool_block_keys(k64, block)).to(dt))
    pos = np.broadcast_to(np.arange(N), (B, N))
    s32 = orc.block_scores(q64, kbar_r, block, scale, pos).astype(np.float32)
    idx = None if topk is None else orc.topk_select(s32, G, pos // block, topk)
    scores = torch.tensor(s32).to(DEV)
    idx_t = None if idx is None else torch.tensor(idx).to(DEV)
    tk = -1 if topk is None else topk
    sdt = sas.SAS_F32 if dt == torch.float32 else sas.SAS_BF16
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    lse_s = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    wsf = sas.workspace(sas.SAS_OP_FWD_GATE, B, Hq, Hkv, N, D, block, tk, sdt, DEV)
    sas.sas_gated_attn_fwd_gate(q, k, v, scores, idx_t, o, lse, lse_s, block, scale, sas.SAS_GATE_STE, wsf)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty((B, Hq, N, C), dtype=torch.float32, device=DEV)
    wsb = sas.workspace(sas.SAS_OP_BWD_GATE, B, Hq, Hkv, N, D, block, tk, sdt, DEV)
    sas.sas_gated_attn_bwd_gate(q, k, v, o, do, scores, idx_t, lse, lse_s, dq, dk, dv, ds, block, scale,
                                sas.SAS_GATE_STE, wsb)
    torch.cuda.synchronize()
    o_ref, lse_ref, lses_ref, dq_r, dk_r, dv_r, ds_r = orc.ste_gate_attention(
        q64, k64, v64, to64(do), s32.astype(np.float64), idx, block, scale)
    if tol["o_abs"] is not None:
        max_abs(to64(o), o_ref, tol["o_abs"], "o")
    else:
        normwise(to64(o), o_ref, tol["o_rel"], "o")
    normwise(to64(lse), lse_ref, tol["lse"], "lse")
    normwise(to64(lse_s), lses_ref, tol["lse"], "lse_s")
    normwise(to64(dq), dq_r, tol["grad"], "dq")
    normwise(to64(dk), dk_r, tol["grad"], "dk")
    normwise(to64(dv), dv_r, tol["grad"], "dv")
    normwise(to64(ds), ds_r, tol["ds"], "ds")
