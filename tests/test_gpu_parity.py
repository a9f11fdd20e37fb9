"""GPU parity of every libsas entry point against the CPU oracle (small shapes).

Inputs come from the seeded generators; selector scores and Top-K indices fed
to the attention calls come from the oracle, so each entry point is compared
on identical inputs.  Tolerances: see tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

from oracle import sas_oracle as orc
from tests.gpu_util import kbar_close, max_abs, normwise, to64, tolerances
from trainable_block_sparse_sas_amd.inputs import Workload, decode_inputs, score_matrix, training_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from trainable_block_sparse_sas_amd import binding as sas
    from trainable_block_sparse_sas_amd.pipeline import DecodeStep, TrainStep

DEV = "cuda"


def _dt(name):
    return torch.float32 if name == "f32" else torch.bfloat16


def _oracle_selector(q, k, block, scale, topk, G):
    """Oracle pooled keys, fp32 scores and (sparse scope) indices for training rows."""
    q64, k64 = to64(q), to64(k)
    kbar = orc.pool_block_keys(k64, block)
    kbar_r = to64(torch.tensor(kbar).to(q.dtype))  # pooled keys are stored in the input dtype
    N = q.shape[2]
    pos = np.broadcast_to(np.arange(N), (q.shape[0], N))
    s32 = orc.block_scores(q64, kbar_r, block, scale, pos).astype(np.float32)
    idx = None
    if topk is not None:
        idx = orc.topk_select(s32, G, pos // block, topk)
    return kbar, kbar_r, s32, idx


TRAIN_CASES = [
    # name, dtype, B, Hq, Hkv, D, N, block, topk
    ("tiny-f32-full", "f32", 1, 2, 1, 64, 512, 64, None),
    ("f32-ragged-sparse", "f32", 2, 4, 2, 64, 300, 64, 2),
    ("f32-block16-sparse", "f32", 1, 2, 1, 128, 130, 16, 3),
    ("bf16-full", "bf16", 1, 8, 2, 128, 384, 64, None),
    ("bf16-ragged-sparse", "bf16", 1, 8, 2, 128, 450, 64, 3),
    ("bf16-g1-d64-sparse", "bf16", 2, 4, 4, 64, 256, 64, 1),
    ("bf16-block32-sparse", "bf16", 1, 4, 1, 128, 200, 32, 2),
    ("bf16-topk0", "bf16", 1, 4, 2, 128, 256, 64, 0),
    # G = 2 and D = 64 at sparse scope; and G = 8 over several token spans of the
    # key-major work items, with block lists longer than one work item
    ("bf16-g2-d64-sparse", "bf16", 2, 4, 2, 64, 640, 64, 4),
    ("bf16-g8-spans-sparse", "bf16", 1, 8, 1, 128, 4672, 64, 5),
    # D = 64 (two P V slots per pass in the combine) with rows selecting 15,
    # 31 and 33 .. 40 blocks: counts where the two lane halves' loops end apart
    ("bf16-d64-many-sel", "bf16", 1, 4, 2, 64, 2600, 64, 40),
]


@pytest.mark.parametrize("case", TRAIN_CASES, ids=[c[0] for c in TRAIN_CASES])
def test_training_parity(case):
    name, dts, B, Hq, Hkv, D, N, block, topk = case
    dt = _dt(dts)
    w = Workload(name, "train", dts, B, Hq, Hkv, D, N, block, topk, index=7)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    scale = w.scale
    G = Hq // Hkv
    tol = tolerances(dt)
    kbar, kbar_r, s32, idx = _oracle_selector(q, k, block, scale, topk, G)
    step = TrainStep(B, Hq, Hkv, N, D, block, topk, dt)

    # Selector: pooled keys and scores.
    step.select(q, k)
    torch.cuda.synchronize()
    gk = to64(step.kbar)
    if dt == torch.float32:
        normwise(gk, kbar, 1e-6, "kbar")
    else:  # fp32 mean rounded to bf16: at most one bf16 step from the rounded exact mean
        kbar_close(gk, kbar_r)
    sc_in = torch.tensor(kbar_r).to(dt).to(DEV)
    sas.sas_score_blocks(q, None, sc_in, step.scores, None, block, scale)
    torch.cuda.synchronize()
    normwise(to64(step.scores), s32.astype(np.float64), 1e-5, "scores")

    # Top-K on the oracle's fp32 scores: bit-exact.
    scores = torch.tensor(s32).to(DEV)
    idx_t = None
    if topk is not None:
        sas.sas_topk_select(scores, step.idx, None, G, block)
        torch.cuda.synchronize()
        assert np.array_equal(step.idx.cpu().numpy(), idx), "topk"
        idx_t = torch.tensor(idx).to(DEV)

    # Forward.
    step.forward(q, k, v, scores, idx_t)
    torch.cuda.synchronize()
    s64 = s32.astype(np.float64)
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(to64(q), to64(k), to64(v), s64, idx, block, scale)
    if tol["o_abs"] is not None:
        max_abs(to64(step.o), o_ref, tol["o_abs"], "o")
    else:
        normwise(to64(step.o), o_ref, tol["o_rel"], "o")
    normwise(to64(step.lse), lse_ref, tol["lse"], "lse")
    normwise(to64(step.lse_s), lses_ref, tol["lse"], "lse_s")

    # Backward.
    step.backward(q, k, v, do, scores, idx_t)
    torch.cuda.synchronize()
    dq, dk, dv, ds = orc.gated_attention_backward(to64(q), to64(k), to64(v), to64(do), s64, idx, block, scale)
    normwise(to64(step.dq), dq, tol["grad"], "dq")
    normwise(to64(step.dk), dk, tol["grad"], "dk")
    normwise(to64(step.dv), dv, tol["grad"], "dv")
    normwise(to64(step.ds), ds, tol["ds"], "ds")


@pytest.mark.parametrize("case", TRAIN_CASES, ids=[c[0] for c in TRAIN_CASES])
def test_training_step_own_path(case):
    """The training step's own path: sas_score_blocks_lse writes the scores of
    sas_score_blocks bit for bit plus the gate normaliser LSE_s (jaehun.me
    review, "Why the Four Design Choices Matter": log g = s - LSE(s));
    sas_gated_attn_fwd_ctx on them (LSE_s given, saved context written) and
    sas_gated_attn_bwd_ctx (lists and log gates from the context) match the
    oracle forward and backward on the same scores and indices.  LSE_s: fp32
    running max and exp sum with the hardware exp2 and log, a few ulps: 1e-5
    normwise."""
    name, dts, B, Hq, Hkv, D, N, block, topk = case
    dt = _dt(dts)
    w = Workload(name, "train", dts, B, Hq, Hkv, D, N, block, topk, index=11)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    scale = w.scale
    tol = tolerances(dt)
    step = TrainStep(B, Hq, Hkv, N, D, block, topk, dt)
    step.lse_s.fill_(float("nan"))
    step.select(q, k)
    s2 = torch.full_like(step.scores, float("nan"))
    sas.sas_score_blocks(q, None, step.kbar, s2, None, block, scale)
    torch.cuda.synchronize()
    assert torch.equal(s2, step.scores), "scores differ from sas_score_blocks"
    s64 = to64(step.scores)
    idx = None if topk is None else step.idx.cpu().numpy()
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(to64(q), to64(k), to64(v), s64, idx, block, scale)
    normwise(to64(step.lse_s), lses_ref, 1e-5, "lse_s")
    lse_s_in = step.lse_s.clone()
    step.forward(q, k, v)  # the step's own scores: LSE_s given, the context saved
    torch.cuda.synchronize()
    assert torch.equal(step.lse_s, lse_s_in), "lse_s is an input of the forward"
    if step.gates is not None:
        # the gated Top-K's log gates stand in for the forward's own: same bits
        o2, lse2 = torch.empty_like(step.o), torch.empty_like(step.lse)
        ctx2 = None if step.ctx is None else torch.empty_like(step.ctx)
        sas.sas_gated_attn_fwd_ctx(q, k, v, step.scores, step.idx, step.lse_s, o2, lse2, block, scale, ctx2,
                                   step.ws_fwd)
        torch.cuda.synchronize()
        assert torch.equal(o2, step.o) and torch.equal(lse2, step.lse), "forward with and without given gates"
    if tol["o_abs"] is not None:
        max_abs(to64(step.o), o_ref, tol["o_abs"], "o")
    else:
        normwise(to64(step.o), o_ref, tol["o_rel"], "o")
    normwise(to64(step.lse), lse_ref, tol["lse"], "lse")
    step.backward(q, k, v, do)  # from the saved context
    torch.cuda.synchronize()
    dq, dk, dv, ds = orc.gated_attention_backward(to64(q), to64(k), to64(v), to64(do), s64, idx, block, scale)
    # history columns only: the columns m >= c(t) keep what the buffers held
    C = step.scores.shape[-1]
    future = torch.arange(C, device=DEV)[None, :] >= (torch.arange(N, device=DEV) // block)[:, None]
    s_mark = torch.full_like(step.scores, 7.0)
    sas.sas_score_blocks_lse(q, None, step.kbar, s_mark, torch.empty_like(step.lse_s), block, scale)
    ds_mark = torch.full_like(step.ds, 7.0)
    sas.sas_gated_attn_bwd_ctx(q, k, v, step.o, do, step.scores, step.idx, step.lse, step.lse_s, step.ctx,
                               step.dq, step.dk, step.dv, ds_mark, block, scale, step.ws_bwd)
    torch.cuda.synchronize()
    fut = future[None, None].expand_as(s_mark)
    assert bool((s_mark[fut] == 7.0).all()), "scores written beyond the history"
    assert torch.equal(s_mark[~fut], step.scores[~fut]), "history scores"
    if step.ctx is not None:  # the saved-context path (matrix cores): ds beyond the history untouched
        assert bool((ds_mark[fut] == 7.0).all()), "ds written beyond the history"
    assert torch.equal(ds_mark[~fut], step.ds[~fut]), "history ds"
    normwise(to64(step.dq), dq, tol["grad"], "dq")
    normwise(to64(step.dk), dk, tol["grad"], "dk")
    normwise(to64(step.dv), dv, tol["grad"], "dv")
    normwise(to64(step.ds), ds, tol["ds"], "ds")


TOPK_CASES = [
    # C, hpr, training(1)-or-None(decode), topk
    (40, 4, 1, 5),
    (300, 1, 1, 32),
    (900, 2, 1, 64),
    (1500, 1, 1, 32),
    (2047, 1, None, 16),
    (8191, 1, None, 32),
    (8191, 1, None, 64),
    (16000, 1, None, 8),
    (3000, 1, None, 17),
    (12000, 1, None, 1),
    (2500, 3, 1, 40),
    (5000, 1, None, 256),
    (12000, 1, None, 40),   # 8-wave runs with 32 candidates a lane, K in 33..64 and 17..32
    (16384, 2, None, 64),
    (9000, 1, None, 24),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=[f"C{c[0]}-h{c[1]}-k{c[3]}" for c in TOPK_CASES])
def test_topk_bit_exact(case):
    C, hpr, Nq, topk = case
    Hkv, block = 2, 4
    if Nq is None:  # decode rows of several lengths, including an idle one
        B = 5
        s = score_matrix((B, Hkv * hpr, C), seed=C)
        s = torch.where(torch.rand(s.shape, generator=torch.Generator().manual_seed(1)) < 0.2,
                        torch.round(s * 4) / 4, s)
        lens = torch.tensor([C * block + 1, 1 + block * 7, 0, C * block // 2, block * (C + 3)],
                            dtype=torch.int32)
        c = np.minimum(np.maximum(lens.numpy() - 1, 0) // block, C)
        c[lens.numpy() <= 0] = 0
        ref = orc.topk_select(s.numpy()[:, :, None, :], hpr, c[:, None], topk)[:, :, 0, :]
        idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=DEV)
        sas.sas_topk_select(s.to(DEV), idx, lens.to(DEV), hpr, block)
    else:
        B = 1
        N = C + 8  # block 1: row t has min(t, C) candidates
        s = score_matrix((B, Hkv * hpr, N, C), seed=C + 1)
        s = torch.round(s * 8) / 8  # many exact ties
        s[0, 0, :, :3] = torch.tensor([float("nan"), -0.0, 0.0])
        s[0, 0, :, 3:5] = torch.tensor([float("inf"), float("-inf")])
        pos = np.arange(N)[None, :]
        ref = orc.topk_select(s.numpy(), hpr, np.minimum(pos, C), topk)
        idx = torch.empty((B, Hkv, N, topk), dtype=torch.int32, device=DEV)
        sas.sas_topk_select(s.to(DEV), idx, None, hpr, 1)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref)


GATED_TOPK_CASES = [
    # C, hpr, block, topk: the one-wave-per-row range (C <= 1024, topk <= 64)
    (40, 4, 1, 5),
    (300, 1, 1, 32),
    (500, 8, 1, 17),
    (900, 2, 1, 64),
    (160, 4, 64, 32),
]


@pytest.mark.parametrize("case", GATED_TOPK_CASES, ids=[f"C{c[0]}-g{c[1]}-b{c[2]}-k{c[3]}" for c in GATED_TOPK_CASES])
def test_topk_gated_bit_exact(case):
    """sas_topk_select_gated: idx bit for bit as the oracle's Top-K (and as
    sas_topk_select), and slot j of row t holds (s[t, m_j] - LSE_s(t)) log2 e
    for the j-th smallest selected block m_j of every head of the group (the
    softmax gate's log g = s - LSE(s) of jaehun.me review, "Why the Four
    Design Choices Matter", in base 2), as fp32 evaluates that expression;
    slots from min(topk, c) on are left as they were."""
    C, hpr, block, topk = case
    Hkv, B = 2, 1
    N = C + 8 if block == 1 else C * block
    s = score_matrix((B, Hkv * hpr, N, C), seed=C + 7)
    s = torch.round(s * 8) / 8  # many exact ties
    s[0, 0, :, :3] = torch.tensor([float("nan"), -0.0, 0.0])
    s[0, 0, :, 3:5] = torch.tensor([float("inf"), float("-inf")])
    lse_s = torch.randn((B, Hkv * hpr, N), generator=torch.Generator().manual_seed(C)) * 3.0
    c = np.minimum(np.arange(N) // block, C)
    ref = orc.topk_select(s.numpy(), hpr, c[None, :], topk)
    idx = torch.empty((B, Hkv, N, topk), dtype=torch.int32, device=DEV)
    gates = torch.full((B, Hkv, N, topk, hpr), 7.0, dtype=torch.float32, device=DEV)
    sd, ld = s.to(DEV), lse_s.to(DEV)
    sas.sas_topk_select_gated(sd, ld, idx, gates, block)
    idx2 = torch.empty_like(idx)
    sas.sas_topk_select(sd, idx2, None, hpr, block)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(idx2.cpu().numpy(), got)
    # expected log gates, in fp32, by slot in ascending block order
    srt = np.sort(np.where(ref >= 0, ref, np.iinfo(np.int32).max), axis=-1)
    valid = srt != np.iinfo(np.int32).max
    m = torch.from_numpy(np.where(valid, srt, 0).astype(np.int64))  # [B, Hkv, N, topk]
    sg = s.reshape(B, Hkv, hpr, N, C)
    lg = lse_s.reshape(B, Hkv, hpr, N)
    sel = torch.gather(sg, 4, m[:, :, None, :, :].expand(B, Hkv, hpr, N, topk))  # [B, Hkv, hpr, N, topk]
    log2e = torch.tensor(1.4426950408889634, dtype=torch.float32)
    exp = ((sel - lg[..., None]) * log2e).permute(0, 1, 3, 4, 2)  # [B, Hkv, N, topk, hpr]
    exp = torch.where(torch.from_numpy(valid)[..., None], exp, torch.tensor(7.0))
    torch.testing.assert_close(gates.cpu(), exp, rtol=0, atol=0, equal_nan=True)


DECODE_CASES = [
    # name, dtype, Hq, Hkv, D, L, block, topk
    ("bf16-g4", "bf16", 8, 2, 128, 2048, 64, 4),
    ("bf16-g5", "bf16", 10, 2, 128, 1536, 64, 3),
    ("bf16-dense", "bf16", 8, 2, 128, 2048, 64, None),
    ("f32-d64", "f32", 4, 1, 64, 1024, 64, 2),
    ("bf16-block32", "bf16", 4, 2, 128, 1000, 32, 5),
    ("bf16-g16-d64", "bf16", 16, 1, 64, 1280, 64, 3),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_parity(case):
    name, dts, Hq, Hkv, D, L, block, topk = case
    dt = _dt(dts)
    B = 5
    w = Workload(name, "decode", dts, B, Hq, Hkv, D, L, block, topk, index=9)
    q, kc, vc, _ = decode_inputs(w, device="cpu")
    # full, ragged, short, idle, and a length above the capacity (counts as L)
    lens = torch.tensor([L, L - 37, 40, 0, 10 * L + 3], dtype=torch.int32)
    q, kc, vc, lens_d = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    scale = w.scale
    G = Hq // Hkv
    tol = tolerances(dt)
    step = DecodeStep(B, Hq, Hkv, L, D, block, topk if topk is not None else 1, dt)
    # Pooled keys.
    step.pool(kc)
    torch.cuda.synchronize()
    kbar = orc.pool_block_keys(to64(kc), block)
    kbar_r = to64(torch.tensor(kbar).to(dt))
    if dt == torch.float32:
        normwise(to64(step.kbar), kbar, 1e-6, "kbar")
    else:
        kbar_close(to64(step.kbar), kbar_r)
    # Group-summed decode scores from the oracle's pooled keys.
    kb = torch.tensor(kbar_r).to(dt).to(DEV)
    sas.sas_score_blocks(q, None, kb, step.u, lens_d, block, scale, group_sum=True, L=L)
    torch.cuda.synchronize()
    u_ref = orc.decode_scores(to64(q), kbar_r, lens.numpy(), L, block, scale, True)
    normwise(to64(step.u), u_ref.astype(np.float64), 1e-5, "u")
    # -inf in exactly the same places: the current block and beyond, idle rows
    assert np.array_equal(np.isneginf(step.u.cpu().numpy()), np.isneginf(u_ref))
    # Per-head decode scores.
    s_h = torch.empty((B, Hq, L // block), dtype=torch.float32, device=DEV)
    sas.sas_score_blocks(q, None, kb, s_h, lens_d, block, scale, group_sum=False, L=L)
    torch.cuda.synchronize()
    s_ref = orc.decode_scores(to64(q), kbar_r, lens.numpy(), L, block, scale, False)
    normwise(to64(s_h), s_ref, 1e-5, "s")
    assert np.array_equal(np.isneginf(s_h.cpu().numpy()), np.isneginf(s_ref))
    # Top-K on the oracle's group sums: bit-exact.  Top-K does not know the
    # capacity, so (as its header asks) the lengths it gets are clamped to L.
    c = orc.decode_candidates(lens.numpy(), L, block)
    idx_ref = None
    if topk is not None:
        idx_ref = orc.topk_select(u_ref[:, :, None, :], 1, c[:, None], topk)[:, :, 0, :]
        sas.sas_topk_select(torch.tensor(u_ref).to(DEV), step.idx, torch.clamp(lens, max=L).to(DEV), 1, block)
        torch.cuda.synchronize()
        assert np.array_equal(step.idx.cpu().numpy(), idx_ref)
    # Attention over the selected blocks (or all blocks).
    idx_in = None if topk is None else torch.tensor(idx_ref).to(DEV)
    step.ws = sas.workspace(sas.SAS_OP_DECODE, B, Hq, Hkv, L, D, block, -1 if topk is None else topk,
                            sas.SAS_BF16 if dt == torch.bfloat16 else sas.SAS_F32)
    sas.sas_sparse_decode(q, kc, vc, lens_d, idx_in, step.o, step.lse, block, scale, step.ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.sparse_decode(to64(q), to64(kc), to64(vc), lens.numpy(), idx_ref, block, scale)
    active = lens.numpy() > 0
    if tol["o_abs"] is not None:
        max_abs(to64(step.o)[active], o_ref[active], tol["o_abs"], "o")
    else:
        normwise(to64(step.o)[active], o_ref[active], tol["o_rel"], "o")
    normwise(to64(step.lse)[active], lse_ref[active], 1e-4, "lse")
    # Idle sequence: zeros and -inf.
    assert torch.all(step.o[~torch.tensor(active)] == 0)
    assert torch.all(step.lse[~torch.tensor(active)] == float("-inf"))
    # The workspace's arrival counters are back at zero: a second call on the
    # same workspace gives the same bits; so does a call for fewer sequences.
    o1, lse1 = step.o.clone(), step.lse.clone()
    step.o.zero_()
    sas.sas_sparse_decode(q, kc, vc, lens_d, idx_in, step.o, step.lse, block, scale, step.ws)
    torch.cuda.synchronize()
    assert torch.equal(step.o, o1) and torch.equal(step.lse, lse1)
    o2, lse2 = step.o[:2].clone(), step.lse[:2].clone()
    sas.sas_sparse_decode(q[:2].contiguous(), kc[:2].contiguous(), vc[:2].contiguous(), lens_d[:2].contiguous(),
                          None if idx_in is None else idx_in[:2].contiguous(), o2, lse2, block, scale, step.ws)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1[:2]) and torch.equal(lse2, lse1[:2])


def test_empty_sizes_are_noops():
    dt = torch.bfloat16
    z = torch.empty((1, 4, 0, 128), dtype=dt, device=DEV)
    zk = torch.empty((1, 2, 0, 128), dtype=dt, device=DEV)
    sc = torch.empty((1, 4, 0, 0), dtype=torch.float32, device=DEV)
    l = torch.empty((1, 4, 0), dtype=torch.float32, device=DEV)
    sas.sas_gated_attn_fwd(z, zk, zk, sc, None, z, l, l, 64, 0.1)
    sas.sas_gated_attn_bwd(z, zk, zk, z, z, sc, None, l, l, z, zk, zk, sc, 64, 0.1)
    torch.cuda.synchronize()


def test_repeated_and_invalid_idx_entries():
    """Repeated entries count once and entries outside [0, c) are ignored."""
    dt = torch.bfloat16
    B, Hq, Hkv, D, N, block = 1, 4, 2, 128, 320, 64
    w = Workload("dup", "train", "bf16", B, Hq, Hkv, D, N, block, 4, index=11)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    _, _, s32, _ = _oracle_selector(q, k, block, w.scale, None, 2)
    r = np.random.default_rng(3)
    idx = r.integers(-2, 6, size=(B, Hkv, N, 4)).astype(np.int32)
    idx[..., 1] = idx[..., 0]
    step = TrainStep(B, Hq, Hkv, N, D, block, 4, dt)
    scores = torch.tensor(s32).to(DEV)
    it = torch.tensor(idx).to(DEV)
    step.forward(q, k, v, scores, it)
    step.backward(q, k, v, do, scores, it)
    torch.cuda.synchronize()
    s64 = s32.astype(np.float64)
    o_ref, _, _ = orc.gated_attention_forward(to64(q), to64(k), to64(v), s64, idx, block, w.scale)
    max_abs(to64(step.o), o_ref, 2e-2, "o")
    dq, dk, dv, ds = orc.gated_attention_backward(to64(q), to64(k), to64(v), to64(do), s64, idx, block, w.scale)
    normwise(to64(step.dq), dq, 2e-2, "dq")
    normwise(to64(step.dk), dk, 2e-2, "dk")
    normwise(to64(step.dv), dv, 2e-2, "dv")
    normwise(to64(step.ds), ds, 2e-2, "ds")


SELECTOR_CASES = [
    # name, dtype, B, Hq, Hkv, D, N, block
    ("f32-d64", "f32", 1, 4, 2, 64, 300, 32),
    ("bf16-g4-d128", "bf16", 1, 8, 2, 128, 1536, 64),
    ("bf16-g2-d64-tail", "bf16", 2, 4, 2, 64, 1130, 64),
    ("bf16-chunks", "bf16", 1, 4, 1, 128, 2600, 32),
]


@pytest.mark.parametrize("case", SELECTOR_CASES, ids=[c[0] for c in SELECTOR_CASES])
def test_selector_backward_parity(case):
    name, dts, B, Hq, Hkv, D, N, block = case
    dt = _dt(dts)
    C = N // block
    g = torch.Generator().manual_seed(N + D)
    q = torch.randn((B, Hq, N, D), generator=g).to(dt)
    k = torch.randn((B, Hkv, N, D), generator=g).to(dt)
    ds = torch.randn((B, Hq, N, C), generator=g)
    kbar = torch.tensor(orc.pool_block_keys(to64(k), block)).to(dt)  # the pooled keys as the GPU holds them
    scale = D ** -0.5
    # oracle on the pooled keys as the GPU holds them
    dq_ref, dkbar_ref, dk_ref = orc.selector_backward(to64(q), to64(k), ds.numpy(), block, scale,
                                                      kbar=to64(kbar))
    ws = sas.workspace(sas.SAS_OP_SELECTOR_BWD, B, Hq, Hkv, N, D, block, -1,
                       sas.SAS_BF16 if dt == torch.bfloat16 else sas.SAS_F32)
    dq = torch.full((B, Hq, N, D), float("nan"), dtype=dt, device=DEV)
    dk = torch.full((B, Hkv, N, D), float("nan"), dtype=dt, device=DEV)
    dkbar = torch.empty((B, Hkv, C, D), dtype=torch.float32, device=DEV)
    qd, kbd, dsd = q.to(DEV), kbar.to(DEV), ds.to(DEV)
    sas.sas_selector_bwd(qd, kbd, dsd, dq, dk, block, scale, dkbar=dkbar, workspace=ws)
    torch.cuda.synchronize()
    tol = 1e-5 if dt == torch.float32 else 2e-2
    normwise(to64(dq), dq_ref, tol, "dq")
    normwise(to64(dkbar), dkbar_ref, tol, "dkbar")
    normwise(to64(dk), dk_ref, tol, "dk")
    assert torch.all(dk[:, :, C * block:] == 0)
    # accumulate: adds onto what dq and dk hold
    dq0 = torch.randn((B, Hq, N, D), generator=g).to(dt)
    dk0 = torch.randn((B, Hkv, N, D), generator=g).to(dt)
    dq2, dk2 = dq0.to(DEV), dk0.to(DEV)
    sas.sas_selector_bwd(qd, kbd, dsd, dq2, dk2, block, scale, accumulate=True, workspace=ws)
    torch.cuda.synchronize()
    normwise(to64(dq2), to64(dq0) + dq_ref, tol, "dq accumulate")
    normwise(to64(dk2), to64(dk0) + dk_ref, tol, "dk accumulate")


PAGED_CASES = [
    # name, Hq, Hkv, D, max_blocks, block, topk
    ("g4-k4", 8, 2, 128, 24, 64, 4),
    ("g5-d64-k3", 10, 2, 64, 20, 64, 3),
    ("block128-k2", 8, 2, 128, 10, 128, 2),
    ("k0-current-only", 4, 1, 128, 8, 64, 0),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_paged_decode_parity(case):
    name, Hq, Hkv, D, maxb, block, topk = case
    dt = torch.bfloat16
    B = 5
    L = maxb * block
    w = Workload(name, "decode", "bf16", B, Hq, Hkv, D, L, block, topk, index=11)
    q, kc, vc, _ = decode_inputs(w, device="cpu")
    # full, ragged, short, idle, over-long (counts as L: block maxb-1 is current)
    lens = torch.tensor([L, L - 37, block + 3, 0, L + 3 * block + 5], dtype=torch.int32)
    G = Hq // Hkv
    # pages in a shuffled pool with spare pages: block m of sequence b -> page table[b, m]
    n_pages = B * maxb + 5
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(7))
    table = perm[: B * maxb].reshape(B, maxb).to(torch.int32)
    kp = torch.zeros((n_pages, Hkv, block, D), dtype=dt)
    vp = torch.zeros((n_pages, Hkv, block, D), dtype=dt)
    for b in range(B):
        for m in range(maxb):
            kp[table[b, m]] = kc[b, :, m * block:(m + 1) * block]
            vp[table[b, m]] = vc[b, :, m * block:(m + 1) * block]
    kpd, vpd, tbd = kp.to(DEV), vp.to(DEV), table.to(DEV)
    kbp = torch.zeros((n_pages, Hkv, D), dtype=dt, device=DEV)
    sas.sas_pool_pages(kpd, kbp, table.reshape(-1).contiguous().to(DEV), block)
    torch.cuda.synchronize()
    kbar = orc.pool_block_keys(to64(kc), block)  # [B, Hkv, C, D]
    kbar_r = to64(torch.tensor(kbar).to(dt))
    kbar_close(to64(kbp[table.long()].permute(0, 2, 1, 3)), kbar_r)
    # the oracle's pooled keys feed the GPU scores, so both rank the same numbers
    kbp_r = torch.zeros((n_pages, Hkv, D), dtype=dt)
    for b in range(B):
        for m in range(maxb):
            kbp_r[table[b, m]] = torch.tensor(kbar_r[b, :, m]).to(dt)
    o = torch.empty((B, Hq, D), dtype=dt, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Hkv, max(topk, 1)), dtype=torch.int32, device=DEV)
    ws = sas.workspace(sas.SAS_OP_PAGED_DECODE, B, Hq, Hkv, L, D, block, topk, sas.SAS_BF16)
    scale = w.scale
    sas.sas_paged_decode(q.to(DEV), kpd, vpd, kbp_r.to(DEV), tbd, lens.to(DEV), topk, o, lse, block, scale,
                         idx_out=idx if topk > 0 else None, workspace=ws)
    torch.cuda.synchronize()
    u_ref = orc.decode_scores(to64(q), kbar_r, lens.numpy(), L, block, scale, True)
    c = orc.decode_candidates(lens.numpy(), L, block)
    # The workspace starts with the group-summed scores the selection was made
    # on: they match the oracle's, and Top-K on them is bit-exact.
    u_gpu = ws[: B * Hkv * maxb * 4].view(torch.float32).reshape(B, Hkv, maxb).cpu().numpy()
    normwise(u_gpu.astype(np.float64), u_ref.astype(np.float64), 1e-5, "u")
    assert np.array_equal(np.isneginf(u_gpu), np.isneginf(u_ref))
    idx_ref = np.zeros((B, Hkv, 0), dtype=np.int64)  # topk 0: the current block only
    active = lens.numpy() > 0
    if topk > 0:
        idx_ref = orc.topk_select(u_gpu[:, :, None, :], 1, c[:, None], topk)[:, :, 0, :]
        got = idx.cpu().numpy()
        assert np.array_equal(got, idx_ref), "paged Top-K"
        # history blocks only, also for the over-long sequence
        assert np.all((got == -1) | ((got >= 0) & (got < c[:, None, None])))
    o_ref, lse_ref = orc.sparse_decode(to64(q), to64(kc), to64(vc), lens.numpy(), idx_ref, block, scale)
    max_abs(to64(o)[active], o_ref[active], 2e-2, "o")
    normwise(to64(lse)[active], lse_ref[active], 1e-4, "lse")
    idle = lens.numpy() <= 0
    assert torch.all(o[torch.tensor(idle)] == 0)


GATE_CASES = [
    # name, dtype, B, Hq, Hkv, D, N, block, topk
    ("f32-full", "f32", 1, 2, 1, 64, 320, 64, None),
    ("f32-ragged-sparse", "f32", 2, 4, 2, 64, 300, 64, 2),
    ("bf16-full", "bf16", 1, 8, 2, 128, 384, 64, None),
    ("bf16-ragged-sparse", "bf16", 1, 8, 2, 128, 450, 64, 3),
]


@pytest.mark.parametrize("gate", ["sigmoid", "raw", "outer"])
@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_gate_variant_parity(case, gate):
    """Sigmoid and raw-logit gates (the pages' gate-activation ablation) and the
    outer gate (gate placement) through sas_gated_attn_fwd_gate / _bwd_gate
    against the oracle at the same tolerances as the softmax gate.  The
    sigmoid and raw gates write lse_s = 0 and their backward takes no lse_s;
    the outer gate's lse_s is the softmax gate's."""
    name, dts, B, Hq, Hkv, D, N, block, topk = case
    dt = _dt(dts)
    w = Workload(name, "train", dts, B, Hq, Hkv, D, N, block, topk, index=11)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    scale = w.scale
    G = Hq // Hkv
    C = N // block
    tol = tolerances(dt)
    _, _, s32, idx = _oracle_selector(q, k, block, scale, topk, G)
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
    torch.cuda.synchronize()
    s64 = s32.astype(np.float64)
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(to64(q), to64(k), to64(v), s64, idx, block, scale,
                                                           gate=gate)
    if tol["o_abs"] is not None:
        max_abs(to64(o), o_ref, tol["o_abs"], "o")
    else:
        normwise(to64(o), o_ref, tol["o_rel"], "o")
    normwise(to64(lse), lse_ref, tol["lse"], "lse")
    if gate == "outer":
        normwise(to64(lse_s), lses_ref, tol["lse"], "lse_s")
    else:
        assert torch.count_nonzero(lse_s).item() == 0, "lse_s"

    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty((B, Hq, N, C), dtype=torch.float32, device=DEV)
    wsb = sas.workspace(sas.SAS_OP_BWD_GATE, B, Hq, Hkv, N, D, block, tk, sdt, DEV)
    sas.sas_gated_attn_bwd_gate(q, k, v, o, do, scores, idx_t, lse, lse_s if gate == "outer" else None, dq, dk,
                                dv, ds, block, scale, g, wsb)
    torch.cuda.synchronize()
    r_dq, r_dk, r_dv, r_ds = orc.gated_attention_backward(to64(q), to64(k), to64(v), to64(do), s64, idx,
                                                          block, scale, gate=gate)
    normwise(to64(dq), r_dq, tol["grad"], "dq")
    normwise(to64(dk), r_dk, tol["grad"], "dk")
    normwise(to64(dv), r_dv, tol["grad"], "dv")
    normwise(to64(ds), r_ds, tol["ds"], "ds")
    if idx is not None and gate != "outer":  # no normaliser: unselected history blocks get exactly 0
        sel = np.zeros((B, Hq, N, C), dtype=bool)
        for b in range(B):
            for h in range(Hq):
                for t in range(N):
                    for m in idx[b, h // G, t]:
                        if 0 <= m < t // block:
                            sel[b, h, t, m] = True
        assert torch.count_nonzero(ds.cpu()[torch.tensor(~sel)]).item() == 0, "ds outside the selection"


@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_ste_gate_parity(case):
    """The hard gate with a straight-through estimator (SAS_GATE_STE) against
    the oracle's reading: o and lse of plain block-sparse attention, lse_s =
    LSE(s), the sparse dq, dk, dv, and ds over every history block."""
    name, dts, B, Hq, Hkv, D, N, block, topk = case
    dt = _dt(dts)
    w = Workload(name, "train", dts, B, Hq, Hkv, D, N, block, topk, index=13)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    scale = w.scale
    G = Hq // Hkv
    C = N // block
    tol = tolerances(dt)
    _, _, s32, idx = _oracle_selector(q, k, block, scale, topk, G)
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
    r = orc.ste_gate_attention(to64(q), to64(k), to64(v), to64(do), s32.astype(np.float64), idx, block, scale)
    o_ref, lse_ref, lses_ref, dq_r, dk_r, dv_r, ds_r = r
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


def test_full_star_by_composition():
    """full* (the pages' full-scope simulation: noise added before Top-K) from
    the existing calls: the caller adds its own noise to the scores given to
    sas_topk_select and passes the clean scores to the attention.  The pages
    give no noise distribution; seeded N(0, 1) noise stands in."""
    B, Hq, Hkv, D, N, block, topk = 1, 8, 2, 128, 450, 64, 3
    w = Workload("full-star", "train", "bf16", B, Hq, Hkv, D, N, block, topk, index=17)
    q, k, v, do = (x.to(DEV) for x in training_inputs(w, device="cpu"))
    G = Hq // Hkv
    tol = tolerances(torch.bfloat16)
    _, _, s32, _ = _oracle_selector(q, k, block, w.scale, None, G)
    noise = torch.randn(s32.shape, generator=torch.Generator().manual_seed(5)).numpy().astype(np.float32)
    noisy = (s32 + noise).astype(np.float32)
    pos = np.broadcast_to(np.arange(N), (B, N)) // block
    idx = orc.topk_select(noisy, G, pos, topk)
    step = TrainStep(B, Hq, Hkv, N, D, block, topk, torch.bfloat16)
    sas.sas_topk_select(torch.tensor(noisy).to(DEV), step.idx, None, G, block)
    torch.cuda.synchronize()
    assert np.array_equal(step.idx.cpu().numpy(), idx), "topk of the noisy scores"
    scores = torch.tensor(s32).to(DEV)
    step.forward(q, k, v, scores, step.idx)
    step.backward(q, k, v, do, scores, step.idx)
    torch.cuda.synchronize()
    s64 = s32.astype(np.float64)
    o_ref, _, _ = orc.gated_attention_forward(to64(q), to64(k), to64(v), s64, idx, block, w.scale)
    max_abs(to64(step.o), o_ref, tol["o_abs"], "o")
    dq, dk, dv, ds = orc.gated_attention_backward(to64(q), to64(k), to64(v), to64(do), s64, idx, block, w.scale)
    normwise(to64(step.ds), ds, tol["ds"], "ds")
    normwise(to64(step.dq), dq, tol["grad"], "dq")


DECODE_STEP_CASES = [
    # name, dtype, Hq, Hkv, D, L, block, topk
    ("bf16-g4-k4", "bf16", 8, 2, 128, 2048, 64, 4),
    ("bf16-g5-k3-ragged-cap", "bf16", 10, 2, 128, 1500, 64, 3),
    ("bf16-block32-k5", "bf16", 4, 2, 128, 1000, 32, 5),
    ("bf16-g16-d64-k9", "bf16", 16, 1, 64, 1280, 64, 9),
    ("bf16-k0", "bf16", 8, 2, 128, 1024, 64, 0),
    ("bf16-k64", "bf16", 8, 2, 128, 64 * 700, 64, 64),
    ("bf16-k40-ties", "bf16", 4, 1, 128, 64 * 300, 64, 40),
    ("bf16-k100", "bf16", 8, 2, 128, 64 * 300, 64, 100),
    ("f32-k3", "f32", 4, 1, 64, 1024, 64, 3),
    ("bf16-block128", "bf16", 8, 2, 128, 2048, 128, 3),
]


@pytest.mark.parametrize("case", DECODE_STEP_CASES, ids=[c[0] for c in DECODE_STEP_CASES])
def test_decode_step_parity(case):
    """sas_decode_step: the scores it leaves in the workspace match the oracle's;
    its selection is the oracle's Top-K on those very scores (bit-exact); o and
    lse match the oracle's sparse decode over that selection."""
    name, dts, Hq, Hkv, D, L, block, topk = case
    dt = _dt(dts)
    B = 5
    w = Workload(name, "decode", dts, B, Hq, Hkv, D, L, block, topk, index=12)
    q, kc, vc, _ = decode_inputs(w, device="cpu")
    if "ties" in name:  # many equal pooled keys: equal scores, ties to the lower block
        kc[:, :, : 64 * 200] = kc[:, :, :64].repeat(1, 1, 200, 1)
    lens = torch.tensor([L, L - 37, 40, 0, 10 * L + 3], dtype=torch.int32)
    kbar_r = to64(torch.tensor(orc.pool_block_keys(to64(kc), block)).to(dt))
    C = L // block
    o = torch.full((B, Hq, D), float("nan"), dtype=dt, device=DEV)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((B, Hkv, max(topk, 1)), -7, dtype=torch.int32, device=DEV)
    ws = sas.workspace(sas.SAS_OP_DECODE_STEP, B, Hq, Hkv, L, D, block, topk,
                       sas.SAS_BF16 if dt == torch.bfloat16 else sas.SAS_F32)
    qd, kcd, vcd, lensd = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    kbd = torch.tensor(kbar_r).to(dt).to(DEV)
    sas.sas_decode_step(qd, kbd, kcd, vcd, lensd, topk, o, lse, block, w.scale,
                        idx_out=idx[..., :topk] if topk > 0 else None, workspace=ws)
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
    assert torch.all(lse[~torch.tensor(active)] == float("-inf"))
    # again, without idx_out and on the dirty workspace: the same bits
    o2 = torch.full_like(o, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    sas.sas_decode_step(qd, kbd, kcd, vcd, lensd, topk, o2, lse2, block, w.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse)


PREFILL_CASES = [
    # name, dtype, Hq, Hkv, D, N, block, max_blocks, seq_len, topk
    ("bf16-g4", "bf16", 8, 2, 128, 640, 64, 14, [640, 600, 130], 3),
    ("bf16-g5-d64", "bf16", 10, 2, 64, 320, 64, 6, [320, 64, 63], 2),
    ("f32-block32", "f32", 4, 1, 64, 200, 32, 8, [200, 33, 1], 2),
    # longer prompts: 47 tiles of the full-scope kernel on the shared zero score row
    ("bf16-g4-long", "bf16", 8, 2, 128, 3000, 64, 48, [3000, 2417, 64], 8),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_then_paged_decode(case):
    """Dense prefill of ragged prompts into a shuffled page pool, then decode
    from those pages: the prefill's o and lse against the oracle's causal
    attention (valid rows), the pages and their pooled keys against the prompt
    and the oracle's pooling, then one decode step of a new token (its K and V
    appended to its page the way a caller does, its page pooled when that
    completes a block) through sas_paged_decode, checked as in the paged test."""
    name, dts, Hq, Hkv, D, N, block, maxb, lens_l, topk = case
    dt = _dt(dts)
    B = len(lens_l)
    w = Workload(name, "train", dts, B, Hq, Hkv, D, N, block, None, index=13)
    q, k, v, _ = training_inputs(w, device="cpu")
    seq = torch.tensor(lens_l, dtype=torch.int32)
    n_pages = B * maxb + 3
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(9))
    table = perm[: B * maxb].reshape(B, maxb).to(torch.int32)
    kp = torch.zeros((n_pages, Hkv, block, D), dtype=dt, device=DEV)
    vp = torch.zeros_like(kp)
    kbp = torch.zeros((n_pages, Hkv, D), dtype=dt, device=DEV)
    o = torch.full((B, Hq, N, D), float("nan"), dtype=dt, device=DEV)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=DEV)
    sdt = sas.SAS_BF16 if dt == torch.bfloat16 else sas.SAS_F32
    ws = sas.workspace(sas.SAS_OP_PREFILL, B, Hq, Hkv, N, D, block, 0, sdt)
    tbd = table.to(DEV)
    sas.sas_prefill_paged(q.to(DEV), k.to(DEV), v.to(DEV), seq.to(DEV), o, lse, kp, vp, kbp, tbd, block, w.scale, ws)
    torch.cuda.synchronize()
    tol = tolerances(dt)
    for b in range(B):
        n = lens_l[b]
        o_ref, lse_ref = orc.causal_attention(to64(q[b:b + 1, :, :n]), to64(k[b:b + 1, :, :n]),
                                              to64(v[b:b + 1, :, :n]), w.scale)
        if tol["o_abs"] is not None:
            max_abs(to64(o[b:b + 1, :, :n]), o_ref, tol["o_abs"], "prefill o")
        else:
            normwise(to64(o[b:b + 1, :, :n]), o_ref, tol["o_rel"], "prefill o")
        normwise(to64(lse[b:b + 1, :, :n]), lse_ref, 1e-4, "prefill lse")
        assert torch.isfinite(o[b]).all()
        # pages hold the prompt's rows exactly; complete blocks hold their pooled keys
        kpc, vpc = kp.cpu(), vp.cpu()
        for m in range((n + block - 1) // block):
            rows = min(block, n - m * block)
            pg = int(table[b, m])
            assert torch.equal(kpc[pg, :, :rows], k[b, :, m * block:m * block + rows])
            assert torch.equal(vpc[pg, :, :rows], v[b, :, m * block:m * block + rows])
        nfull = n // block
        if nfull:
            kbar_ref = to64(torch.tensor(orc.pool_block_keys(to64(k[b:b + 1, :, : nfull * block]), block)).to(dt))
            got = to64(kbp[table[b, :nfull].long()].permute(1, 0, 2))[None]
            kbar_close(got, kbar_ref)
    if dt != torch.bfloat16:
        return  # the paged decode is bf16 only
    # One decode step: a new token per sequence at position seq_len[b].
    gen = torch.Generator().manual_seed(77)
    qn = torch.randn((B, Hq, D), generator=gen).to(dt)
    kn = torch.randn((B, Hkv, D), generator=gen).to(dt)
    vn = torch.randn((B, Hkv, D), generator=gen).to(dt)
    kc = torch.zeros((B, Hkv, maxb * block, D), dtype=dt)
    vc = torch.zeros_like(kc)
    for b in range(B):
        n = lens_l[b]
        kc[b, :, :n], vc[b, :, :n] = k[b, :, :n], v[b, :, :n]
        kc[b, :, n], vc[b, :, n] = kn[b], vn[b]
        pg = int(table[b, n // block])
        kp[pg, :, n % block] = kn[b].to(DEV)  # the caller appends the new token to its page
        vp[pg, :, n % block] = vn[b].to(DEV)
        if (n + 1) % block == 0:  # the append completes a block: pool that page
            sas.sas_pool_pages(kp, kbp, torch.tensor([pg], dtype=torch.int32, device=DEV), block)
    lens = seq + 1
    L = maxb * block
    od = torch.empty((B, Hq, D), dtype=dt, device=DEV)
    lsed = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=DEV)
    wsd = sas.workspace(sas.SAS_OP_PAGED_DECODE, B, Hq, Hkv, L, D, block, topk, sas.SAS_BF16)
    sas.sas_paged_decode(qn.to(DEV), kp, vp, kbp, tbd, lens.to(DEV), topk, od, lsed, block, w.scale, idx_out=idx,
                         workspace=wsd)
    torch.cuda.synchronize()
    C = maxb
    kbar_r = np.zeros((B, Hkv, C, D))
    for b in range(B):
        nfull = (lens_l[b] + 1) // block
        if nfull:
            kbar_r[b, :, :nfull] = to64(torch.tensor(orc.pool_block_keys(to64(kc[b:b + 1, :, : nfull * block]),
                                                                         block)).to(dt))[0]
    u_ref = orc.decode_scores(to64(qn), kbar_r, lens.numpy(), L, block, w.scale, True)
    u_gpu = wsd[: B * Hkv * C * 4].view(torch.float32).reshape(B, Hkv, C).cpu().numpy()
    normwise(u_gpu.astype(np.float64), u_ref.astype(np.float64), 1e-5, "u")
    c = orc.decode_candidates(lens.numpy(), L, block)
    idx_ref = orc.topk_select(u_gpu[:, :, None, :], 1, c[:, None], topk)[:, :, 0, :]
    assert np.array_equal(idx.cpu().numpy(), idx_ref), "Top-K on the decode's own scores"
    o_ref, lse_ref = orc.sparse_decode(to64(qn), to64(kc), to64(vc), lens.numpy(), idx_ref, block, w.scale)
    max_abs(to64(od), o_ref, 2e-2, "decode o")
    normwise(to64(lsed), lse_ref, 1e-4, "decode lse")
