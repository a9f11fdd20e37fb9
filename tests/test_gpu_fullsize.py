"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

The oracle computes sampled outputs one by one (rows for o, lse, lse_s, dq, ds;
keys for dk, dv), plus whole-tensor checks where it is cheap (pooled keys,
Top-K, decode).  Selector scores and Top-K indices fed to the attention calls
are the oracle's, so every entry point sees identical inputs; the all-GPU
chain is checked separately, where only near-tie flips of the Top-K may differ.
"""
import numpy as np
import pytest
import torch

from oracle import sas_oracle as orc
from tests.gpu_util import kbar_close, max_abs, normwise, to64
from trainable_block_sparse_sas_amd.inputs import WORKLOADS, Workload, decode_inputs, training_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if torch.cuda.is_available():
    from trainable_block_sparse_sas_amd import binding as sas
    from trainable_block_sparse_sas_amd.pipeline import DecodeStep, TrainStep

DEV = "cuda"


def _oracle_scores_f32(q64, kbar_r, block, scale):
    """Oracle scores for every row, one head at a time, stored as fp32."""
    B, Hq, N, D = q64.shape
    C = kbar_r.shape[2]
    out = np.empty((B, Hq, N, C), dtype=np.float32)
    pos = np.broadcast_to(np.arange(N), (1, N))
    G = Hq // kbar_r.shape[1]
    for b in range(B):
        for h in range(Hq):
            out[b, h] = orc.block_scores(q64[b:b + 1, h:h + 1], kbar_r[b:b + 1, h // G:h // G + 1], block, scale,
                                         pos)[0, 0].astype(np.float32)
    return out


def _sample_rows(N, block, n=24, seed=0):
    r = np.random.default_rng(seed)
    fixed = [0, 1, block - 1, block, block + 5, N // 2, N - block - 1, N - 2, N - 1]
    return np.unique(np.concatenate([fixed, r.integers(0, N, size=n)]))


def _rowwise(got, ref, tol, what):
    """Each row on its own: max|got - ref| <= tol * max|ref| over that row, so a
    small-norm row (a long softmax average) is held to its own scale."""
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    err = np.max(np.abs(got - ref), axis=1)
    scale = np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    bad = err > tol * scale
    assert not bad.any(), f"{what}: {bad.sum()} rows off, worst {np.max(err / scale):.3e}"


def _ds_invariants(step, scores, idx, G, w):
    """Invariants of the gate gradient on the GPU's own outputs, over every row
    of every head ([Blog] 方法核心, Fig. 4 and the inner-gate gradient; [Review]
    "Why the Four Design Choices Matter", Eq. 5): ds = dbeta - g sum(dbeta)
    with sum(g) = 1 gives sum_m ds = 0 over the history; at sparse scope an
    unselected block has dbeta = 0, so ds/g is one value per row there."""
    ds = step.ds[0]  # [Hq, N, C] fp32 on the GPU
    C, N = w.C, w.N
    hist = (torch.arange(C, device=DEV)[None, :] < (torch.arange(N, device=DEV) // w.block)[:, None])
    for h in range(w.Hq):
        d = ds[h]
        assert torch.all(d[~hist] == 0), f"ds outside the history, head {h}"
        tot = d.sum(dim=1, dtype=torch.float64)
        mag = d.abs().sum(dim=1, dtype=torch.float64)
        bad = tot.abs() > 1e-4 * mag + 1e-30
        assert not bool(bad.any()), f"sum_m ds != 0 on {int(bad.sum())} rows of head {h}"
    if idx is None:
        return
    rows = _sample_rows(N, w.block, n=400, seed=11)
    rows = rows[rows // w.block >= w.topk + 2]  # rows with unselected history
    s = scores[0][:, rows].double().cpu().numpy()
    lse_s = step.lse_s[0][:, rows].double().cpu().numpy()
    dsr = ds[:, rows].double().cpu().numpy()
    for h in range(w.Hq):
        for i, t in enumerate(rows):
            c = t // w.block
            uns = np.setdiff1d(np.arange(c), idx[0, h // G, t])
            g = np.exp(s[h, i, uns] - lse_s[h, i])
            keep = g > 1e-30
            r = dsr[h, i, uns][keep] / g[keep]
            assert np.max(np.abs(r - r.mean())) <= 1e-4 * max(abs(r.mean()), 1e-30) + 1e-12, (h, t)


@pytest.mark.parametrize("wi", [1, 2], ids=["train-8k-full", "train-32k-sparse"])
def test_training_fullsize(wi):
    w = WORKLOADS[wi]
    dt = w.torch_dtype
    q, k, v, do = training_inputs(w, device=DEV)
    q64, k64 = to64(q), to64(k)
    G = w.Hq // w.Hkv
    # Pooled keys: GPU vs oracle (at most one bf16 step apart).
    step = TrainStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk, dt)
    step.select(q, k)
    torch.cuda.synchronize()
    kbar = orc.pool_block_keys(k64, w.block)
    kbar_r = to64(torch.tensor(kbar).to(dt))
    kbar_close(to64(step.kbar), kbar_r)
    gpu_chain_idx = None if w.topk is None else step.idx.cpu().numpy()
    s32 = _oracle_scores_f32(q64, kbar_r, w.block, w.scale)
    rows = _sample_rows(w.N, w.block)
    if step.gates is not None:  # the gated Top-K of the step's selection
        _check_gates(step, rows, G)
    # GPU scores from the oracle's pooled keys, sampled rows.
    kbar_dev = torch.tensor(kbar_r).to(dt).to(DEV)
    sas.sas_score_blocks(q, None, kbar_dev, step.scores, None, w.block, w.scale)
    # the same scores through the score kernel that also writes LSE_s
    s_lse = torch.full_like(step.scores, float("-inf"))  # it writes the history columns only
    lse_s_sc = torch.empty_like(step.lse_s)
    sas.sas_score_blocks_lse(q, None, kbar_dev, s_lse, lse_s_sc, w.block, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(s_lse[:, :, rows], step.scores[:, :, rows]), "scores (score kernel with LSE_s)"
    del s_lse
    normwise(to64(step.scores[:, :, rows]), s32[:, :, rows].astype(np.float64), 1e-5, "scores")
    scores = torch.tensor(s32).to(DEV)
    idx = None
    g_chk = w.Hkv - 1
    if w.topk is not None:
        sas.sas_topk_select(scores, step.idx, None, G, w.block)
        torch.cuda.synchronize()
        gidx = step.idx.cpu().numpy()
        pos = np.arange(w.N)[None, :] // w.block
        ref_g = orc.topk_select(s32[:, g_chk * G:(g_chk + 1) * G], G, pos, w.topk)
        assert np.array_equal(gidx[:, g_chk:g_chk + 1], ref_g), "topk (one KV head, every row)"
        ref_rows = orc.topk_select(s32[:, :, rows], G, pos[:, rows], w.topk)
        assert np.array_equal(gidx[:, :, rows], ref_rows), "topk (sampled rows, every KV head)"
        idx = gidx
        # The all-GPU chain (GPU pooled keys and scores): rows may differ only at near-ties.
        diff = np.any(gpu_chain_idx != gidx, axis=-1)
        assert diff.mean() < 1e-3, f"chain Top-K differs on {diff.mean():.2%} of rows"
    idx_t = None if idx is None else torch.tensor(idx).to(DEV)
    step.forward(q, k, v, scores, idx_t)
    step.backward(q, k, v, do, scores, idx_t)
    torch.cuda.synchronize()
    v64, do64, s64 = to64(v), to64(do), s32.astype(np.float64)
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(q64, k64, v64, s64, idx, w.block, w.scale, rows=rows)
    max_abs(to64(step.o[:, :, rows]), o_ref, 2e-2, "o")
    _rowwise(to64(step.o[:, :, rows]), o_ref, 2e-2, "o per row")
    normwise(to64(step.lse[:, :, rows]), lse_ref, 1e-4, "lse")
    normwise(to64(step.lse_s[:, :, rows]), lses_ref, 1e-4, "lse_s")
    normwise(to64(lse_s_sc[:, :, rows]), lses_ref, 1e-4, "lse_s (score kernel)")
    _ds_invariants(step, scores, idx, G, w)
    for h in (0, w.Hq // 2 + 1, w.Hq - 1):
        dq_r, ds_r = orc.row_gradients(q64, k64, v64, do64, s64, idx, w.block, w.scale, 0, h, rows)
        normwise(to64(step.dq[0, h, rows]), dq_r, 2e-2, f"dq h{h}")
        normwise(to64(step.ds[0, h, rows]), ds_r, 2e-2, f"ds h{h}")
    if idx is None:
        keys = np.array([0, 1, w.block - 1, w.block, w.N // 2 + 3, w.N - w.block, w.N - 1])
        attend = None
    else:
        # late blocks (few selecting rows keep the oracle quick) plus the last block
        C = w.C
        keys = np.array([(C - 90) * w.block + 3, (C - 7) * w.block, (C - 2) * w.block + 63, w.N - 1])
        kb = np.unique(keys // w.block)
        tsel = np.any(np.isin(idx[0, g_chk], kb), axis=-1)  # tokens selecting one of the blocks
        own = np.isin(np.arange(w.N) // w.block, kb)
        attend = np.nonzero(tsel | own)[0]
    dk_r, dv_r = orc.key_gradients(q64, k64, v64, do64, s64, idx, w.block, w.scale, 0, g_chk, keys,
                                   rows=attend)
    normwise(to64(step.dk[0, g_chk, keys]), dk_r, 2e-2, "dk")
    normwise(to64(step.dv[0, g_chk, keys]), dv_r, 2e-2, "dv")


def _check_gates(step, rows, G):
    """The log gates sas_topk_select_gated wrote beside the step's selection, on
    sampled rows: slot j holds (s - LSE_s) log2 e of the j-th smallest selected
    block for every head of the group, bit for bit as fp32 evaluates it from
    the step's own scores and LSE_s."""
    idx = step.idx[:, :, rows].cpu()
    big = torch.iinfo(torch.int32).max
    srt, _ = torch.sort(torch.where(idx >= 0, idx, torch.full_like(idx, big)), dim=-1)
    valid = srt != big
    m = torch.where(valid, srt, torch.zeros_like(srt)).long()
    B, Hkv, R, K = idx.shape
    C = step.scores.shape[-1]
    s = step.scores[:, :, rows].cpu().reshape(B, Hkv, G, R, C)
    lse_s = step.lse_s[:, :, rows].cpu().reshape(B, Hkv, G, R)
    sel = torch.gather(s, 4, m[:, :, None].expand(B, Hkv, G, R, K))
    log2e = torch.tensor(1.4426950408889634, dtype=torch.float32)
    want = ((sel - lse_s[..., None]) * log2e).permute(0, 1, 3, 4, 2)
    got = step.gates[:, :, rows].cpu()
    assert torch.equal(got[valid], want[valid]), "log gates of the gated Top-K"


@pytest.mark.parametrize("gate", ["sigmoid", "raw", "outer"])
def test_gate_variant_fullsize(gate):
    """The sigmoid, raw-logit and outer gates at the 32K sparse training shape, through
    sas_gated_attn_fwd_gate / _bwd_gate on the oracle's scores and selection:
    sampled rows of o, lse, dq and ds, and sampled keys of dk and dv."""
    w = WORKLOADS[2]
    dt = w.torch_dtype
    q, k, v, do = training_inputs(w, device=DEV)
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(do)
    G = w.Hq // w.Hkv
    kbar_r = to64(torch.tensor(orc.pool_block_keys(k64, w.block)).to(dt))
    s32 = _oracle_scores_f32(q64, kbar_r, w.block, w.scale)
    pos = np.arange(w.N)[None, :] // w.block
    rows = _sample_rows(w.N, w.block, seed=3)
    scores = torch.tensor(s32).to(DEV)
    # the selection: the GPU Top-K on the oracle's scores, bit-exact on the sampled rows
    idx_t = torch.empty((w.B, w.Hkv, w.N, w.topk), dtype=torch.int32, device=DEV)
    sas.sas_topk_select(scores, idx_t, None, G, w.block)
    torch.cuda.synchronize()
    idx = idx_t.cpu().numpy()
    assert np.array_equal(idx[:, :, rows], orc.topk_select(s32[:, :, rows], G, pos[:, rows], w.topk)), "topk"
    g = {"sigmoid": sas.SAS_GATE_SIGMOID, "raw": sas.SAS_GATE_RAW, "outer": sas.SAS_GATE_OUTER}[gate]
    B, Hq, Hkv, N, D, C = w.B, w.Hq, w.Hkv, w.N, w.D, w.C
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    lse_s = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    wsf = sas.workspace(sas.SAS_OP_FWD_GATE, B, Hq, Hkv, N, D, w.block, w.topk, sas.SAS_BF16, DEV)
    sas.sas_gated_attn_fwd_gate(q, k, v, scores, idx_t, o, lse, lse_s, w.block, w.scale, g, wsf)
    torch.cuda.synchronize()
    del wsf
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty((B, Hq, N, C), dtype=torch.float32, device=DEV)
    wsb = sas.workspace(sas.SAS_OP_BWD_GATE, B, Hq, Hkv, N, D, w.block, w.topk, sas.SAS_BF16, DEV)
    sas.sas_gated_attn_bwd_gate(q, k, v, o, do, scores, idx_t, lse, lse_s if gate == "outer" else None, dq, dk,
                                dv, ds, w.block, w.scale, g, wsb)
    torch.cuda.synchronize()
    del wsb
    s64 = s32.astype(np.float64)
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(q64, k64, v64, s64, idx, w.block, w.scale, rows=rows,
                                                           gate=gate)
    max_abs(to64(o[:, :, rows]), o_ref, 2e-2, "o")
    normwise(to64(lse[:, :, rows]), lse_ref, 1e-4, "lse")
    if gate == "outer":
        normwise(to64(lse_s[:, :, rows]), lses_ref, 1e-4, "lse_s")
    else:
        assert torch.count_nonzero(lse_s).item() == 0, "lse_s"
    for h in (1, Hq - 2):
        dq_r, ds_r = orc.row_gradients(q64, k64, v64, do64, s64, idx, w.block, w.scale, 0, h, rows, gate=gate)
        normwise(to64(dq[0, h, rows]), dq_r, 2e-2, f"dq h{h}")
        normwise(to64(ds[0, h, rows]), ds_r, 2e-2, f"ds h{h}")
    g_chk = 1
    keys = np.array([(C - 60) * w.block + 5, (C - 3) * w.block + 40, N - 1])
    kb = np.unique(keys // w.block)
    attend = np.nonzero(np.any(np.isin(idx[0, g_chk], kb), axis=-1) | np.isin(np.arange(N) // w.block, kb))[0]
    dk_r, dv_r = orc.key_gradients(q64, k64, v64, do64, s64, idx, w.block, w.scale, 0, g_chk, keys, rows=attend,
                                   gate=gate)
    normwise(to64(dk[0, g_chk, keys]), dk_r, 2e-2, "dk")
    normwise(to64(dv[0, g_chk, keys]), dv_r, 2e-2, "dv")


def test_selector_bwd_fullsize():
    """The selector backward at the 32K training shape, on a seeded ds of the
    same shape as the attention backward's output."""
    w = WORKLOADS[2]
    dt = w.torch_dtype
    q, k, _, _ = training_inputs(w, device="cpu")
    C, G = w.C, w.Hq // w.Hkv
    ds = torch.randn((w.B, w.Hq, w.N, C), generator=torch.Generator().manual_seed(4242))
    kbar_r = to64(torch.tensor(orc.pool_block_keys(to64(k), w.block)).to(dt))
    qd, dsd = q.to(DEV), ds.to(DEV)
    kbd = torch.tensor(kbar_r).to(dt).to(DEV)
    dq = torch.empty((w.B, w.Hq, w.N, w.D), dtype=dt, device=DEV)
    dk = torch.empty((w.B, w.Hkv, w.N, w.D), dtype=dt, device=DEV)
    dkbar = torch.empty((w.B, w.Hkv, C, w.D), dtype=torch.float32, device=DEV)
    ws = sas.workspace(sas.SAS_OP_SELECTOR_BWD, w.B, w.Hq, w.Hkv, w.N, w.D, w.block, -1, sas.SAS_BF16)
    sas.sas_selector_bwd(qd, kbd, dsd, dq, dk, w.block, w.scale, dkbar=dkbar, workspace=ws)
    torch.cuda.synchronize()
    rows = _sample_rows(w.N, w.block)
    for h in (0, w.Hq // 2 + 1, w.Hq - 1):
        ref = orc.selector_dq_rows(kbar_r, ds.numpy(), w.block, w.scale, 0, h, rows)
        normwise(to64(dq[0, h, rows]), ref, 2e-2, f"dq h{h}")
    blocks = np.array([0, 1, C // 2, C - 2, C - 1])
    for g in (0, w.Hkv - 1):
        ref = orc.selector_dkbar_blocks(to64(q), ds.numpy(), w.block,
                                        w.scale, 0, g, G, blocks)
        normwise(to64(dkbar[0, g, blocks]), ref, 2e-2, f"dkbar g{g}")
        toks = np.concatenate([np.arange(m * w.block, (m + 1) * w.block) for m in blocks])
        normwise(to64(dk[0, g, toks]), np.repeat(ref / w.block, w.block, axis=0), 2e-2, f"dk g{g}")


@pytest.mark.parametrize("wi", [3, 4], ids=["decode-128k-b8", "decode-512k-b1"])
def test_decode_fullsize(wi):
    w = WORKLOADS[wi]
    dt = w.torch_dtype
    q, kc, vc, lens = decode_inputs(w, device=DEV)
    G = w.Hq // w.Hkv
    step = DecodeStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk, dt)
    step.pool(kc)
    step.select(q, lens)  # the all-GPU chain
    step.attend(q, kc, vc, lens)
    torch.cuda.synchronize()
    chain_idx = step.idx.cpu().numpy()
    chain_o = to64(step.o)
    q64 = to64(q)
    lens_np = lens.cpu().numpy()
    # Oracle pooled keys, one (sequence, KV head) at a time.
    kbar = np.empty((w.B, w.Hkv, w.C, w.D))
    for b in range(w.B):
        for g in range(w.Hkv):
            kbar[b, g] = orc.pool_block_keys(to64(kc[b:b + 1, g:g + 1]), w.block)[0, 0]
    kbar_r = to64(torch.tensor(kbar).to(dt))
    kbar_close(to64(step.kbar), kbar_r)
    u_ref = orc.decode_scores(q64, kbar_r, lens_np, w.N, w.block, w.scale, True)
    sas.sas_score_blocks(q, None, torch.tensor(kbar_r).to(dt).to(DEV), step.u, lens, w.block, w.scale,
                         group_sum=True, L=w.N)
    torch.cuda.synchronize()
    normwise(to64(step.u), u_ref.astype(np.float64), 1e-5, "u")
    c = (lens_np - 1) // w.block
    idx_ref = orc.topk_select(u_ref[:, :, None, :], 1, c[:, None], w.topk)[:, :, 0, :]
    sas.sas_topk_select(torch.tensor(u_ref).to(DEV), step.idx, lens, 1, w.block)
    torch.cuda.synchronize()
    assert np.array_equal(step.idx.cpu().numpy(), idx_ref), "topk"
    # Selection is non-trivial: the shifted blocks dominate the top of the ranking.
    assert len(np.unique(idx_ref)) > w.topk
    step.attend(q, kc, vc, lens, torch.tensor(idx_ref).to(DEV))
    torch.cuda.synchronize()
    kc64, vc64 = None, None
    o_ref = np.empty((w.B, w.Hq, w.D))
    lse_ref = np.empty((w.B, w.Hq))
    for b in range(w.B):
        for g in range(w.Hkv):
            sl = slice(g * G, (g + 1) * G)
            ob, lb = orc.sparse_decode(q64[b:b + 1, sl], to64(kc[b:b + 1, g:g + 1]), to64(vc[b:b + 1, g:g + 1]),
                                       lens_np[b:b + 1], idx_ref[b:b + 1, g:g + 1], w.block, w.scale)
            o_ref[b, sl], lse_ref[b, sl] = ob[0], lb[0]
    max_abs(to64(step.o), o_ref, 2e-2, "o")
    normwise(to64(step.lse), lse_ref, 1e-4, "lse")
    # All-GPU chain: same selection except at near-ties, and then the same output.
    same = np.all(chain_idx == idx_ref, axis=-1)
    assert same.mean() > 0.95
    for b in range(w.B):
        for g in range(w.Hkv):
            if same[b, g]:
                sl = slice(g * G, (g + 1) * G)
                max_abs(chain_o[b, sl], o_ref[b, sl], 2e-2, "chain o")
    if wi == 4:  # dense decode on the same inputs: every cached position
        dstep = DecodeStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, None, dt)
        dstep.attend(q, kc, vc, lens)
        torch.cuda.synchronize()
        for g in range(w.Hkv):
            sl = slice(g * G, (g + 1) * G)
            ob, _ = orc.sparse_decode(q64[:, sl], to64(kc[:, g:g + 1]), to64(vc[:, g:g + 1]), lens_np, None,
                                      w.block, w.scale)
            max_abs(to64(dstep.o[:, sl]), ob, 2e-2, "dense o")


@pytest.mark.parametrize("wi,topk", [(3, 16), (3, 32), (4, 32)],
                         ids=["decode-128k-b8-k16", "decode-128k-b8-k32", "decode-512k-b1-k32"])
def test_decode_step_fullsize(wi, topk):
    """sas_decode_step at the benchmark sizes (128K tokens x 8 sequences at the
    configured K = 16 and at the metric's 2048-token budget, K = 32; 512K x 1),
    in the configuration bench.py times: its scores against the oracle's, its
    selection bit-exact against the oracle's Top-K on those scores, o and lse
    against the oracle's sparse decode over that selection."""
    w = WORKLOADS[wi].with_(topk=topk)
    dt = w.torch_dtype
    q, kc, vc, lens = decode_inputs(w, device=DEV)
    G = w.Hq // w.Hkv
    lens_np = lens.cpu().numpy()
    kbar = np.empty((w.B, w.Hkv, w.C, w.D))
    for b in range(w.B):
        for g in range(w.Hkv):
            kbar[b, g] = orc.pool_block_keys(to64(kc[b:b + 1, g:g + 1]), w.block)[0, 0]
    kbar_r = to64(torch.tensor(kbar).to(dt))
    o = torch.empty((w.B, w.Hq, w.D), dtype=dt, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((w.B, w.Hkv, topk), dtype=torch.int32, device=DEV)
    ws = sas.workspace(sas.SAS_OP_DECODE_STEP, w.B, w.Hq, w.Hkv, w.N, w.D, w.block, topk, sas.SAS_BF16)
    sas.sas_decode_step(q, torch.tensor(kbar_r).to(dt).to(DEV), kc, vc, lens, topk, o, lse, w.block, w.scale,
                        idx_out=idx, workspace=ws)
    torch.cuda.synchronize()
    q64 = to64(q)
    u_ref = orc.decode_scores(q64, kbar_r, lens_np, w.N, w.block, w.scale, True)
    u_gpu = ws[: w.B * w.Hkv * w.C * 4].view(torch.float32).reshape(w.B, w.Hkv, w.C).cpu().numpy()
    normwise(u_gpu.astype(np.float64), u_ref.astype(np.float64), 1e-5, "u")
    c = orc.decode_candidates(lens_np, w.N, w.block)
    idx_ref = orc.topk_select(u_gpu[:, :, None, :], 1, c[:, None], topk)[:, :, 0, :]
    assert np.array_equal(idx.cpu().numpy(), idx_ref), "Top-K on the step's own scores"
    assert len(np.unique(idx_ref)) > topk  # selection is non-trivial
    o_ref = np.empty((w.B, w.Hq, w.D))
    lse_ref = np.empty((w.B, w.Hq))
    for b in range(w.B):
        for g in range(w.Hkv):
            sl = slice(g * G, (g + 1) * G)
            ob, lb = orc.sparse_decode(q64[b:b + 1, sl], to64(kc[b:b + 1, g:g + 1]), to64(vc[b:b + 1, g:g + 1]),
                                       lens_np[b:b + 1], idx_ref[b:b + 1, g:g + 1], w.block, w.scale)
            o_ref[b, sl], lse_ref[b, sl] = ob[0], lb[0]
    max_abs(to64(o), o_ref, 2e-2, "o")
    _rowwise(to64(o), o_ref, 2e-2, "o per row")
    normwise(to64(lse), lse_ref, 1e-4, "lse")


@pytest.mark.parametrize("wi,topk", [(3, 16), (4, 32)], ids=["decode-128k-b8-k16", "decode-512k-b1-k32"])
def test_paged_decode_fullsize_matches_contiguous(wi, topk):
    """The paged decode chain at the benchmark sizes, in bench.py's page layout
    (pages of one block x all KV heads in a shuffled pool with spare pages, a
    block table per sequence): the pooled pages against the oracle's pooling
    (a sample), and the selection, o and lse bit for bit equal to
    sas_decode_step on the same caches laid out contiguously with the same
    pooled keys (the same kernels; only the addressing differs).
    sas_decode_step itself is held to the oracle in test_decode_step_fullsize."""
    w = WORKLOADS[wi].with_(topk=topk)
    dt = w.torch_dtype
    q, kc, vc, lens = decode_inputs(w, device=DEV)
    C, blk = w.C, w.block
    n_pages = w.B * C + 7
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(3))
    table = perm[: w.B * C].reshape(w.B, C).to(torch.int32).to(DEV)
    rows = table.reshape(-1).long()
    kp = torch.zeros((n_pages, w.Hkv, blk, w.D), dtype=dt, device=DEV)
    vp = torch.zeros_like(kp)
    kp[rows] = kc.view(w.B, w.Hkv, C, blk, w.D).permute(0, 2, 1, 3, 4).reshape(w.B * C, w.Hkv, blk, w.D)
    vp[rows] = vc.view(w.B, w.Hkv, C, blk, w.D).permute(0, 2, 1, 3, 4).reshape(w.B * C, w.Hkv, blk, w.D)
    kbp = torch.zeros((n_pages, w.Hkv, w.D), dtype=dt, device=DEV)
    sas.sas_pool_pages(kp, kbp, table.reshape(-1).contiguous(), blk)
    torch.cuda.synchronize()
    kbar = kbp[rows].reshape(w.B, C, w.Hkv, w.D).permute(0, 2, 1, 3).contiguous()  # [B, Hkv, C, D]
    ref = orc.pool_block_keys(to64(kc[:1, :2]), blk)  # sequence 0, KV heads 0 and 1
    kbar_close(to64(kbar[:1, :2]), to64(torch.tensor(ref).to(dt)), "pooled pages")
    outs = []
    for paged in (False, True):
        o = torch.empty((w.B, w.Hq, w.D), dtype=dt, device=DEV)
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
        idx = torch.empty((w.B, w.Hkv, topk), dtype=torch.int32, device=DEV)
        if paged:
            ws = sas.workspace(sas.SAS_OP_PAGED_DECODE, w.B, w.Hq, w.Hkv, w.N, w.D, blk, topk, sas.SAS_BF16)
            sas.sas_paged_decode(q, kp, vp, kbp, table, lens, topk, o, lse, blk, w.scale, idx_out=idx,
                                 workspace=ws)
        else:
            ws = sas.workspace(sas.SAS_OP_DECODE_STEP, w.B, w.Hq, w.Hkv, w.N, w.D, blk, topk, sas.SAS_BF16)
            sas.sas_decode_step(q, kbar, kc, vc, lens, topk, o, lse, blk, w.scale, idx_out=idx, workspace=ws)
        torch.cuda.synchronize()
        outs.append((idx, o, lse))
        del ws
    (i1, o1, l1), (i2, o2, l2) = outs
    assert torch.equal(i1, i2), "paged selection"
    assert torch.equal(o1, o2), "paged o"
    assert torch.equal(l1, l2), "paged lse"
    assert len(torch.unique(i1)) > topk  # selection is non-trivial


def test_training_at_the_largest_topk():
    """Sparse scope at Top-K 256, the largest the calls take (and the largest
    rank the selection lists encode): 257 history blocks and a ragged tail.
    Top-K bit-exact on every row; o, lse, lse_s on sampled rows; dq and ds
    through the oracle's row gradients; dk and dv on keys of late blocks."""
    B, Hq, Hkv, D, block, topk = 1, 2, 1, 64, 64, 256
    N = 258 * block + 37
    w = Workload("train-topk256", "train", "bf16", B, Hq, Hkv, D, N, block, topk, index=90)
    dt = w.torch_dtype
    q, k, v, do = training_inputs(w, device=DEV)
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(do)
    G, C = Hq // Hkv, N // block
    kbar_r = to64(torch.tensor(orc.pool_block_keys(k64, block)).to(dt))
    s32 = _oracle_scores_f32(q64, kbar_r, block, w.scale)
    pos = np.arange(N)[None, :] // block
    idx = orc.topk_select(s32, G, pos, topk)
    step = TrainStep(B, Hq, Hkv, N, D, block, topk, dt)
    scores = torch.tensor(s32).to(DEV)
    sas.sas_topk_select(scores, step.idx, None, G, block)
    torch.cuda.synchronize()
    assert np.array_equal(step.idx.cpu().numpy(), idx), "topk 256, every row"
    idx_t = torch.tensor(idx).to(DEV)
    step.forward(q, k, v, scores, idx_t)
    step.backward(q, k, v, do, scores, idx_t)
    torch.cuda.synchronize()
    rows = _sample_rows(N, block)
    s64 = s32.astype(np.float64)
    o_ref, lse_ref, lses_ref = orc.gated_attention_forward(q64, k64, v64, s64, idx, block, w.scale, rows=rows)
    max_abs(to64(step.o[:, :, rows]), o_ref, 2e-2, "o")
    _rowwise(to64(step.o[:, :, rows]), o_ref, 2e-2, "o per row")
    normwise(to64(step.lse[:, :, rows]), lse_ref, 1e-4, "lse")
    normwise(to64(step.lse_s[:, :, rows]), lses_ref, 1e-4, "lse_s")
    for h in range(Hq):
        dq_r, ds_r = orc.row_gradients(q64, k64, v64, do64, s64, idx, block, w.scale, 0, h, rows)
        normwise(to64(step.dq[0, h, rows]), dq_r, 2e-2, f"dq h{h}")
        normwise(to64(step.ds[0, h, rows]), ds_r, 2e-2, f"ds h{h}")
    keys = np.array([(C - 6) * block + 5, (C - 1) * block + 63, N - 1])
    kb = np.unique(keys // block)
    attend = np.nonzero(np.any(np.isin(idx[0, 0], kb), axis=-1) | np.isin(np.arange(N) // block, kb))[0]
    dk_r, dv_r = orc.key_gradients(q64, k64, v64, do64, s64, idx, block, w.scale, 0, 0, keys, rows=attend)
    normwise(to64(step.dk[0, 0, keys]), dk_r, 2e-2, "dk")
    normwise(to64(step.dv[0, 0, keys]), dv_r, 2e-2, "dv")


def test_decode_step_at_the_largest_sizes():
    """sas_decode_step at the largest history the calls take (16384 blocks of
    64 tokens: a 1M-token cache) and the largest Top-K (256): scores against the
    oracle's, the selection bit-exact on those scores, o and lse against the
    oracle's sparse decode."""
    block, topk = 64, 256
    L = 16384 * block
    w = Workload("decode-1m-k256", "decode", "bf16", 1, 4, 1, 128, L, block, topk, index=91)
    dt = w.torch_dtype
    q, kc, vc, lens = decode_inputs(w, device=DEV)
    C = L // block
    kbar_r = to64(torch.tensor(orc.pool_block_keys(to64(kc), block)).to(dt))
    o = torch.empty((w.B, w.Hq, w.D), dtype=dt, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((w.B, w.Hkv, topk), dtype=torch.int32, device=DEV)
    ws = sas.workspace(sas.SAS_OP_DECODE_STEP, w.B, w.Hq, w.Hkv, L, w.D, block, topk, sas.SAS_BF16)
    sas.sas_decode_step(q, torch.tensor(kbar_r).to(dt).to(DEV), kc, vc, lens, topk, o, lse, block, w.scale,
                        idx_out=idx, workspace=ws)
    torch.cuda.synchronize()
    lens_np = lens.cpu().numpy()
    q64 = to64(q)
    u_ref = orc.decode_scores(q64, kbar_r, lens_np, L, block, w.scale, True)
    u_gpu = ws[: w.B * w.Hkv * C * 4].view(torch.float32).reshape(w.B, w.Hkv, C).cpu().numpy()
    normwise(u_gpu.astype(np.float64), u_ref.astype(np.float64), 1e-5, "u")
    c = orc.decode_candidates(lens_np, L, block)
    idx_ref = orc.topk_select(u_gpu[:, :, None, :], 1, c[:, None], topk)[:, :, 0, :]
    assert np.array_equal(idx.cpu().numpy(), idx_ref), "Top-K 256 over 16383 candidates"
    o_ref, lse_ref = orc.sparse_decode(q64, to64(kc), to64(vc), lens_np, idx_ref, block, w.scale)
    max_abs(to64(o), o_ref, 2e-2, "o")
    _rowwise(to64(o), o_ref, 2e-2, "o per row")
    normwise(to64(lse), lse_ref, 1e-4, "lse")
