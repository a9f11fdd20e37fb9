"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something other than itself: the worked
example printed on the pages, closed forms, textbook / library attention
(torch's scaled_dot_product_attention and autograd in float64), finite
differences, brute-force enumeration, and invariants the method implies.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import sas_oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.default_rng(seed)


def rand_problem(seed, B=1, Hq=2, Hkv=1, N=64, D=8, block=8):
    r = rng(seed)
    q = r.standard_normal((B, Hq, N, D))
    k = r.standard_normal((B, Hkv, N, D))
    v = r.standard_normal((B, Hkv, N, D))
    do = r.standard_normal((B, Hq, N, D))
    C = N // block
    s = r.standard_normal((B, Hq, N, C))
    return q, k, v, do, s


def causal_sdpa(q, k, v, scale, mask=None, is_causal=False):
    """Library attention in float64 over [Hq,N,D] with GQA expansion."""
    Hq, Hkv = q.shape[0], k.shape[0]
    G = Hq // Hkv
    kk = k.repeat_interleave(G, dim=0)
    vv = v.repeat_interleave(G, dim=0)
    return F.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, is_causal=is_causal, scale=scale)


# ---------------------------------------------------------------------------
# Worked example printed on the pages
# ---------------------------------------------------------------------------

def test_worked_example_gate_and_selection():
    ex = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    block, C = ex["block"], ex["num_history_blocks"]
    s_row = np.array(ex["scores"])
    tol = ex["printed_rounding"]
    # A query in block C (the current block B_0 of the page) with C history blocks.
    N = (C + 1) * block
    t = N - 1
    D = C + 1
    q = np.zeros((1, 1, N, D))  # q = 0: every logit is 0, only the gate biases remain
    k = rng(1).standard_normal((1, 1, N, D))
    v = np.zeros((1, 1, N, D))
    for j in range(N):
        v[0, 0, j, j // block] = 1.0  # one-hot block id: o reads out the mass per block
    s = np.zeros((1, 1, N, C))
    s[0, 0, :, :] = s_row
    # Step 2: g = softmax(s); the page prints e^s and their sum.
    np.testing.assert_allclose(np.exp(s_row), ex["exp_scores_printed"], atol=0.006)
    np.testing.assert_allclose(np.exp(s_row).sum(), ex["exp_sum_printed"], atol=0.006)
    o, lse, lse_s = orc.gated_attention_forward(q, k, v, s, None, block, 1.0, rows=[t])
    log_g_printed = np.array(ex["log_gates_printed"])
    # Step 4: log g = s - LSE(s); the oracle's LSE must reproduce the printed log gates.
    np.testing.assert_allclose(s_row - lse_s[0, 0, 0], log_g_printed, atol=tol)
    # Full scope: the current block has gate 1 on its 64 keys, block m has g_m on each key.
    g = np.exp(log_g_printed)
    g = g / g.sum()
    Z = block * 1.0 + block * g.sum()
    expect = np.concatenate([block * g / Z, [block / Z]])
    np.testing.assert_allclose(o[0, 0, 0], expect, atol=0.01)
    # Step 3: Top-2 picks B_2 then B_1.
    sc = np.zeros((1, 1, N, C), dtype=np.float32)
    sc[...] = s_row.astype(np.float32)
    idx = orc.topk_select(sc, 1, np.array([[j // block for j in range(N)]]), ex["topk"])
    assert list(idx[0, 0, t]) == ex["selected_zero_based_in_order"]
    # Step 4 at sparse scope: only B_0, B_2, B_1 take part, with biases log g.
    o2, _, _ = orc.gated_attention_forward(q, k, v, s, idx, block, 1.0, rows=[t])
    gsel = np.exp(np.array([ex["bias_added_printed"]["B_1"], ex["bias_added_printed"]["B_2"]]))
    Z2 = block * (1.0 + gsel.sum())
    expect2 = np.array([block * gsel[0] / Z2, block * gsel[1] / Z2, 0.0, 0.0, block / Z2])
    np.testing.assert_allclose(o2[0, 0, 0], expect2, atol=0.01)


# ---------------------------------------------------------------------------
# Forward: special cases that reduce to library attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_history_block_is_dense_causal(seed):
    """With one history block its gate is 1, so the layer is plain causal attention."""
    block, D = 16, 8
    N = 2 * block
    q, k, v, do, s = rand_problem(seed, Hq=4, Hkv=2, N=N, D=D, block=block)
    scale = 1 / math.sqrt(D)
    o, lse, lse_s = orc.gated_attention_forward(q, k, v, s, None, block, scale)
    ref = causal_sdpa(*(torch.tensor(x[0]) for x in (q, k, v)), scale, is_causal=True)
    np.testing.assert_allclose(o[0], ref.numpy(), rtol=0, atol=1e-12)
    # Gradients against autograd of the library routine; the gate gradient is 0.
    qt, kt, vt = (torch.tensor(x[0], requires_grad=True) for x in (q, k, v))
    out = causal_sdpa(qt, kt, vt, scale, is_causal=True)
    (out * torch.tensor(do[0])).sum().backward()
    dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, None, block, scale)
    np.testing.assert_allclose(dq[0], qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk[0], kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv[0], vt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(ds, 0.0, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_equal_scores_give_uniform_gates(seed):
    """Equal scores on c history blocks: every gate is 1/c, bias -log c (closed form)."""
    block, D, N = 8, 8, 48
    q, k, v, do, _ = rand_problem(seed, Hq=2, Hkv=1, N=N, D=D, block=block)
    s = np.full((1, 2, N, N // block), 0.37)
    scale = 0.5
    o, _, _ = orc.gated_attention_forward(q, k, v, s, None, block, scale)
    t = np.arange(N)
    c = t // block
    j = np.arange(N)
    bias = np.where(j[None, :] // block == c[:, None], np.where(j[None, :] <= t[:, None], 0.0, -np.inf),
                    np.where(j[None, :] // block < c[:, None], -np.log(np.maximum(c, 1))[:, None], -np.inf))
    ref = causal_sdpa(*(torch.tensor(x[0]) for x in (q, k, v)), scale, mask=torch.tensor(bias))
    np.testing.assert_allclose(o[0], ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("seed", [5, 6])
def test_topk_zero_is_block_diagonal_causal(seed):
    """Sparse scope with no selected block: each query sees only its own block causally."""
    block, D, N = 8, 8, 40
    q, k, v, do, s = rand_problem(seed, Hq=2, Hkv=1, N=N, D=D, block=block)
    idx = np.zeros((1, 1, N, 0), dtype=np.int32)
    o, _, _ = orc.gated_attention_forward(q, k, v, s, idx, block, 0.3)
    t = np.arange(N)
    same = (t[None, :] // block == t[:, None] // block) & (t[None, :] <= t[:, None])
    ref = causal_sdpa(*(torch.tensor(x[0]) for x in (q, k, v)), 0.3, mask=torch.tensor(same))
    np.testing.assert_allclose(o[0], ref.numpy(), atol=1e-12)


def _torch_sas(q, k, v, s, sel, block, scale):
    """SAS forward assembled from library pieces (log_softmax, SDPA) for autograd.

    sel: bool [Hq, N, C] selection (history only).  The bias is the library's
    log_softmax of s over each row's history, spread over the keys of each block.
    """
    Hq, N, D = q.shape
    C = s.shape[-1]
    t = torch.arange(N)
    c = t // block
    hist = torch.arange(C)[None, :] < c[:, None]
    logg = torch.log_softmax(s.masked_fill(~hist, float("-inf")), dim=-1)
    logg = torch.where(hist, logg, torch.zeros((), dtype=s.dtype))
    key_block = torch.arange(N) // block
    per_key = logg[..., key_block]  # [Hq, N, N]
    use = sel[..., key_block] & (key_block[None, :] < c[:, None])
    own = (key_block[None, :] == c[:, None]) & (t[None, :] <= t[:, None])
    neg = torch.full((), float("-inf"), dtype=s.dtype)
    mask = torch.where(own, torch.zeros((), dtype=s.dtype), torch.where(use, per_key, neg))
    return causal_sdpa(q, k, v, scale, mask=mask)


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("seed", [7, 8])
def test_against_library_autograd(seed, sparse):
    """Forward and all four gradients against autograd through library ops."""
    block, D, N, Hq, Hkv, K = 8, 8, 56, 4, 2, 3
    q, k, v, do, s = rand_problem(seed, Hq=Hq, Hkv=Hkv, N=N, D=D, block=block)
    scale = 1 / math.sqrt(D)
    C = N // block
    pos = np.arange(N)[None, :]
    if sparse:
        idx = orc.topk_select(s.astype(np.float32), Hq // Hkv, pos // block, K)
        sel = np.zeros((Hq, N, C), dtype=bool)
        for h in range(Hq):
            for t in range(N):
                for m in idx[0, h // (Hq // Hkv), t]:
                    if m >= 0:
                        sel[h, t, m] = True
    else:
        idx = None
        sel = np.ones((Hq, N, C), dtype=bool)
    o, _, _ = orc.gated_attention_forward(q, k, v, s, idx, block, scale)
    qt, kt, vt, st = (torch.tensor(x[0], requires_grad=True) for x in (q, k, v, s))
    out = _torch_sas(qt, kt, vt, st, torch.tensor(sel), block, scale)
    np.testing.assert_allclose(o[0], out.detach().numpy(), atol=1e-12)
    (out * torch.tensor(do[0])).sum().backward()
    dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, idx, block, scale)
    np.testing.assert_allclose(dq[0], qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk[0], kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv[0], vt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(ds[0], st.grad.numpy(), atol=1e-11)


def test_topk_at_least_history_equals_full_scope():
    """K >= number of history blocks reproduces full scope, forward and backward."""
    block, D, N = 8, 8, 48
    q, k, v, do, s = rand_problem(11, Hq=2, Hkv=1, N=N, D=D, block=block)
    C = N // block
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, C)
    a = orc.gated_attention_forward(q, k, v, s, idx, block, 0.4)
    b = orc.gated_attention_forward(q, k, v, s, None, block, 0.4)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-13)
    ga = orc.gated_attention_backward(q, k, v, do, s, idx, block, 0.4)
    gb = orc.gated_attention_backward(q, k, v, do, s, None, block, 0.4)
    for x, y in zip(ga, gb):
        np.testing.assert_allclose(x, y, atol=1e-13)


# ---------------------------------------------------------------------------
# Backward: finite differences and invariants
# ---------------------------------------------------------------------------

def _loss(q, k, v, do, s, idx, block, scale):
    o, _, _ = orc.gated_attention_forward(q, k, v, s, idx, block, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("sparse", [False, True])
def test_finite_differences(sparse):
    """Central differences of L = sum(dO * o) in fp64 match every gradient."""
    block, D, N, Hq, Hkv = 4, 4, 20, 2, 1
    q, k, v, do, s = rand_problem(21, Hq=Hq, Hkv=Hkv, N=N, D=D, block=block)
    scale = 0.7
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, 2) if sparse else None
    dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, idx, block, scale)
    eps = 1e-6
    r = rng(5)

    def fd(arr, pos):
        a0 = arr[pos]
        arr[pos] = a0 + eps
        lp = _loss(q, k, v, do, s, idx, block, scale)
        arr[pos] = a0 - eps
        lm = _loss(q, k, v, do, s, idx, block, scale)
        arr[pos] = a0
        return (lp - lm) / (2 * eps)

    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for _ in range(12):
            pos = tuple(int(r.integers(0, n)) for n in arr.shape)
            assert abs(fd(arr, pos) - grad[pos]) < 1e-7 * max(1.0, abs(grad[pos]))
    # Every history score of a few rows (selected and unselected alike).
    for t in (5, 11, 19):
        for h in range(Hq):
            for m in range(t // block):
                pos = (0, h, t, m)
                assert abs(fd(s, pos) - ds[pos]) < 1e-7, (pos, fd(s, pos), ds[pos])


def test_gate_gradient_invariants():
    """sum_m ds = 0 over the history; unselected blocks share ds/g (the sparse-scope
    "indirect" gradient of the pages' gradient-behaviour figure); shifting a row of
    s by a constant changes nothing."""
    block, D, N = 8, 8, 80
    q, k, v, do, s = rand_problem(31, Hq=4, Hkv=1, N=N, D=D, block=block)
    scale = 0.35
    idx = orc.topk_select(s.astype(np.float32), 4, np.arange(N)[None, :] // block, 2)
    dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, idx, block, scale)
    np.testing.assert_allclose(ds.sum(axis=-1), 0.0, atol=1e-12)
    for h in range(4):
        for t in range(N):
            c = t // block
            if c < 4:
                continue
            sel = set(int(m) for m in idx[0, 0, t] if m >= 0)
            uns = [m for m in range(c) if m not in sel]
            gate = np.exp(s[0, h, t, :c] - np.log(np.exp(s[0, h, t, :c]).sum()))
            ratios = ds[0, h, t, uns] / gate[uns]
            np.testing.assert_allclose(ratios, ratios[0], rtol=1e-9, atol=1e-12)
    shift = rng(2).standard_normal((1, 4, N, 1)) * 3
    s2 = s + shift
    idx2 = orc.topk_select(s2.astype(np.float32), 4, np.arange(N)[None, :] // block, 2)
    g1 = orc.gated_attention_backward(q, k, v, do, s, idx, block, scale)
    g2 = orc.gated_attention_backward(q, k, v, do, s2, idx, block, scale)
    for x, y in zip(g1, g2):
        np.testing.assert_allclose(x, y, atol=1e-10)
    o1 = orc.gated_attention_forward(q, k, v, s, idx, block, scale)[0]
    o2 = orc.gated_attention_forward(q, k, v, s2, idx, block, scale)[0]
    np.testing.assert_allclose(o1, o2, atol=1e-12)


def test_inner_gate_gradient_closed_form():
    """dbeta_m = g_m * dg_m^inner = sum_{i in B_m} p_i dO.(v_i - o) (paper Eq. 5),
    with p from the library softmax; ds is dbeta - g * sum(dbeta)."""
    block, D, N = 8, 8, 40
    q, k, v, do, s = rand_problem(41, Hq=1, Hkv=1, N=N, D=D, block=block)
    scale = 0.5
    _, _, _, ds = orc.gated_attention_backward(q, k, v, do, s, None, block, scale)
    qt, kt, vt, st = (torch.tensor(x[0]) for x in (q, k, v, s))
    C = N // block
    for t in (17, 30, 39):
        c = t // block
        logg = torch.log_softmax(st[0, t, :c], dim=0)
        z = torch.full((N,), float("-inf"), dtype=torch.float64)
        for j in range(N):
            m = j // block
            if m < c:
                z[j] = scale * qt[0, t] @ kt[0, j] + logg[m]
            elif m == c and j <= t:
                z[j] = scale * qt[0, t] @ kt[0, j]
        p = torch.softmax(z, dim=0)
        o = p @ vt[0]
        dO = torch.tensor(do[0, 0, t])
        dbeta = torch.stack([(p[m * block:(m + 1) * block] * ((vt[0, m * block:(m + 1) * block] - o) @ dO)).sum()
                             for m in range(c)])
        expect = dbeta - torch.exp(logg) * dbeta.sum()
        np.testing.assert_allclose(ds[0, 0, t, :c], expect.numpy(), atol=1e-12)
        np.testing.assert_allclose(ds[0, 0, t, c:], 0.0)


# ---------------------------------------------------------------------------
# Selector scores and Top-K
# ---------------------------------------------------------------------------

def test_pool_and_scores_closed_form():
    block, D = 8, 16
    r = rng(3)
    w = r.standard_normal((4, D))
    k = np.repeat(w[None, None, :, None, :], block, axis=3).reshape(1, 1, 4 * block, D)
    kbar = orc.pool_block_keys(k, block)
    np.testing.assert_allclose(kbar[0, 0], w, atol=1e-15)
    # Against the library average pool on random keys.
    k2 = r.standard_normal((2, 3, 5 * block + 3, D))
    ref = F.avg_pool1d(torch.tensor(k2).transpose(-1, -2).reshape(6, D, -1), block).reshape(2, 3, D, 5)
    np.testing.assert_allclose(orc.pool_block_keys(k2, block), ref.transpose(-1, -2).numpy(), atol=1e-14)
    q = r.standard_normal((1, 2, 40, D))
    s = orc.block_scores(q, kbar, block, 0.25, np.arange(40)[None, :])
    for t in range(40):
        c = t // block
        for m in range(4):
            if m < c:
                assert abs(s[0, 1, t, m] - 0.25 * float(q[0, 1, t] @ w[m])) < 1e-12
            else:
                assert s[0, 1, t, m] == -np.inf


def test_topk_brute_force():
    r = rng(9)
    for trial in range(200):
        C = int(r.integers(1, 40))
        G = int(r.integers(1, 4))
        K = int(r.integers(0, 12))
        c = int(r.integers(0, C + 1))
        sc = r.standard_normal((1, G, 1, C)).astype(np.float32)
        if trial % 3 == 0:  # many exact ties
            sc = np.round(sc).astype(np.float32)
        idx = orc.topk_select(sc, G, np.array([[c]]), K)[0, 0, 0]
        u = sc[0, 0, 0].copy()
        for h in range(1, G):
            u = np.float32(u + sc[0, h, 0])
        cand = sorted(range(c), key=lambda m: (-float(u[m]), m))[:K]
        assert list(idx[: len(cand)]) == cand
        assert all(x == -1 for x in idx[len(cand):])


def test_topk_special_values():
    sc = np.array([[[[0.5, -0.0, 0.0, np.nan, -np.inf, 0.5, np.inf]]]], dtype=np.float32)
    idx = orc.topk_select(sc, 1, np.array([[7]]), 7)[0, 0, 0]
    # +inf first; the 0.5 tie goes to the lower index; -0.0 equals +0.0 (lower index
    # first); NaN ranks as -inf and ties with -inf by index.
    assert list(idx) == [6, 0, 5, 1, 2, 3, 4]
    idx = orc.topk_select(sc, 1, np.array([[3]]), 5)[0, 0, 0]
    assert list(idx) == [0, 1, 2, -1, -1]


def test_topk_group_sum_order():
    """The group sum is ((s0 + s1) + s2) in fp32, which can differ from other orders."""
    a = np.float32(1e8)
    sc = np.zeros((1, 3, 1, 2), dtype=np.float32)
    # block 0: (1e8 + 1) + -1e8 = 0 in fp32 (1e8 + 1 rounds to 1e8)
    sc[0, :, 0, 0] = [a, 1.0, -a]
    # block 1: (1e8 + -1e8) + 0.5 = 0.5
    sc[0, :, 0, 1] = [a, -a, 0.5]
    idx = orc.topk_select(sc, 3, np.array([[2]]), 1)[0, 0, 0]
    assert list(idx) == [1]
    sc[0, :, 0, 1] = [a, -a, -0.5]
    idx = orc.topk_select(sc, 3, np.array([[2]]), 1)[0, 0, 0]
    assert list(idx) == [0]


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def _decode_problem(seed, B=2, Hq=4, Hkv=2, L=96, D=8):
    r = rng(seed)
    return (r.standard_normal((B, Hq, D)), r.standard_normal((B, Hkv, L, D)),
            r.standard_normal((B, Hkv, L, D)))


def test_decode_dense_is_library_attention():
    q, kc, vc = _decode_problem(1)
    lens = np.array([96, 37])
    o, lse = orc.sparse_decode(q, kc, vc, lens, None, 8, 0.3)
    for b in range(2):
        n = lens[b]
        ref = causal_sdpa(torch.tensor(q[b][:, None, :]), torch.tensor(kc[b, :, :n]),
                          torch.tensor(vc[b, :, :n]), 0.3)
        np.testing.assert_allclose(o[b], ref[:, 0].numpy(), atol=1e-12)


def test_decode_topk_at_least_history_is_dense():
    q, kc, vc = _decode_problem(2)
    lens = np.array([96, 61])
    block = 8
    u = orc.decode_scores(q, orc.pool_block_keys(kc, block), lens, kc.shape[2], block, 0.3, True)
    c = (lens - 1) // block
    idx = orc.topk_select(u[:, :, None, :], 1, c[:, None], 12)[:, :, 0, :]
    a = orc.sparse_decode(q, kc, vc, lens, idx, block, 0.3)
    b = orc.sparse_decode(q, kc, vc, lens, None, block, 0.3)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12)


def test_decode_current_block_only_and_no_gate():
    q, kc, vc = _decode_problem(3)
    block = 16
    lens = np.array([9, 40])
    idx = np.array([[[1, 0], [0, 5]], [[1, 1], [-1, 7]]], dtype=np.int32)
    o, _ = orc.sparse_decode(q, kc, vc, lens, idx, block, 0.3)
    # len <= b: only the current block; idx is ignored.
    ref = causal_sdpa(torch.tensor(q[0][:, None, :]), torch.tensor(kc[0, :, :9]), torch.tensor(vc[0, :, :9]), 0.3)
    np.testing.assert_allclose(o[0], ref[:, 0].numpy(), atol=1e-12)
    # pos 39 -> current block 2 (keys 32..39); KV head 0 repeats block 1 (counted once),
    # KV head 1 holds only invalid entries.  No gate: plain softmax over those keys.
    for g, keys in ((0, list(range(16, 32)) + list(range(32, 40))), (1, list(range(32, 40)))):
        ref = causal_sdpa(torch.tensor(q[1, 2 * g:2 * g + 2][:, None, :]), torch.tensor(kc[1][g:g + 1][:, keys]),
                          torch.tensor(vc[1][g:g + 1][:, keys]), 0.3)
        np.testing.assert_allclose(o[1, 2 * g:2 * g + 2], ref[:, 0].numpy(), atol=1e-12)


def test_decode_scores_group_sum():
    q, kc, _ = _decode_problem(4, L=64)
    block = 8
    kbar = orc.pool_block_keys(kc, block)
    lens = np.array([64, 30])
    s = orc.decode_scores(q, kbar, lens, 64, block, 0.5, False)
    u = orc.decode_scores(q, kbar, lens, 64, block, 0.5, True)
    for b in range(2):
        c = (lens[b] - 1) // block
        for g in range(2):
            for m in range(8):
                if m < c:
                    want = np.float32(np.float32(0.5 * q[b, 2 * g] @ kbar[b, g, m]) +
                                      np.float32(0.5 * q[b, 2 * g + 1] @ kbar[b, g, m]))
                    assert u[b, g, m] == want
                    assert abs(s[b, 2 * g, m] - 0.5 * q[b, 2 * g] @ kbar[b, g, m]) < 1e-12
                else:
                    assert u[b, g, m] == -np.inf


def test_row_and_key_gradient_helpers_match_full_backward():
    block, D, N = 8, 8, 64
    q, k, v, do, s = rand_problem(51, Hq=4, Hkv=2, N=N, D=D, block=block)
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, 2)
    for sc in (None, idx):
        dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, sc, block, 0.4)
        rows = [0, 9, 33, 63]
        rdq, rds = orc.row_gradients(q, k, v, do, s, sc, block, 0.4, 0, 3, rows)
        np.testing.assert_allclose(rdq, dq[0, 3, rows], atol=1e-12)
        np.testing.assert_allclose(rds, ds[0, 3, rows], atol=1e-12)
        keys = [1, 17, 40, 63]
        kdk, kdv = orc.key_gradients(q, k, v, do, s, sc, block, 0.4, 0, 1, keys, row_chunk=7)
        np.testing.assert_allclose(kdk, dk[0, 1, keys], atol=1e-12)
        np.testing.assert_allclose(kdv, dv[0, 1, keys], atol=1e-12)
        o, lse, lse_s = orc.gated_attention_forward(q, k, v, s, sc, block, 0.4)
        o2, lse2, lse_s2 = orc.gated_attention_forward(q, k, v, s, sc, block, 0.4, rows=rows)
        np.testing.assert_allclose(o2, o[:, :, rows], atol=1e-13)
        np.testing.assert_allclose(lse2, lse[:, :, rows], atol=1e-13)


def test_decode_idle_and_overlong_sequences():
    """Idle sequences give zero output and lse -inf; lengths beyond the cache clamp."""
    q, kc, vc = _decode_problem(5, L=64)
    idx = np.array([[[0, 1], [1, 0]], [[0, 2], [3, 1]]], dtype=np.int32)
    o, lse = orc.sparse_decode(q, kc, vc, np.array([0, 500]), idx, 16, 0.3)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    o2, lse2 = orc.sparse_decode(q, kc, vc, np.array([0, 64]), idx, 16, 0.3)
    np.testing.assert_array_equal(o[1], o2[1])
    od, _ = orc.sparse_decode(q, kc, vc, np.array([-3, 64]), None, 16, 0.3)
    assert np.all(od[0] == 0)
    u = orc.decode_scores(q, orc.pool_block_keys(kc, 16), np.array([0, 64]), 64, 16, 0.3, True)
    assert np.all(u[0] == -np.inf)


@pytest.mark.parametrize("L_max,block", [(64, 16), (70, 16), (48, 16), (100, 32)])
def test_decode_scores_over_long_lengths(L_max, block):
    """Lengths at, just above and far above the capacity: the candidates are the
    complete blocks before the block holding position min(len, L_max) - 1, found
    here by searching for the block whose token range holds that position (not
    by division), so the current block is -inf however long the length is; the
    same reading as sparse_decode, whose output for an over-long length equals
    the one for L_max."""
    r = rng(17)
    B, Hq, Hkv, D = 1, 2, 1, 8
    C = L_max // block
    q = r.standard_normal((B, Hq, D))
    kc = r.standard_normal((B, Hkv, L_max, D))
    vc = r.standard_normal((B, Hkv, L_max, D))
    kbar = orc.pool_block_keys(kc, block)
    ref_s = orc.decode_scores(q, kbar, np.array([L_max]), L_max, block, 0.3, False)
    for n in (L_max, L_max + 1, L_max + block, 10 * L_max):
        s = orc.decode_scores(q, kbar, np.array([n]), L_max, block, 0.3, False)
        p = min(n, L_max) - 1
        cur = next(m for m in range(C + 1) if m * block <= p < (m + 1) * block)
        for m in range(C):
            assert np.all(np.isfinite(s[0, :, m]) == (m < cur)), (n, m, cur)
        np.testing.assert_array_equal(s, ref_s)
        u = orc.decode_scores(q, kbar, np.array([n]), L_max, block, 0.3, True)
        assert np.all(np.isfinite(u[0, 0]) == (np.arange(C) < cur))
        assert orc.decode_candidates(np.array([n]), L_max, block)[0] == cur
        # full selection over the candidates = dense decode, also over-long
        idx = np.arange(cur, dtype=np.int32).reshape(1, 1, cur)
        o, lse = orc.sparse_decode(q, kc, vc, np.array([n]), idx, block, 0.3)
        od, lsed = orc.sparse_decode(q, kc, vc, np.array([L_max]), None, block, 0.3)
        np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lsed, rtol=1e-12)


# ---------------------------------------------------------------------------
# Selector backward (mean-pool selector)
# ---------------------------------------------------------------------------

def _selector_problem(seed, B=1, Hq=4, Hkv=2, N=40, D=6, block=8):
    r = rng(seed)
    q = r.standard_normal((B, Hq, N, D))
    k = r.standard_normal((B, Hkv, N, D))
    C = N // block
    w = r.standard_normal((B, Hq, N, C))  # the upstream ds
    return q, k, w, C


def _selector_loss(q, k, w, block, scale):
    """sum over the finite scores of w * s, through the oracle's own forward."""
    N = q.shape[2]
    kbar = orc.pool_block_keys(k, block)
    s = orc.block_scores(q, kbar, block, scale, np.broadcast_to(np.arange(N), (q.shape[0], N)))
    return float(np.sum(np.where(np.isfinite(s), w * s, 0.0)))


@pytest.mark.parametrize("N", [40, 37])  # 37: a tail of 5 tokens outside every complete block
def test_selector_backward_finite_differences(N):
    q, k, w, C = _selector_problem(3, N=N)
    block, scale = 8, 0.37
    dq, dkbar, dk = orc.selector_backward(q, k, w[..., : N // block], block, scale)
    eps = 1e-5
    for arr, grad in ((q, dq), (k, dk)):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            a0 = arr[i]
            arr[i] = a0 + eps
            lp = _selector_loss(q, k, w[..., : N // block], block, scale)
            arr[i] = a0 - eps
            lm = _selector_loss(q, k, w[..., : N // block], block, scale)
            arr[i] = a0
            assert abs((lp - lm) / (2 * eps) - grad[i]) < 1e-7, (i, (lp - lm) / (2 * eps), grad[i])


def test_selector_backward_against_library_autograd():
    q, k, w, C = _selector_problem(5, B=2, Hq=6, Hkv=3, N=48, D=8, block=8)
    block, scale = 8, 0.25
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    B, Hq, N, D = q.shape
    G = Hq // k.shape[1]
    kbar = kt[:, :, : C * block].reshape(B, k.shape[1], C, block, D).mean(dim=3)
    s = scale * torch.matmul(qt, kbar.repeat_interleave(G, dim=1).transpose(-1, -2).contiguous())
    mask = torch.arange(C)[None, :] < (torch.arange(N) // block)[:, None]
    (torch.where(mask, s, torch.zeros_like(s)) * torch.tensor(w)).sum().backward()
    dq, dkbar, dk = orc.selector_backward(q, k, w, block, scale)
    assert np.allclose(dq, qt.grad.numpy(), atol=1e-12, rtol=1e-10)
    assert np.allclose(dk, kt.grad.numpy(), atol=1e-12, rtol=1e-10)


def test_selector_backward_bilinear_identity_and_pool_structure():
    # s is bilinear in (q, K̄), so sum ds * s = sum q . dq = sum K̄ . dK̄; every
    # token of block m carries dK̄[m] / b and the tail carries nothing.
    q, k, w, C = _selector_problem(7, N=45)
    block, scale = 8, 0.5
    C = 45 // block
    w = w[..., :C]
    dq, dkbar, dk = orc.selector_backward(q, k, w, block, scale)
    kbar = orc.pool_block_keys(k, block)
    s = orc.block_scores(q, kbar, block, scale, np.arange(45)[None, :])
    lhs = np.sum(np.where(np.isfinite(s), w * s, 0.0))
    assert abs(lhs - np.sum(q * dq)) < 1e-10
    assert abs(lhs - np.sum(kbar * dkbar)) < 1e-10
    for m in range(C):
        for j in range(m * block, (m + 1) * block):
            assert np.allclose(dk[:, :, j], dkbar[:, :, m] / block, atol=0, rtol=1e-15)
    assert np.all(dk[:, :, C * block:] == 0)
    # queries of block 0 have no history: zero gradient
    assert np.all(dq[:, :, :block] == 0)
    # with N a multiple of b no query has the last block in its history
    q2, k2, w2, C2 = _selector_problem(8, N=48)
    _, dkbar2, _ = orc.selector_backward(q2, k2, w2, block, scale)
    assert np.all(dkbar2[:, :, C2 - 1] == 0) and np.any(dkbar2[:, :, C2 - 2] != 0)


def test_selector_subset_helpers_match_full_backward():
    q, k, w, C = _selector_problem(11, B=2, Hq=6, Hkv=2, N=53, D=5, block=8)
    block, scale = 8, 0.3
    C = 53 // block
    w = w[..., :C]
    dq, dkbar, _ = orc.selector_backward(q, k, w, block, scale)
    kbar = orc.pool_block_keys(k, block)
    rows = [0, 7, 8, 30, 52]
    for b in range(2):
        for h in (0, 3, 5):
            assert np.allclose(orc.selector_dq_rows(kbar, w, block, scale, b, h, rows), dq[b, h, rows],
                               atol=1e-13, rtol=1e-12)
        for g in range(2):
            blocks = [0, 2, C - 1]
            assert np.allclose(orc.selector_dkbar_blocks(q, w, block, scale, b, g, 3, blocks),
                               dkbar[b, g, blocks], atol=1e-13, rtol=1e-12)


# ---------------------------------------------------------------------------
# Gate activations other than the softmax (the pages' ablation: sigmoid gate,
# raw logit injected into the attention logits)
# ---------------------------------------------------------------------------

def _gate_value(gate, s):
    return 1.0 / (1.0 + np.exp(-s)) if gate == "sigmoid" else np.exp(s)


@pytest.mark.parametrize("gate", ["sigmoid", "raw"])
@pytest.mark.parametrize("sparse", [False, True])
def test_gate_variant_forward_as_multiplicative_gate(gate, sparse):
    """With gate value g_m (sigmoid(s_m), or e^{s_m} for the raw logit) the
    forward is the gate multiplying exp(z) inside the softmax: o = sum_j g e^z v /
    sum_j g e^z, own block g = 1 (blog 方法核心 / review "New Approach" with the
    gate of the ablation), written out key by key."""
    block, D, N = 4, 5, 28
    q, k, v, do, s = rand_problem(61, Hq=2, Hkv=1, N=N, D=D, block=block)
    scale = 0.6
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, 2) if sparse else None
    o, lse, lse_s = orc.gated_attention_forward(q, k, v, s, idx, block, scale, gate=gate)
    np.testing.assert_array_equal(lse_s, 0.0)
    for h in range(2):
        for t in range(N):
            c = t // block
            sel = set(range(c)) if idx is None else {int(m) for m in idx[0, 0, t] if 0 <= m < c}
            num = np.zeros(D)
            den = 0.0
            for j in range(t + 1):
                m = j // block
                if m == c:
                    w = 1.0
                elif m in sel:
                    w = _gate_value(gate, s[0, h, t, m])
                else:
                    continue
                e = w * math.exp(scale * float(q[0, h, t] @ k[0, 0, j]))
                num += e * v[0, 0, j]
                den += e
            np.testing.assert_allclose(o[0, h, t], num / den, rtol=1e-12, atol=1e-13)
            assert abs(lse[0, h, t] - math.log(den)) < 1e-12


@pytest.mark.parametrize("gate", ["sigmoid", "raw"])
@pytest.mark.parametrize("sparse", [False, True])
def test_gate_variant_finite_differences(gate, sparse):
    """Central differences of L = sum(dO * o) in fp64 match dq, dk, dv and ds
    for the sigmoid and raw-logit gates."""
    block, D, N, Hq, Hkv = 4, 4, 20, 2, 1
    q, k, v, do, s = rand_problem(71, Hq=Hq, Hkv=Hkv, N=N, D=D, block=block)
    scale = 0.7
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, 2) if sparse else None
    dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, idx, block, scale, gate=gate)
    eps = 1e-6
    r = rng(9)

    def loss():
        o, _, _ = orc.gated_attention_forward(q, k, v, s, idx, block, scale, gate=gate)
        return float(np.sum(o * do))

    def fd(arr, pos):
        a0 = arr[pos]
        arr[pos] = a0 + eps
        lp = loss()
        arr[pos] = a0 - eps
        lm = loss()
        arr[pos] = a0
        return (lp - lm) / (2 * eps)

    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for _ in range(8):
            pos = tuple(int(r.integers(0, n)) for n in arr.shape)
            assert abs(fd(arr, pos) - grad[pos]) < 1e-7 * max(1.0, abs(grad[pos]))
    for t in (6, 13, 19):
        for h in range(Hq):
            for m in range(s.shape[3]):
                pos = (0, h, t, m)
                assert abs(fd(s, pos) - ds[pos]) < 1e-7, (gate, pos, fd(s, pos), ds[pos])


@pytest.mark.parametrize("gate", ["sigmoid", "raw"])
def test_gate_variant_inner_gradient_closed_form(gate):
    """ds_m = dg_m^inner * dg/ds with the pages' inner-gate gradient
    dg_m = sum_{i in B_m} (p_i / g_m) dO.(v_i - o) (review "Why the Four Design
    Choices Matter", paper Eq. 5) and dg/ds = g (1 - g) for the sigmoid gate,
    e^s for the raw logit; p from the library softmax."""
    block, D, N = 8, 8, 40
    q, k, v, do, s = rand_problem(43, Hq=1, Hkv=1, N=N, D=D, block=block)
    scale = 0.5
    _, _, _, ds = orc.gated_attention_backward(q, k, v, do, s, None, block, scale, gate=gate)
    qt, kt, vt, st = (torch.tensor(x[0]) for x in (q, k, v, s))
    for t in (17, 30, 39):
        c = t // block
        g = torch.sigmoid(st[0, t, :c]) if gate == "sigmoid" else torch.exp(st[0, t, :c])
        z = torch.full((N,), float("-inf"), dtype=torch.float64)
        for j in range(t + 1):
            m = j // block
            z[j] = scale * qt[0, t] @ kt[0, j] + (torch.log(g[m]) if m < c else 0.0)
        p = torch.softmax(z, dim=0)
        o = p @ vt[0]
        dO = torch.tensor(do[0, 0, t])
        dg = torch.stack([(p[m * block:(m + 1) * block] / g[m] * ((vt[0, m * block:(m + 1) * block] - o) @ dO)).sum()
                          for m in range(c)])
        dgds = g * (1 - g) if gate == "sigmoid" else g
        np.testing.assert_allclose(ds[0, 0, t, :c], (dg * dgds).numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(ds[0, 0, t, c:], 0.0)


def test_gate_variants_reduce_to_plain_sparse_attention():
    """Raw logit s = 0 (gate 1) and a saturated sigmoid (s = 40) both give plain
    causal attention over the own block and the selected blocks: library
    attention with that mask."""
    block, D, N = 4, 6, 32
    q, k, v, do, s = rand_problem(81, Hq=2, Hkv=1, N=N, D=D, block=block)
    scale = 0.45
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, 3)
    mask = torch.zeros((N, N), dtype=torch.bool)
    for t in range(N):
        c = t // block
        for j in range(t + 1):
            m = j // block
            mask[t, j] = m == c or m in {int(x) for x in idx[0, 0, t] if 0 <= x < c}
    expect = causal_sdpa(torch.tensor(q[0]), torch.tensor(k[0]), torch.tensor(v[0]), scale,
                         mask=mask).numpy()
    o_raw = orc.gated_attention_forward(q, k, v, np.zeros_like(s), idx, block, scale, gate="raw")[0]
    o_sig = orc.gated_attention_forward(q, k, v, np.full_like(s, 40.0), idx, block, scale, gate="sigmoid")[0]
    np.testing.assert_allclose(o_raw[0], expect, atol=1e-12)
    np.testing.assert_allclose(o_sig[0], expect, atol=1e-12)


# ---------------------------------------------------------------------------
# The outer gate (the pages' gate-placement ablation): g = softmax(s) scales
# each block's value contribution after an ungated softmax
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("sparse", [False, True])
def test_outer_gate_forward_written_out(sparse):
    """o_t = sum_j g_{m(j)} e^{z_j} v_j / sum_j e^{z_j} over the attended keys, z
    with no bias, g = softmax of the row's history scores, own block g = 1."""
    block, D, N = 4, 5, 28
    q, k, v, do, s = rand_problem(91, Hq=2, Hkv=1, N=N, D=D, block=block)
    scale = 0.6
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, 2) if sparse else None
    o, lse, lse_s = orc.gated_attention_forward(q, k, v, s, idx, block, scale, gate="outer")
    for h in range(2):
        for t in range(N):
            c = t // block
            sel = set(range(c)) if idx is None else {int(m) for m in idx[0, 0, t] if 0 <= m < c}
            gate = np.exp(s[0, h, t, :c] - np.log(np.sum(np.exp(s[0, h, t, :c])))) if c else np.zeros(0)
            num = np.zeros(D)
            den = 0.0
            for j in range(t + 1):
                m = j // block
                if m != c and m not in sel:
                    continue
                e = math.exp(scale * float(q[0, h, t] @ k[0, 0, j]))
                num += (1.0 if m == c else gate[m]) * e * v[0, 0, j]
                den += e
            np.testing.assert_allclose(o[0, h, t], num / den, rtol=1e-12, atol=1e-13)
            assert abs(lse[0, h, t] - math.log(den)) < 1e-12
            if c:
                assert abs(lse_s[0, h, t] - math.log(np.sum(np.exp(s[0, h, t, :c])))) < 1e-12


@pytest.mark.parametrize("sparse", [False, True])
def test_outer_gate_finite_differences(sparse):
    block, D, N, Hq, Hkv = 4, 4, 20, 2, 1
    q, k, v, do, s = rand_problem(73, Hq=Hq, Hkv=Hkv, N=N, D=D, block=block)
    scale = 0.7
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, 2) if sparse else None
    dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, idx, block, scale, gate="outer")
    eps = 1e-6
    r = rng(19)

    def loss():
        o, _, _ = orc.gated_attention_forward(q, k, v, s, idx, block, scale, gate="outer")
        return float(np.sum(o * do))

    def fd(arr, pos):
        a0 = arr[pos]
        arr[pos] = a0 + eps
        lp = loss()
        arr[pos] = a0 - eps
        lm = loss()
        arr[pos] = a0
        return (lp - lm) / (2 * eps)

    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for _ in range(8):
            pos = tuple(int(r.integers(0, n)) for n in arr.shape)
            assert abs(fd(arr, pos) - grad[pos]) < 1e-7 * max(1.0, abs(grad[pos]))
    for t in (6, 13, 19):
        for h in range(Hq):
            for m in range(s.shape[3]):
                pos = (0, h, t, m)
                assert abs(fd(s, pos) - ds[pos]) < 1e-7, (pos, fd(s, pos), ds[pos])


def test_outer_gate_gradient_closed_form():
    """ds through the pages' outer-gate gradient dg_m = sum_{i in B_m} p_i dO.v_i
    (review "Why the Four Design Choices Matter", paper Eq. 5), p the library
    softmax of the ungated logits, pushed through the library softmax's
    backward to the scores."""
    block, D, N = 8, 8, 40
    q, k, v, do, s = rand_problem(47, Hq=1, Hkv=1, N=N, D=D, block=block)
    scale = 0.5
    _, _, _, ds = orc.gated_attention_backward(q, k, v, do, s, None, block, scale, gate="outer")
    qt, kt, vt = (torch.tensor(x[0, 0]) for x in (q, k, v))
    for t in (17, 30, 39):
        c = t // block
        z = scale * (kt[:t + 1] @ qt[t])
        p = torch.softmax(z, dim=0)
        dO = torch.tensor(do[0, 0, t])
        dg = torch.stack([(p[m * block:(m + 1) * block] * (vt[m * block:(m + 1) * block] @ dO)).sum()
                          for m in range(c)])
        sv = torch.tensor(s[0, 0, t, :c], requires_grad=True)
        torch.softmax(sv, dim=0).backward(dg)
        np.testing.assert_allclose(ds[0, 0, t, :c], sv.grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(ds[0, 0, t, c:], 0.0)


def test_outer_gate_with_one_history_block_is_the_inner_gate():
    """With one history block g = 1, so placing it inside or outside the softmax
    gives the same output (rows of block 1)."""
    block, D, N = 8, 6, 16
    q, k, v, do, s = rand_problem(53, Hq=2, Hkv=1, N=N, D=D, block=block)
    o_out = orc.gated_attention_forward(q, k, v, s, None, block, 0.4, gate="outer")[0]
    o_in = orc.gated_attention_forward(q, k, v, s, None, block, 0.4)[0]
    np.testing.assert_allclose(o_out, o_in, atol=1e-13)


# ---------------------------------------------------------------------------
# The hard gate with a straight-through estimator (the pages' ranking ablation)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("topk", [0, 2])
def test_ste_gate_against_autograd(topk):
    """Library autograd with the straight-through trick: a multiplicative gate
    h = hard + g - g.detach() (hard: 1 on selected blocks and the own block, 0
    on dropped ones; g = softmax(s) over the history, 1 on the own block)
    inside o = sum h e^z v / sum h e^z.  Its forward is the hard gate's, its
    gradients are the oracle's, dropped blocks' ds included."""
    block, D, N = 4, 5, 28
    q, k, v, do, s = rand_problem(97, Hq=2, Hkv=1, N=N, D=D, block=block)
    scale = 0.6
    C = N // block
    idx = orc.topk_select(s.astype(np.float32), 2, np.arange(N)[None, :] // block, topk)
    o, lse, lse_s, dq, dk, dv, ds = orc.ste_gate_attention(q, k, v, do, s, idx, block, scale)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    st = torch.tensor(s, requires_grad=True)
    dot = torch.tensor(do)
    loss = 0.0
    for h in range(2):
        for t in range(N):
            c = t // block
            sel = {int(m) for m in idx[0, 0, t] if 0 <= m < c}
            gsoft = torch.softmax(st[0, h, t, :c], dim=0) if c else None
            z = scale * (kt[0, 0, :t + 1] @ qt[0, h, t])
            hk = []
            for j in range(t + 1):
                m = j // block
                if m == c:
                    hk.append(torch.tensor(1.0, dtype=torch.float64))
                else:
                    hard = 1.0 if m in sel else 0.0
                    hk.append(hard + gsoft[m] - gsoft[m].detach())
            hk = torch.stack(hk)
            w = hk * torch.exp(z - z.max())
            out = (w[:, None] * vt[0, 0, :t + 1]).sum(0) / w.sum()
            np.testing.assert_allclose(out.detach().numpy(), o[0, h, t], atol=1e-12)
            loss = loss + (out * dot[0, h, t]).sum()
    loss.backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(ds, st.grad.numpy(), atol=1e-11)
    assert np.any(ds[0, :, :, :][np.broadcast_to(np.arange(C)[None, None, :], ds.shape[1:]) < 3] != 0)


# ---------------------------------------------------------------------------
# Dense prefill
# ---------------------------------------------------------------------------

def test_causal_attention_is_library_causal_sdpa():
    """The prefill oracle against the library's causal attention (fp64), and
    against the gated forward at one history block (which is dense causal)."""
    r = rng(21)
    B, Hq, Hkv, N, D = 2, 4, 2, 37, 8
    q = r.standard_normal((B, Hq, N, D))
    k = r.standard_normal((B, Hkv, N, D))
    v = r.standard_normal((B, Hkv, N, D))
    o, lse = orc.causal_attention(q, k, v, 0.4)
    for b in range(B):
        ref = causal_sdpa(torch.tensor(q[b]), torch.tensor(k[b]), torch.tensor(v[b]), 0.4, is_causal=True)
        np.testing.assert_allclose(o[b], ref.numpy(), atol=1e-12)
        # lse by its definition through the library's logsumexp
        G = Hq // Hkv
        for h in range(Hq):
            z = 0.4 * torch.tensor(q[b, h]) @ torch.tensor(k[b, h // G]).T
            z = z.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
            np.testing.assert_allclose(lse[b, h], torch.logsumexp(z, dim=-1).numpy(), rtol=1e-12)
    # N = 2 b: every query has at most one history block, whose gate is 1
    block = 16
    q2, k2, v2 = q[:, :, : 2 * block], k[:, :, : 2 * block], v[:, :, : 2 * block]
    s = orc.block_scores(q2, orc.pool_block_keys(k2, block), block, 0.4, np.broadcast_to(np.arange(2 * block), (B, 2 * block)))
    og, lg, _ = orc.gated_attention_forward(q2, k2, v2, s, None, block, 0.4)
    o2, l2 = orc.causal_attention(q2, k2, v2, 0.4)
    np.testing.assert_allclose(og, o2, atol=1e-12)
    np.testing.assert_allclose(lg, l2, rtol=1e-12)
