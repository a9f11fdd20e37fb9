"""Plain fp64 CPU oracle for SAS gated block-sparse attention.

TEST INFRASTRUCTURE ONLY.  This module is imported by the test suite, by the
package's smoke check and by the benchmark's CPU-baseline leg; the product path
(the HIP library and its Python binding) never imports it, and it imports
nothing from the product path.  It is numpy only, works in float64 and favours
the most literal reading of the formulas over speed: every step writes out the
definition on whole matrices (one query head at a time), with no tiling, fusion
or reordering.

Pages it follows (the text of the web pages about the method):
  [Blog]   shibing624.github.io, "SAS：别再让稀疏注意力'抄作业'了，让语言模型
           损失直接教它怎么排序" -- sections 问题动机 (block-sparse attention
           formula), 方法核心 (the SAS formula, the gate g = softmax(s), the
           inner-gate gradient).
  [Review] jaehun.me, "SAS: Simple Attention Sparsification via End-to-End
           Optimization of Context Ranking" -- "Background" (paper Eq. 1-3),
           "New Approach" (paper Eq. 4 and Eq. 9), "Why the Four Design
           Choices Matter" (log g = s - LSE(s); paper Eq. 5), "How It Works:
           A Concrete Walkthrough" (worked example; paper Alg. 1 and Alg. 2),
           "Our Perspective" (pooling-based block summaries).

Readings where the pages are silent (each also listed in the design notes):
  * logits are scaled by `scale` (1/sqrt(D) in every workload); the selector
    score uses the same scale;
  * the current block of query t is block c(t) = t // b (causally masked);
    its history is blocks 0 .. c(t)-1; queries in block 0 have no history;
  * selection is per (query token, KV head): the fp32 scores of the group's
    query heads are summed in head-index order, and Top-K keeps exactly
    min(K, c) blocks, ordered by score descending, ties to the lower block
    index, -0.0 equal to +0.0, NaN ranked as -inf, rows padded with -1;
  * the gate softmax always runs over all history blocks (also at sparse
    scope); unselected history blocks receive -inf logits;
  * decode: the new token is already in the cache at position len-1; it
    attends to its own block plus the selected history blocks with no gate;
  * idx entries outside [0, c) are ignored and a repeated entry counts once;
  * gate activations other than the softmax (sigmoid, raw logit: the pages'
    ablation of the gate activation) keep everything else as it is: the own
    block's gate is 1, unselected history blocks get -inf, and with no
    normaliser an unselected block's ds is 0 and LSE_s is reported as 0;
  * the outer gate (the pages' gate-placement ablation) is g = softmax(s)
    multiplying each attended key's value contribution after a softmax of
    the ungated logits; `lse` is then the log-sum-exp of those logits.

Parity status: every function below is pinned by tests that do not re-type
its formula (library attention routines, autograd, finite differences,
closed forms, the worked example, brute force).  Whole-pipeline results at
bf16 have no error bound on the pages: that tolerance is a derived reading.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _logsumexp(x, axis=-1):
    """log(sum(exp(x))) along `axis`; an all -inf slice gives -inf."""
    x = _as64(x)
    m = np.max(x, axis=axis, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        out = np.log(np.sum(np.exp(x - m_safe), axis=axis, keepdims=True)) + m_safe
    return np.squeeze(out, axis=axis)


# ----------------------------------------------------------------------------
# a1 / a2: pooled block keys and selector scores
# ----------------------------------------------------------------------------

def pool_block_keys(k, block):
    """Mean-pooled key summary of every complete block.

    K̄[b,g,m,:] = (1/b) * sum_{j in B_m} K[b,g,j,:]   (pooling-based block
    summaries: [Review] "Our Perspective"; partition into blocks of b tokens:
    [Review] "Background", paper Eq. 3).
    k: [B, Hkv, L, D] -> [B, Hkv, L // block, D] float64.
    """
    k = _as64(k)
    B, H, L, D = k.shape
    C = L // block
    return k[:, :, : C * block].reshape(B, H, C, block, D).mean(axis=3)


def history_blocks(position, block):
    """Number of complete history blocks c = position // b of a query at `position`."""
    return np.asarray(position) // block


def block_scores(q, kbar, block, scale, positions):
    """Selector scores s[b,h,t,m] = scale * q[b,h,t] . K̄[b,g(h),m] for m < c(t).

    Entries with m >= c(t) (the current block and the future) are -inf.
    q: [B, Hq, Nq, D]; kbar: [B, Hkv, C, D]; positions: [B, Nq] integer
    position of each query.  Query head h reads KV head h // (Hq/Hkv).
    Returns float64 [B, Hq, Nq, C].  ([Review] "Background", paper Eq. 3:
    one relevance score per history block.)
    """
    q = _as64(q)
    kbar = _as64(kbar)
    B, Hq, Nq, D = q.shape
    Hkv, C = kbar.shape[1], kbar.shape[2]
    G = Hq // Hkv
    c = history_blocks(positions, block)  # [B, Nq]
    valid = np.arange(C)[None, :] < c[:, :, None]  # [B, Nq, C]
    s = np.full((B, Hq, Nq, C), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            full = scale * (q[b, h] @ kbar[b, h // G].T)
            s[b, h] = np.where(valid[b], full, NEG_INF)
    return s


def selector_backward(q, k, ds, block, scale, kbar=None):
    """Gradient of the mean-pool selector score for an upstream ds = dL/ds.

    The selector score is s[b,h,t,m] = scale * q[b,h,t] . K̄[b,g(h),m] for
    history blocks m < c(t), with K̄ the mean of each complete block of K
    (block_scores and pool_block_keys above).  This is the last link of the
    gradient path from the output through the gate to the selector ([Review]
    "A Concrete Walkthrough", Step 5; pooling-based block summaries: [Review]
    "Our Perspective").  Entries m >= c(t) of ds are not part of s and are
    ignored.  By the chain rule through the bilinear score and the mean:
      dq[b,h,t]    = scale * sum_{m < c(t)} ds[b,h,t,m] K̄[b,g(h),m]
      dK̄[b,g,m]    = scale * sum_{h of g} sum_{t: m < c(t)} ds[b,h,t,m] q[b,h,t]
      dk[b,g,j]    = dK̄[b,g,j // b] / b for j in a complete block, else 0.
    q: [B, Hq, N, D]; k: [B, Hkv, N, D]; ds: [B, Hq, N, C] with C = N // block.
    kbar: the pooled keys to use for dq when they are held rounded (e.g. in
    bf16); None pools k.
    Returns float64 dq [B, Hq, N, D], dkbar [B, Hkv, C, D], dk [B, Hkv, N, D].
    """
    q = _as64(q)
    ds = _as64(ds)
    kbar = pool_block_keys(k, block) if kbar is None else _as64(kbar)
    B, Hq, N, D = q.shape
    Hkv, C = kbar.shape[1], kbar.shape[2]
    G = Hq // Hkv
    c = history_blocks(np.arange(N), block)
    valid = np.arange(C)[None, :] < c[:, None]  # [N, C]
    dq = np.zeros_like(q)
    dkbar = np.zeros((B, Hkv, C, D))
    for b in range(B):
        for h in range(Hq):
            dsm = np.where(valid, ds[b, h, :, :C], 0.0)
            dq[b, h] = scale * (dsm @ kbar[b, h // G])
            dkbar[b, h // G] += scale * (dsm.T @ q[b, h])
    dk = np.zeros((B, Hkv, N, D))
    dk[:, :, : C * block] = np.repeat(dkbar / block, block, axis=2)
    return dq, dkbar, dk


def selector_dq_rows(kbar, ds, block, scale, b, h, rows):
    """dq of selected query rows of head h in batch b: the row-local part of
    `selector_backward`, scale * sum_{m < c(t)} ds[t,m] K̄_m.  kbar: [B, Hkv, C, D]
    (pooled keys as held); ds: [B, Hq, N, C]; Hq is read from ds.  Returns [R, D]."""
    Hq, C = ds.shape[1], kbar.shape[2]
    G = Hq // kbar.shape[1]
    rows = np.asarray(rows)
    c = history_blocks(rows, block)
    dsr = np.where(np.arange(C)[None, :] < c[:, None], _as64(ds[b, h][rows][:, :C]), 0.0)
    return scale * (dsr @ _as64(kbar[b, h // G]))


def selector_dkbar_blocks(q, ds, block, scale, b, g, G, blocks):
    """dK̄ of selected blocks of KV head g in batch b (G query heads per KV
    head): the block-local part of `selector_backward`, scale * sum over the
    group's heads and the queries t with m < c(t), i.e. t >= (m+1) b, of
    ds[t,m] q_t.  q: [B, Hq, N, D]; ds: [B, Hq, N, C].  Returns [M, D]."""
    D = q.shape[3]
    out = np.zeros((len(blocks), D))
    for i, m in enumerate(blocks):
        t0 = (int(m) + 1) * block
        for h in range(g * G, (g + 1) * G):
            out[i] += scale * (_as64(ds[b, h, t0:, m]) @ _as64(q[b, h, t0:]))
    return out


def group_sum_scores(scores_f32, heads_per_row):
    """fp32 sum of the scores of each KV head's query heads, in head-index order.

    scores_f32: float32 [B, Hkv*heads_per_row, Nq, C] -> float32 [B, Hkv, Nq, C],
    u = ((s_h0 + s_h1) + s_h2) + ... with every addition rounded to fp32.
    """
    s = np.asarray(scores_f32, dtype=np.float32)
    B, H, Nq, C = s.shape
    s = s.reshape(B, H // heads_per_row, heads_per_row, Nq, C)
    u = s[:, :, 0].copy()
    for i in range(1, heads_per_row):
        u = (u + s[:, :, i]).astype(np.float32)
    return u


# ----------------------------------------------------------------------------
# a3 / a7: hard Top-K block selection
# ----------------------------------------------------------------------------

def topk_select(scores_f32, heads_per_row, num_candidates, topk):
    """Hard Top-K over each row's history blocks ([Review] "Background", paper
    Eq. 3; inference I = Top-K(s, K): "A Concrete Walkthrough", Step 6).

    scores_f32: float32 [B, Hkv*heads_per_row, Nq, C].
    num_candidates: int [B, Nq], the row's c (only blocks m < c compete).
    Returns int32 [B, Hkv, Nq, topk]: the min(topk, c) best blocks by the fp32
    group-summed score, descending, ties to the lower index; -0.0 counts as
    +0.0 and NaN as -inf; the remaining slots hold -1.
    """
    u = group_sum_scores(scores_f32, heads_per_row)
    u = np.where(np.isnan(u), np.float32(-np.inf), u)
    u = np.where(u == 0, np.float32(0.0), u)  # -0.0 -> +0.0
    B, Hkv, Nq, C = u.shape
    c = np.asarray(num_candidates).reshape(B, 1, Nq, 1)
    m = np.broadcast_to(np.arange(C), u.shape)
    # Blocks that do not compete sort after every candidate: lexsort orders
    # by the last key first (not-a-candidate flag), then -score, then index.
    not_candidate = (m >= c).astype(np.int8)
    order = np.lexsort((m, -u.astype(np.float64), not_candidate), axis=-1)
    out = np.full((B, Hkv, Nq, topk), -1, dtype=np.int32)
    take = min(topk, C)
    out[..., :take] = order[..., :take]
    slot = np.arange(topk).reshape(1, 1, 1, topk)
    out = np.where(slot < np.minimum(c, topk), out, -1)
    return out.astype(np.int32)


# ----------------------------------------------------------------------------
# a4 / a5: SAS gated attention, forward and backward
# ----------------------------------------------------------------------------

def _selection_mask(idx_row_sets, c, C):
    """Boolean [rows, C]: block m is selected for the row (m < c only)."""
    rows = len(c)
    sel = np.zeros((rows, C), dtype=bool)
    for r in range(rows):
        for m in idx_row_sets[r]:
            m = int(m)
            if 0 <= m < c[r]:
                sel[r, m] = True
    return sel


GATES = ("softmax", "sigmoid", "raw", "outer")


def _log_sigmoid(x):
    """log(1 / (1 + e^-x)) = -log(1 + e^-x), without overflow."""
    return -np.logaddexp(0.0, -x)


def _row_terms(s_rows, idx_rows, rows, block, N, C, gate="softmax"):
    """Per-row gate terms shared by forward and backward.

    For each query t in `rows`: c(t), LSE_s(t) over its history blocks,
    beta[t,m] = log g_m, the selection mask, and the additive bias over all N
    keys:
        0          own block, key j <= t   (current block gate is 1, log 1 = 0)
        beta[t,m]  key j in a selected history block m
        -inf       any other key (unselected history, the future)
    The gate activation ([Review] "Why the Four Design Choices Matter", gate
    activation; [Blog] 方法核心, the ablation table's gate-activation row):
        softmax  g = softmax(s) over the history, beta = s - LSE_s (the SAS
                 gate: [Blog] 方法核心, [Review] "New Approach", paper Eq. 4)
        sigmoid  g = sigmoid(s) per block, beta = log sigmoid(s)
        raw      the logit injected as it is, beta = s (g = e^s)
        outer    g = softmax(s) as for the SAS gate, placed outside the
                 softmax ([Review] "Why the Four Design Choices Matter", gate
                 placement): the logits take no bias (0 on the own block and
                 the gated history, -inf elsewhere) and the gate scales each
                 key's value contribution instead (gk below).
    Only the softmax-normalised gates (softmax, outer) have LSE_s; the others
    report LSE_s = 0.  gk[t,j] is the factor on key j's value contribution:
    the outer gate's g of the key's block (1 on the own block, 0 on keys the
    row does not attend); 1 for the gates inside the softmax.
    """
    if gate not in GATES:
        raise ValueError(f"unknown gate {gate!r}")
    rows = np.asarray(rows)
    c = rows // block
    hist = np.arange(C)[None, :] < c[:, None]  # [R, C]
    s_hist = np.where(hist, _as64(s_rows), NEG_INF)
    if gate in ("softmax", "outer"):
        lse_s = _logsumexp(s_hist, axis=-1)  # -inf when c == 0
        with np.errstate(invalid="ignore"):
            beta = np.where(hist, s_hist - lse_s[:, None], NEG_INF)
    else:
        lse_s = np.zeros(len(rows))
        beta = np.where(hist, _log_sigmoid(s_hist) if gate == "sigmoid" else s_hist, NEG_INF)
    if idx_rows is None:  # full scope: every history block is gated
        sel = hist.copy()
    else:
        sel = _selection_mask(idx_rows, c, C)
    key = np.arange(N)
    key_block = key // block
    own = (key_block[None, :] == c[:, None]) & (key[None, :] <= rows[:, None])
    kb = np.minimum(key_block, C - 1)
    hist_key = (key_block[None, :] < c[:, None]) & np.take_along_axis(
        sel, np.broadcast_to(kb, (len(rows), N)), axis=1)
    beta_key = np.take_along_axis(beta, np.broadcast_to(kb, (len(rows), N)), axis=1)
    if gate == "outer":
        bias = np.where(own | hist_key, 0.0, NEG_INF)
        gk = np.where(own, 1.0, np.where(hist_key, np.exp(np.where(hist_key, beta_key, 0.0)), 0.0))
    else:
        bias = np.where(own, 0.0, np.where(hist_key, beta_key, NEG_INF))
        gk = np.ones((len(rows), N))
    return c, lse_s, beta, sel, bias, gk


def _head_rows(q, k, v, s, idx, b, h, G, block, scale, rows, gate="softmax"):
    N = k.shape[2]
    C = s.shape[3]
    g = h // G
    idx_rows = None if idx is None else [idx[b, g, t] for t in rows]
    c, lse_s, beta, sel, bias, gk = _row_terms(s[b, h, rows], idx_rows, rows, block, N, C, gate)
    z = scale * (_as64(q[b, h, rows]) @ _as64(k[b, g]).T) + bias
    lse = _logsumexp(z, axis=-1)
    p = np.exp(z - lse[:, None])
    return c, lse_s, beta, sel, p, lse, gk


def _block_sums(x, block, C):
    """[R, N] -> [R, C]: sums over the keys of each block."""
    out = np.zeros((x.shape[0], C))
    for m in range(C):
        out[:, m] = x[:, m * block:(m + 1) * block].sum(axis=1)
    return out


def _row_backward(p, gk, doh, vh, sel, beta, s_rows, c, block, gate):
    """dz [R,N] and ds [R,C] of a head's rows: with w = gk p the weights on v,
    o = w v, dP = dO v^T, Delta = dO . o and dz = p (gk dP - Delta).  Gates
    inside the softmax: dbeta = the dz sum of each selected block, ds by
    `_gate_ds`.  The outer gate: dg_m = sum_{i in B_m} p_i dP_i (the pages'
    outer-gate gradient, [Review] "Why the Four Design Choices Matter", paper
    Eq. 5), ds = g (dg - sum_m' g dg), i.e. the softmax gate's rule applied to
    g dg."""
    C = sel.shape[1]
    o = (gk * p) @ vh
    delta = np.sum(doh * o, axis=-1)
    dp = doh @ vh.T
    dz = p * (gk * dp - delta[:, None])
    if gate == "outer":
        dbeta = np.where(sel, _block_sums(gk * p * dp, block, C), 0.0)
        return dz, _gate_ds("softmax", dbeta, beta, s_rows, c)
    dbeta = np.where(sel, _block_sums(dz, block, C), 0.0)
    return dz, _gate_ds(gate, dbeta, beta, s_rows, c)


def _gate_ds(gate, dbeta, beta, s_rows, c):
    """ds from dbeta (the dz sum of each selected history block, 0 otherwise)
    by the chain rule through beta = log g(s), zero outside the history:
        softmax  ds = dbeta - g * sum_m' dbeta      (log g = s - LSE(s))
        sigmoid  ds = dbeta * (1 - sigmoid(s))      (d log sigmoid(s) / ds)
        raw      ds = dbeta                         (beta = s)
    """
    C = dbeta.shape[1]
    hist = np.arange(C)[None, :] < c[:, None]
    if gate == "softmax":
        g = np.where(hist, np.exp(np.where(hist, beta, 0.0)), 0.0)
        return np.where(hist, dbeta - g * dbeta.sum(axis=1, keepdims=True), 0.0)
    if gate == "sigmoid":
        one_minus = np.exp(_log_sigmoid(-np.where(hist, _as64(s_rows), 0.0)))
        return np.where(hist, dbeta * one_minus, 0.0)
    return np.where(hist, dbeta, 0.0)


def gated_attention_forward(q, k, v, s, idx, block, scale, rows=None, gate="softmax"):
    """SAS forward o = softmax(q K_S^T * scale + log g_S) V_S
    ([Blog] 方法核心 and [Review] "New Approach", paper Eq. 9); `gate` picks the
    gate activation (see `_row_terms`).

    q: [B,Hq,N,D]; k, v: [B,Hkv,N,D]; s: [B,Hq,N,C] selector scores;
    idx: None (full scope: all history blocks gated) or int [B,Hkv,N,K]
    (sparse scope: only the selected history blocks take part).
    rows: optional list of query positions to evaluate (default: all).
    Returns (o [B,Hq,R,D], lse [B,Hq,R], lse_s [B,Hq,R]) in float64, where lse
    is the log-sum-exp of the biased logits and lse_s that of the row's
    history scores (-inf for rows without history).
    """
    B, Hq, N, D = q.shape
    G = Hq // k.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    R = len(rows)
    o = np.zeros((B, Hq, R, D))
    lse = np.zeros((B, Hq, R))
    lse_s = np.zeros((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            _, ls, _, _, p, l, gk = _head_rows(q, k, v, s, idx, b, h, G, block, scale, rows, gate)
            o[b, h] = (gk * p) @ _as64(v[b, h // G])
            lse[b, h] = l
            lse_s[b, h] = ls
    return o, lse, lse_s


def gated_attention_backward(q, k, v, do, s, idx, block, scale, gate="softmax"):
    """Gradients of L = sum(dO * o) for the SAS forward, with s held as an input.

    Returns (dq, dk, dv, ds) in float64.  dq, dk, dv are the partial
    derivatives of the attention at fixed s (dk, dv summed over the query
    heads that share a KV head).  ds is the selector-score gradient through
    the log-softmax gate: with dbeta[t,m] = sum_{j in B_m} dz[t,j] for
    selected m (0 otherwise) and g = softmax(s) over the history,
        ds[t,m] = dbeta[t,m] - g[t,m] * sum_{m' in H(t)} dbeta[t,m'],
    zero outside the history.  dbeta is g_m times the inner-gate gradient of
    [Blog] 方法核心 / [Review] "Why the Four Design Choices Matter" (paper
    Eq. 5); the second term is the chain rule through log g = s - LSE(s).
    The sigmoid and raw gates take their own chain rule (`_gate_ds`).
    The recomputed forward is this oracle's own (exact o and softmax).
    """
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    C = s.shape[3]
    rows = np.arange(N)
    dq = np.zeros((B, Hq, N, D))
    dk = np.zeros((B, Hkv, N, D))
    dv = np.zeros((B, Hkv, N, D))
    ds = np.zeros((B, Hq, N, C))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            c, _, beta, sel, p, _, gk = _head_rows(q, k, v, s, idx, b, h, G, block, scale, rows, gate)
            qh, kh, vh, doh = _as64(q[b, h]), _as64(k[b, g]), _as64(v[b, g]), _as64(do[b, h])
            dz, ds[b, h] = _row_backward(p, gk, doh, vh, sel, beta, s[b, h], c, block, gate)
            dq[b, h] = scale * (dz @ kh)
            dk[b, g] += scale * (dz.T @ qh)
            dv[b, g] += (gk * p).T @ doh
    return dq, dk, dv, ds


def row_gradients(q, k, v, do, s, idx, block, scale, b, h, rows, gate="softmax"):
    """dq and ds of selected query rows (row-local parts of the backward).

    Same definitions as `gated_attention_backward`, evaluated only for the
    query positions in `rows` of head h in batch b.  Returns (dq [R,D], ds [R,C]).
    """
    Hq = q.shape[1]
    G = Hq // k.shape[1]
    C = s.shape[3]
    g = h // G
    rows = np.asarray(rows)
    c, _, beta, sel, p, _, gk = _head_rows(q, k, v, s, idx, b, h, G, block, scale, rows, gate)
    vh, kh, doh = _as64(v[b, g]), _as64(k[b, g]), _as64(do[b, h, rows])
    dz, ds = _row_backward(p, gk, doh, vh, sel, beta, s[b, h, rows], c, block, gate)
    dq = scale * (dz @ kh)
    return dq, ds


def key_gradients(q, k, v, do, s, idx, block, scale, b, g, keys, row_chunk=1024, rows=None,
                  gate="softmax"):
    """dk and dv of selected keys of KV head g in batch b.

    dk[j] = scale * sum_{h in group(g)} sum_t dz[h,t,j] q[h,t];
    dv[j] = sum_{h in group(g)} sum_t gk p[h,t,j] dO[h,t]; the sums run over every
    query row (rows that do not attend key j contribute p = dz = 0), or over
    `rows` when given, which must then hold every row that attends the keys.
    Rows are visited in chunks only to bound memory; each row is computed
    exactly as in `gated_attention_backward`.  Returns (dk [J,D], dv [J,D]).
    """
    B, Hq, N, D = q.shape
    G = Hq // k.shape[1]
    keys = np.asarray(keys)
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    kmin = int(keys.min())
    all_rows = np.arange(kmin, N) if rows is None else np.asarray(rows)
    for h in range(g * G, (g + 1) * G):
        for r0 in range(0, len(all_rows), row_chunk):
            rows = all_rows[r0:r0 + row_chunk]
            _, _, _, _, p, _, gk = _head_rows(q, k, v, s, idx, b, h, G, block, scale, rows, gate)
            vh = _as64(v[b, g])
            doh = _as64(do[b, h, rows])
            o = (gk * p) @ vh
            delta = np.sum(doh * o, axis=-1)
            pk, gkk = p[:, keys], gk[:, keys]
            dz = pk * (gkk * (doh @ vh[keys].T) - delta[:, None])
            dk += scale * (dz.T @ _as64(q[b, h, rows]))
            dv += (gkk * pk).T @ doh
    return dk, dv


def ste_gate_attention(q, k, v, do, s, idx, block, scale):
    """The hard gate with a straight-through estimator ([Review] "Why the Four
    Design Choices Matter", ranking preservation; [Blog] 方法核心, the ablation
    table's hard-gate row), read as: the forward is plain block-sparse
    attention over the own block and the selected blocks (hard gate 1 there,
    0 on dropped blocks, normalised over that set S only); dq, dk, dv are its
    gradients; and the gate gradient of every history block m, selected or
    dropped, is that of a multiplicative gate at its hard value,
        dh_m = sum_{i in B_m} p_i dO.(v_i - o),  p_i = exp(z_i - LSE_S),
    (for a dropped block p_i is the weight the pages describe as unbounded),
    passed straight through to the soft gate g = softmax(s):
        ds_m = g_m (dh_m - sum_m' g_m' dh_m').
    Returns (o, lse, lse_s, dq, dk, dv, ds), lse = LSE_S and lse_s = LSE(s)
    over the history."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    C = s.shape[3]
    zero = np.zeros_like(_as64(s))
    o, lse, _ = gated_attention_forward(q, k, v, zero, idx, block, scale, gate="raw")
    dq, dk, dv, _ = gated_attention_backward(q, k, v, do, zero, idx, block, scale, gate="raw")
    rows = np.arange(N)
    c = rows // block
    hist = np.arange(C)[None, :] < c[:, None]
    lse_s = np.zeros((B, Hq, N))
    ds = np.zeros((B, Hq, N, C))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            z = scale * (_as64(q[b, h]) @ _as64(k[b, g]).T)
            p = np.exp(z - lse[b, h][:, None])          # exp(z_i - LSE_S), every key
            p = np.where(np.arange(N)[None, :] <= rows[:, None], p, 0.0)
            dpd = _as64(do[b, h]) @ _as64(v[b, g]).T - np.sum(_as64(do[b, h]) * o[b, h], axis=-1)[:, None]
            dh = np.where(hist, _block_sums(p * dpd, block, C), 0.0)
            s_hist = np.where(hist, _as64(s[b, h]), NEG_INF)
            ls = _logsumexp(s_hist, axis=-1)
            lse_s[b, h] = ls
            with np.errstate(invalid="ignore"):
                gs = np.where(hist, np.exp(s_hist - ls[:, None]), 0.0)
            ds[b, h] = np.where(hist, gs * (dh - np.sum(gs * dh, axis=1, keepdims=True)), 0.0)
    return o, lse, lse_s, dq, dk, dv, ds


# ----------------------------------------------------------------------------
# Dense prefill (inference, no gate)
# ----------------------------------------------------------------------------

def causal_attention(q, k, v, scale):
    """Plain causal attention of a prompt, no gate: o_t = softmax over j <= t of
    scale * q_t . k_j, times v ([Blog] 问题动机, attention over the full
    context; [Blog] 方法核心, kernel paragraph: the serving path prefills
    densely and decodes sparsely).

    q: [B, Hq, N, D]; k, v: [B, Hkv, N, D]; query head h reads KV head h // G.
    Returns (o [B,Hq,N,D], lse [B,Hq,N]) in float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, N, D = q.shape
    G = Hq // k.shape[1]
    o = np.zeros((B, Hq, N, D))
    lse = np.zeros((B, Hq, N))
    future = np.triu(np.ones((N, N), dtype=bool), k=1)
    for b in range(B):
        for h in range(Hq):
            z = scale * (q[b, h] @ k[b, h // G].T)
            z[future] = NEG_INF
            l = _logsumexp(z, axis=-1)
            o[b, h] = np.exp(z - l[:, None]) @ v[b, h // G]
            lse[b, h] = l
    return o, lse


# ----------------------------------------------------------------------------
# a8: sparse decode attention (inference, no gate)
# ----------------------------------------------------------------------------

def sparse_decode(q, k_cache, v_cache, cache_len, idx, block, scale):
    """One decode step per sequence: o = softmax(scale * q K_S^T) V_S over
    S = current block ∪ selected history blocks, with no gate
    ([Blog] 问题动机 block-sparse attention formula; [Review] "Background",
    paper Eq. 2, and "A Concrete Walkthrough", Step 6 / paper Alg. 2).

    q: [B, Hq, D]; caches: [B, Hkv, L_max, D]; cache_len: [B] (the new token
    sits at position len-1); idx: int [B, Hkv, K] (entries outside [0, c)
    ignored, repeats counted once) or None for dense decode over every
    cached position.  A length <= 0 marks an idle sequence (o = 0, lse = -inf)
    and a length above L_max counts as L_max (readings: the pages describe
    only live sequences).  Returns (o [B,Hq,D], lse [B,Hq]) in float64.
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    L = k_cache.shape[2]
    for b in range(B):
        n = min(int(cache_len[b]), L)  # lengths above the capacity count as the capacity
        if n <= 0:  # idle sequence: no query; output 0 and lse -inf
            lse[b] = -np.inf
            continue
        pos = n - 1
        c = pos // block
        if idx is None:
            keys_by_g = [np.arange(pos + 1)] * Hkv
        else:
            keys_by_g = []
            for g in range(Hkv):
                blocks = sorted({int(m) for m in idx[b, g] if 0 <= int(m) < c})
                parts = [np.arange(m * block, (m + 1) * block) for m in blocks]
                parts.append(np.arange(c * block, pos + 1))
                keys_by_g.append(np.concatenate(parts))
        for h in range(Hq):
            g = h // G
            keys = keys_by_g[g]
            kk = _as64(k_cache[b, g, keys])
            vv = _as64(v_cache[b, g, keys])
            z = scale * (kk @ _as64(q[b, h]))
            l = _logsumexp(z)
            o[b, h] = np.exp(z - l) @ vv
            lse[b, h] = l
    return o, lse


def decode_scores(q, kbar, cache_len, L_max, block, scale, group_sum):
    """Decode-mode selector scores for one new token per sequence
    ([Review] "A Concrete Walkthrough", Step 6 / paper Alg. 2: score the
    history blocks of the new token; [Review] "Background", paper Eq. 3).

    q: [B, Hq, D]; kbar: [B, Hkv, C, D] with C = L_max // block; L_max is the
    cache capacity.  Lengths are read exactly as in `sparse_decode`: a length
    above L_max counts as L_max, and the query sits at position len-1, so the
    blocks m < (len-1)//b compete; an idle sequence (len <= 0) has none.
    group_sum=False: float64 [B, Hq, C]; group_sum=True: float32 [B, Hkv, C],
    the fp32 sum (head-index order) of each head's score rounded to fp32.
    Non-candidates hold -inf (the current block included).
    """
    B, Hq, D = q.shape
    lens = np.minimum(np.asarray(cache_len), int(L_max))  # as sparse_decode
    pos = (lens - 1).reshape(B, 1)
    s = block_scores(np.asarray(q)[:, :, None, :], kbar, block, scale, np.maximum(pos, 0))[:, :, 0, :]
    s[(lens <= 0)] = NEG_INF  # idle: no candidates
    if not group_sum:
        return s
    G = Hq // kbar.shape[1]
    return group_sum_scores(s.astype(np.float32)[:, :, None, :], G)[:, :, 0, :]


def decode_candidates(cache_len, L_max, block):
    """Number of history blocks each decode query ranks: (min(len, L_max)-1)//b,
    0 for an idle sequence (the readings of `sparse_decode`)."""
    lens = np.minimum(np.asarray(cache_len), int(L_max))
    return np.where(lens > 0, (np.maximum(lens, 1) - 1) // block, 0)
