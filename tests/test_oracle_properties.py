"""Property tests of the oracle over random tiny shapes (hypothesis, derandomized).

Each property ties the oracle to something other than itself, over shapes the
fixed pins do not reach: ragged N (a partial last block), every group size,
Top-K from 0 to beyond the history, tiny head dimensions.

- The SAS forward and all four gradients equal library attention with the SAS
  logits written as a float mask, differentiated by library autograd
  ([Blog] 方法核心: the SAS logits and the inner-gate gradient; [Review] "New
  Approach", Eq. 9; "Why the Four Design Choices Matter", log g = s - LSE(s)).
- The gate gradient sums to zero over each row's history and is proportional
  to g on the unselected blocks ([Blog] 方法核心, Fig. 4; [Review] Eq. 5).
- Decode equals library attention over the current block's keys up to the
  token and the selected history blocks, with no gate ([Review] "How It Works:
  A Concrete Walkthrough", Step 6), for ragged, idle and over-long lengths and
  for repeated or out-of-range idx entries.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from oracle import sas_oracle as orc  # noqa: E402

SETTINGS = settings(max_examples=30, deadline=None, derandomize=True)


@st.composite
def train_shapes(draw):
    block = draw(st.sampled_from([2, 4, 8]))
    C = draw(st.integers(1, 5))                  # complete blocks
    tail = draw(st.integers(0, block - 1))       # tokens of a partial last block
    Hkv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    D = draw(st.sampled_from([2, 4, 8]))
    topk = draw(st.one_of(st.none(), st.integers(0, C + 1)))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return block, C * block + tail, Hkv, G, D, topk, seed


def _sas_mask(s, sel, block, N):
    """Float mask [Hq, N, N] of the SAS logits: 0 on the own block up to the
    row, log_softmax(s) over the row's history on selected history blocks,
    -inf elsewhere (library log_softmax, so autograd reaches s)."""
    Hq, _, C = s.shape
    t = torch.arange(N)
    c = t // block
    hist = torch.arange(C)[None, :] < c[:, None]                      # [N, C]
    logg = torch.log_softmax(s.masked_fill(~hist, float("-inf")), dim=-1)
    logg = torch.where(hist, logg, torch.zeros((), dtype=s.dtype))
    logg = torch.cat([logg, torch.zeros(Hq, N, 1, dtype=s.dtype)], dim=-1)  # a column for the tail block
    kb = t // block                                                   # block of each key (C: the tail)
    per_key = logg[..., kb]
    selp = torch.cat([sel, torch.zeros(Hq, N, 1, dtype=torch.bool)], dim=-1)
    use = selp[..., kb] & (kb[None, :] < c[:, None])
    own = (kb[None, :] == c[:, None]) & (t[None, :] <= t[:, None])
    neg = torch.full((), float("-inf"), dtype=s.dtype)
    return torch.where(own, torch.zeros((), dtype=s.dtype), torch.where(use, per_key, neg))


def _selection(idx, Hq, G, N, C):
    sel = np.zeros((Hq, N, C), dtype=bool)
    if idx is None:
        sel[:] = True
        return sel
    for h in range(Hq):
        for t in range(N):
            for m in idx[0, h // G, t]:
                if 0 <= m < C:
                    sel[h, t, m] = True
    return sel


@SETTINGS
@given(train_shapes())
def test_forward_and_gradients_equal_library_autograd(shape):
    block, N, Hkv, G, D, topk, seed = shape
    Hq, C = Hkv * G, N // block
    r = np.random.default_rng(seed)
    q = r.standard_normal((1, Hq, N, D))
    k = r.standard_normal((1, Hkv, N, D))
    v = r.standard_normal((1, Hkv, N, D))
    do = r.standard_normal((1, Hq, N, D))
    s = r.standard_normal((1, Hq, N, C))
    scale = 1 / math.sqrt(D)
    pos = np.arange(N)[None, :]
    idx = None if topk is None else orc.topk_select(s.astype(np.float32), G, pos // block, topk)
    sel = _selection(idx, Hq, G, N, C)
    o, lse, _ = orc.gated_attention_forward(q, k, v, s, idx, block, scale)
    qt, kt, vt, sv = (torch.tensor(x[0], requires_grad=True) for x in (q, k, v, s))
    mask = _sas_mask(sv, torch.tensor(sel), block, N)
    kk, vv = kt.repeat_interleave(G, dim=0), vt.repeat_interleave(G, dim=0)
    out = F.scaled_dot_product_attention(qt, kk, vv, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(o[0], out.detach().numpy(), atol=1e-12)
    ref_lse = torch.logsumexp((qt @ kk.transpose(-1, -2)) * scale + mask, dim=-1)
    np.testing.assert_allclose(lse[0], ref_lse.detach().numpy(), atol=1e-12)
    (out * torch.tensor(do[0])).sum().backward()
    dq, dk, dv, ds = orc.gated_attention_backward(q, k, v, do, s, idx, block, scale)
    np.testing.assert_allclose(dq[0], qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk[0], kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv[0], vt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(ds[0], sv.grad.numpy(), atol=1e-11)


@SETTINGS
@given(train_shapes())
def test_gate_gradient_invariants(shape):
    block, N, Hkv, G, D, topk, seed = shape
    Hq, C = Hkv * G, N // block
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((1, h, N, D)) for h in (Hq, Hkv, Hkv))
    do = r.standard_normal((1, Hq, N, D))
    s = r.standard_normal((1, Hq, N, C))
    pos = np.arange(N)[None, :]
    idx = None if topk is None else orc.topk_select(s.astype(np.float32), G, pos // block, topk)
    sel = _selection(idx, Hq, G, N, C)
    _, _, _, ds = orc.gated_attention_backward(q, k, v, do, s, idx, block, 1 / math.sqrt(D))
    for h in range(Hq):
        for t in range(N):
            c = t // block
            row = ds[0, h, t]
            assert np.all(row[c:] == 0)
            if c == 0:
                continue
            assert abs(row[:c].sum()) <= 1e-12 * max(1.0, np.abs(row[:c]).sum())
            g = np.exp(s[0, h, t, :c] - np.logaddexp.reduce(s[0, h, t, :c]))
            off = ~sel[h, t, :c]
            if off.sum() >= 2:  # ds_m / g_m is the same on every unselected block
                ratio = row[:c][off] / g[off]
                assert np.ptp(ratio) <= 1e-9 * max(1.0, np.abs(ratio).max())


@st.composite
def decode_shapes(draw):
    block = draw(st.sampled_from([2, 4, 8]))
    C = draw(st.integers(1, 6))
    L = C * block + draw(st.integers(0, block - 1))   # capacity, possibly not a multiple of the block
    B = draw(st.integers(1, 3))
    Hkv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 4))
    D = draw(st.sampled_from([2, 4, 8]))
    lens = draw(st.lists(st.integers(-2, L + 3 * block), min_size=B, max_size=B))
    K = draw(st.integers(0, C + 2))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return block, L, B, Hkv, G, D, lens, K, seed


@SETTINGS
@given(decode_shapes())
def test_decode_equals_library_attention_over_the_selection(shape):
    block, L, B, Hkv, G, D, lens, K, seed = shape
    Hq = Hkv * G
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, D))
    kc = r.standard_normal((B, Hkv, L, D))
    vc = r.standard_normal((B, Hkv, L, D))
    lens = np.array(lens, dtype=np.int64)
    C = L // block
    # arbitrary entries: repeats, the current block, out-of-range and -1
    idx = r.integers(-2, C + 2, size=(B, Hkv, K)) if K > 0 else np.zeros((B, Hkv, 0), dtype=np.int64)
    scale = 1 / math.sqrt(D)
    o, lse = orc.sparse_decode(q, kc, vc, lens, idx, block, scale)
    for b in range(B):
        n = min(int(lens[b]), L)
        if n <= 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        pos = n - 1
        c = pos // block
        for g in range(Hkv):
            hist = {int(m) for m in idx[b, g] if 0 <= m < c}
            keys = [j for j in range(L) if (j // block == c and j <= pos) or (j // block in hist)]
            kt = torch.tensor(kc[b, g, keys])
            vt = torch.tensor(vc[b, g, keys])
            for h in range(g * G, (g + 1) * G):
                qt = torch.tensor(q[b, h])[None, None]
                ref = F.scaled_dot_product_attention(qt, kt[None], vt[None], scale=scale)[0, 0]
                np.testing.assert_allclose(o[b, h], ref.numpy(), atol=1e-12)
                np.testing.assert_allclose(lse[b, h], torch.logsumexp(kt @ torch.tensor(q[b, h]) * scale, 0).item(),
                                           atol=1e-12)
