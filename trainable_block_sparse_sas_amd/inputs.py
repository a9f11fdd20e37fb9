"""Seeded synthetic inputs and the workload table.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic, so both the HIP path (via the tests and the benchmark)
and the CPU oracle can consume the very same tensors.

Workloads (shapes of the models the pages train and serve: Qwen3-4B/8B/14B
attention layers, block size 64, training at 32K tokens with Top-K 32,
decode at 128K and 512K tokens):

  0  tiny-f32-full     fp32, B1, Hq2/Hkv1, D64, N512, b64, full scope
  1  train-8k-full     bf16, B1, Hq32/Hkv8, D128, N8192, b64, full scope
  2  train-32k-sparse  bf16, B1, Hq32/Hkv8, D128, N32768, b64, Top-K 32
  3  decode-128k-b8    bf16, B8, Hq32/Hkv8, D128, cache 131072, b64, Top-K 16
  4  decode-512k-b1    bf16, B1, Hq40/Hkv8, D128, cache 524288, b64, Top-K 32

Recipe: one torch.Generator seeded with 1000 + workload index on the device
the tensors live on; draws in order q, k, v, dO (training) or q, k, v, then
the shifted blocks and their directions (decode); values are drawn in fp32
from N(0, 1) and cast once to the workload dtype.  Decode caches give 1% of
the blocks of every (sequence, KV head) a +3 shift along a random unit
direction (separate directions for K and V), so that selection is not
trivial.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "train" or "decode"
    dtype: str  # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    N: int  # training sequence length, or decode cache length
    block: int = 64
    topk: Optional[int] = None  # None: full scope (training) / dense (decode)
    index: int = -1
    extra: dict = field(default_factory=dict)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def C(self):
        return self.N // self.block

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny-f32-full", "train", "f32", 1, 2, 1, 64, 512, 64, None, 0),
    Workload("train-8k-full", "train", "bf16", 1, 32, 8, 128, 8192, 64, None, 1),
    Workload("train-32k-sparse", "train", "bf16", 1, 32, 8, 128, 32768, 64, 32, 2),
    Workload("decode-128k-b8", "decode", "bf16", 8, 32, 8, 128, 131072, 64, 16, 3),
    Workload("decode-512k-b1", "decode", "bf16", 1, 40, 8, 128, 524288, 64, 32, 4),
]


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device, dtype):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def training_inputs(w: Workload, device="cpu", seed=None):
    """q [B,Hq,N,D], k, v [B,Hkv,N,D], dO [B,Hq,N,D], all N(0,1) in the workload dtype."""
    seed = 1000 + w.index if seed is None else seed
    gen = generator(seed, device)
    dt = w.torch_dtype
    q = _randn((w.B, w.Hq, w.N, w.D), gen, device, dt)
    k = _randn((w.B, w.Hkv, w.N, w.D), gen, device, dt)
    v = _randn((w.B, w.Hkv, w.N, w.D), gen, device, dt)
    do = _randn((w.B, w.Hq, w.N, w.D), gen, device, dt)
    return q, k, v, do


def decode_inputs(w: Workload, device="cpu", seed=None, shift=3.0, shift_frac=0.01):
    """q [B,Hq,D]; k_cache, v_cache [B,Hkv,L,D]; cache_len [B] int32 (full caches).

    round(shift_frac * C) blocks per (sequence, KV head) are chosen without
    replacement; each gets `shift` times a random unit vector added to every
    token, drawn separately for K and V.
    """
    seed = 1000 + w.index if seed is None else seed
    gen = generator(seed, device)
    dt = w.torch_dtype
    L, C = w.N, w.N // w.block
    q = _randn((w.B, w.Hq, w.D), gen, device, dt)
    k = torch.randn((w.B, w.Hkv, L, w.D), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((w.B, w.Hkv, L, w.D), generator=gen, device=device, dtype=torch.float32)
    n_shift = int(round(shift_frac * C))
    if n_shift > 0 and shift != 0.0:
        for b in range(w.B):
            for g in range(w.Hkv):
                blocks = torch.randperm(C, generator=gen, device=device)[:n_shift]
                for t in (k, v):
                    z = torch.randn((n_shift, w.D), generator=gen, device=device)
                    u = z / z.norm(dim=1, keepdim=True)
                    view = t[b, g, : C * w.block].view(C, w.block, w.D)
                    view[blocks] += shift * u[:, None, :]
    k = k.to(dt)
    v = v.to(dt)
    cache_len = torch.full((w.B,), L, dtype=torch.int32, device=device)
    return q, k, v, cache_len


def score_matrix(shape, device="cpu", seed=0, dtype=torch.float32):
    """Plain N(0,1) fp32 score-like values, for Top-K and gate tests."""
    gen = generator(seed, device)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)
