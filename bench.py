"""Benchmark of the SAS hot path on one MI355X.

Training step (the headline): pool + score -> Top-K -> gated forward -> gated
backward at 32K tokens, sparse scope, Top-K 32 (Qwen3-8B-like layer: 32 query
heads / 8 KV heads, head dim 128, block 64), bf16, inputs resident in HBM.
`value` is algorithmic TFLOP/s: (4*D + 10*D) * attended pairs per step divided
by the step time, where attended pairs count each query row's own-block keys
(causal) plus the keys of its selected history blocks, exactly.

Also reported: per-kernel times (HIP events on the launch stream), the same
shape at full scope, the 8K-token full-scope step (Qwen3-4B-like layer), and
sparse decode tokens/s at 128K (batch 8; Top-K 16 as configured and 32, the
2048-token budget) and 512K (batch 1, Top-K 32, plus the dense-decode ratio),
each decode step being score + Top-K + sparse attention over one attention
layer (sas_decode_step, with the separate calls timed beside it), with the
256 MB last-level cache flushed between timed steps.  The CPU oracle is timed
on a sample of the training step and on the whole 512K decode step.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--quick | --decode-only | --full-only]
"""
from __future__ import annotations

import argparse
import json
import statistics
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--quick", action="store_true", help="training workload only (no decode, no full scope)")
    ap.add_argument("--workload", default="train-32k-sparse")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the two decode workloads (one JSON line of decode results)")
    ap.add_argument("--full-only", action="store_true",
                    help="only the full-scope step on the training shape (one JSON line; for profiling)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device copy first (counter calibration)")
    return ap.parse_args()


def attended_pairs(N, block, topk, Hq, B):
    """Exact count of (query row, key) pairs the SAS forward attends."""
    t = __import__("numpy").arange(N, dtype="int64")
    own = t % block + 1
    c = t // block
    hist = c if topk is None else __import__("numpy").minimum(c, topk)
    return int((own + block * hist).sum()) * Hq * B


class Timer:
    """Events recorded on torch's current stream, which the library launches on."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = {}

    def span(self, name):
        torch = self.torch
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        timer = self

        class _Span:
            def __enter__(self):
                start.record()

            def __exit__(self, *exc):
                end.record()
                timer.marks.setdefault(name, []).append((start, end))

        return _Span()

    def ms(self, name, median=False):
        ev = self.marks.get(name, [])
        if median and ev:
            return statistics.median(s.elapsed_time(e) for s, e in ev)
        return sum(s.elapsed_time(e) for s, e in ev) / max(1, len(ev))


def bench_train(torch, w, steps, warmup, scope_topk="cfg"):
    from trainable_block_sparse_sas_amd.inputs import training_inputs
    from trainable_block_sparse_sas_amd.pipeline import TrainStep

    topk = w.topk if scope_topk == "cfg" else scope_topk
    q, k, v, do = training_inputs(w, device="cuda")
    step = TrainStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, topk, w.torch_dtype)
    tm = Timer(torch)

    def one(record):
        if record:
            with tm.span("select"):
                step.select(q, k)
            with tm.span("fwd"):
                step.forward(q, k, v)
            with tm.span("bwd"):
                step.backward(q, k, v, do)
        else:
            step.run(q, k, v, do)

    for _ in range(warmup):
        one(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        one(False)
    s1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms_step = s0.elapsed_time(s1) / steps
    # Per-stage split in separate, event-bracketed steps; the library brackets
    # each of its kernels with HIP events on the same stream meanwhile.
    from trainable_block_sparse_sas_amd import binding as sas
    sas.sas_profile_read()
    sas.sas_profile_enable(True)
    n_split = max(2, steps // 2)
    for _ in range(n_split):
        one(True)
    torch.cuda.synchronize()
    sas.sas_profile_enable(False)
    kernels = {name: (ms / cnt, cnt // n_split) for name, (ms, cnt) in sas.sas_profile_read().items()}
    pairs = attended_pairs(w.N, w.block, topk, w.Hq, w.B)
    fl_fwd = 4 * w.D * pairs
    fl_bwd = 10 * w.D * pairs
    return dict(ms_step=ms_step, wall_ms_step=wall, pairs=pairs, flops_fwd=fl_fwd, flops_bwd=fl_bwd,
                ms_select=tm.ms("select"), ms_fwd=tm.ms("fwd"), ms_bwd=tm.ms("bwd"), kernels=kernels)


def bench_decode(torch, w, steps, warmup, dense=False):
    """Decode step times, median over `steps` iterations, with the last-level
    cache and L2 flushed before each timed span by a 1 GiB read (a sum over a
    1 GiB buffer).  A 1 GiB write flush leaves the memory-side cache full of
    dirty lines whose write-back then competes with the decode reads; its step
    time is reported beside it.  The step is sas_decode_step (scores, Top-K,
    per-block attention and merge, launched by one call); the same step through the separate calls
    (sas_score_blocks, sas_topk_select, sas_sparse_decode) is timed beside it.
    Dense decode is sas_sparse_decode over every cached position."""
    from trainable_block_sparse_sas_amd.inputs import decode_inputs
    from trainable_block_sparse_sas_amd.pipeline import DecodeStep
    from trainable_block_sparse_sas_amd import binding as sas

    q, kc, vc, lens = decode_inputs(w, device="cuda")
    step = DecodeStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, None if dense else w.topk, w.torch_dtype)
    step.pool(kc)  # pooled keys are kept beside the cache (prefill time)
    torch.cuda.synchronize()
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB > 256 MB last-level cache
    acc = torch.zeros(1, dtype=torch.float32, device="cuda")
    tiny = torch.zeros(16, dtype=torch.float32, device="cuda")
    ws = None
    if not dense:
        ws = sas.workspace(sas.SAS_OP_DECODE_STEP, w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk,
                           sas.SAS_BF16 if w.torch_dtype == torch.bfloat16 else sas.SAS_F32)

    def read_flush(i):
        torch.sum(flush, dim=0, keepdim=True, out=acc)

    def write_flush(i):
        flush.fill_(float(i & 7))

    def fused_step():
        sas.sas_decode_step(q, step.kbar, kc, vc, lens, w.topk, step.o, step.lse, w.block, w.scale,
                            idx_out=step.idx, workspace=ws)

    def separate_step():
        if not dense:
            step.select(q, lens)
        step.attend(q, kc, vc, lens)

    def timed(fn, pre, n, name, tm):
        for i in range(warmup + n):
            pre(i)
            if i < warmup:
                fn()
                continue
            with tm.span(name):
                fn()
        torch.cuda.synchronize()
        return tm.ms(name, median=True)

    tm = Timer(torch)
    run_step = separate_step if dense else fused_step
    ms = timed(run_step, read_flush, steps, "step", tm)
    ms_wf = timed(run_step, write_flush, steps, "step_wf", tm)
    floor = timed(lambda: tiny.fill_(1.0), read_flush, steps, "floor", tm)
    ms_sep = ms if dense else timed(separate_step, read_flush, steps, "separate", tm)
    # per-kernel durations: the library brackets each launch with HIP events on
    # its stream (read flush before every step, as above)
    sas.sas_profile_read()
    sas.sas_profile_enable(True)
    for i in range(steps):
        read_flush(i)
        run_step()
    torch.cuda.synchronize()
    sas.sas_profile_enable(False)
    kernels = {name: t / max(cnt, 1) for name, (t, cnt) in sas.sas_profile_read().items()}
    C = w.N // w.block
    kv_blocks = C if dense else (w.topk + 1)
    kv_bytes = w.B * w.Hkv * kv_blocks * w.block * w.D * 2 * 2
    kbar_bytes = 0 if dense else w.B * w.Hkv * C * w.D * 2
    # algorithmic bytes of one step: pooled keys and attended K, V read; q read,
    # o written; the group scores (fp32) written once
    qo_bytes = 2 * w.B * w.Hq * w.D * 2
    u_bytes = 0 if dense else w.B * w.Hkv * C * 4
    step_bytes = kv_bytes + kbar_bytes + qo_bytes + u_bytes
    return dict(ms_step=ms, tokens_per_s=w.B / (ms * 1e-3), kv_bytes=kv_bytes, kbar_bytes=kbar_bytes,
                step_bytes=step_bytes, ms_step_write_flush=ms_wf, ms_event_floor=floor, ms_separate=ms_sep,
                attend_gbs=kv_bytes / (ms * 1e-3) / 1e9, kernels=kernels)


def decode_traffic(kernel_substr):
    """HBM bytes per dispatch of a decode kernel from the committed counter
    summary (profiles/decode_hbm_traffic.md), or None."""
    path = os.path.join(ROOT, "profiles", "decode_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    hits = []
    with open(path) as fh:
        for line in fh:
            if line.startswith("| `") and kernel_substr in line:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                try:
                    hits.append(float(cells[-1]))
                except ValueError:
                    pass
    return int(hits[0]) if len(hits) == 1 else None


def decode_roofline(r, w):
    """Roofline of the decode attention kernel (the step's KV reads): the K and
    V bytes of the attended blocks over the kernel's average HIP-event time,
    against the 8 TB/s HBM peak; traffic from the committed FETCH/WRITE summary
    of the same kernel instantiation (the average over the workloads that share
    it)."""
    ms = r["kernels"].get("decode_partial")
    if not ms:
        return None
    ach = r["kv_bytes"] / (ms * 1e-3) / 1e9
    G = w.Hq // w.Hkv
    inst = f"decode_mfma_kernel<{w.D}, {G}, true>"
    return {"bound": "hbm", "kernel": "decode_partial", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": decode_traffic(inst),
            "bytes_per_launch": r["kv_bytes"], "avg_launch_ms": round(ms, 5),
            "timing": "HIP events around each launch on its stream (includes the event-pair overhead "
                      "of a few microseconds; the rocprofv3 kernel trace gives the bare duration)"}


def bench_paged_decode(torch, w, steps, warmup):
    """The same decode step over a paged copy of the cache (pages of one block
    per sequence and KV head, shuffled in a pool; sas_paged_decode runs scores,
    Top-K and attention), median over `steps` spans after a 1 GiB read flush."""
    from trainable_block_sparse_sas_amd.inputs import decode_inputs
    from trainable_block_sparse_sas_amd import binding as sas

    q, kc, vc, lens = decode_inputs(w, device="cuda")
    B, Hkv, L, D = kc.shape
    C = L // w.block
    n_pages = B * C
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(5)).to("cuda")
    table = perm.reshape(B, C).to(torch.int32).contiguous()
    kp = torch.empty((n_pages, Hkv, w.block, D), dtype=kc.dtype, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = kc.reshape(B, Hkv, C, w.block, D).permute(0, 2, 1, 3, 4).reshape(n_pages, Hkv, w.block, D)
    vp[perm] = vc.reshape(B, Hkv, C, w.block, D).permute(0, 2, 1, 3, 4).reshape(n_pages, Hkv, w.block, D)
    del kc, vc
    kbp = torch.empty((n_pages, Hkv, D), dtype=kp.dtype, device="cuda")
    sas.sas_pool_pages(kp, kbp, table.reshape(-1).contiguous(), w.block)
    o = torch.empty((B, w.Hq, D), dtype=kp.dtype, device="cuda")
    lse = torch.empty((B, w.Hq), dtype=torch.float32, device="cuda")
    ws = sas.workspace(sas.SAS_OP_PAGED_DECODE, B, w.Hq, Hkv, L, D, w.block, w.topk,
                       sas.SAS_BF16 if kp.dtype == torch.bfloat16 else sas.SAS_F32)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    acc = torch.zeros(1, dtype=torch.float32, device="cuda")
    tm = Timer(torch)
    for i in range(warmup + steps):
        torch.sum(flush, dim=0, keepdim=True, out=acc)
        if i < warmup:
            sas.sas_paged_decode(q, kp, vp, kbp, table, lens, w.topk, o, lse, w.block, w.scale, workspace=ws)
            continue
        with tm.span("paged"):
            sas.sas_paged_decode(q, kp, vp, kbp, table, lens, w.topk, o, lse, w.block, w.scale, workspace=ws)
    torch.cuda.synchronize()
    ms = tm.ms("paged", median=True)
    return {"ms_step": round(ms, 4), "tokens_per_s": round(B / (ms * 1e-3), 1),
            "layout": "pages of one block x all KV heads, shuffled pool; block table per sequence"}


# Algorithmic work of the matrix-core kernels per attended (query row, key)
# pair: the forward's S = QK^T and PV (4D flops; fwd_sel at sparse scope,
# fwd_mfma at full scope); the dK/dV kernel's S and dP recompute plus P^T dO
# and dS^T Q (8D), and at sparse scope also the rows' dQ shares dS K (2D); at
# full scope the dQ kernel's S and dP recompute plus dS K (6D; bwd_dq).
KERNEL_FLOPS_PER_PAIR = {"fwd_sel": 4, "fwd_mfma": 4, "bwd_dq": 6, "bwd_dkdv": 8}
SPARSE_KERNEL_FLOPS_PER_PAIR = dict(KERNEL_FLOPS_PER_PAIR, bwd_dkdv=10)
KERNEL_SOURCES = {"fwd_sel": "attn_fwd_sel.hip", "fwd_mfma": "attn_fwd_mfma.hip",
                  "bwd_dq": "attn_bwd_mfma.hip", "bwd_dkdv": "attn_bwd_mfma.hip"}


def kernel_source_hash(kernel):
    import hashlib
    csrc = os.path.join(ROOT, "trainable_block_sparse_sas_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "common.h", "mfma.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary of this kernel
    and workload, if the kernel's sources are unchanged since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline(kernels, pairs, D, workload, sparse=True):
    """Roofline entry for the kernel with the largest share of the step."""
    per_pair = SPARSE_KERNEL_FLOPS_PER_PAIR if sparse else KERNEL_FLOPS_PER_PAIR
    name = max((k for k in kernels if k in per_pair),
               key=lambda k: kernels[k][0] * kernels[k][1])
    ms = kernels[name][0]
    flops = per_pair[name] * D * pairs
    ach = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic(name, workload)
    out = {"bound": "mfma", "kernel": name, "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS,
           "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 5),
           "traffic": traffic,
           "flops_per_launch": flops, "avg_launch_ms": round(ms, 4),
           "timing": "HIP events around each launch on its stream (library kernel timing)"}
    if traffic:
        # The algorithmic work puts the kernel on the matrix-core side of the
        # roofline (its flops per unique byte are far above the ridge point),
        # so `bound` is "mfma".  The measured HBM bytes over the same launch
        # time say which peak the implementation is nearer: the sparse-scope
        # kernels re-read gathered rows and round-trip partials, and are held
        # by HBM traffic rather than by the matrix cores.
        hbm = traffic / (ms * 1e-3) / 1e12
        out["traffic_TBps"] = round(hbm, 3)
        out["traffic_frac_of_hbm_peak"] = round(hbm * 1000.0 / PEAK_HBM_GBS, 4)
        out["measured_limit"] = "hbm" if hbm * 1000.0 / PEAK_HBM_GBS > ach / PEAK_BF16_TFLOPS else "mfma"
    return out


def bench_selector_bwd(torch, w, steps):
    """The mean-pool selector's backward (sas_selector_bwd, accumulating into
    dq and dk) on the ds of one sparse training step, timed on its own.
    Work: per (query row, history block) score entry, 2D flops for dq and 2D
    for dK̄; the ds array is fp32 [B, Hq, N, C]."""
    from trainable_block_sparse_sas_amd.inputs import training_inputs
    from trainable_block_sparse_sas_amd.pipeline import TrainStep
    from trainable_block_sparse_sas_amd import binding as sas

    q, k, v, do = training_inputs(w, device="cuda")
    step = TrainStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk, w.torch_dtype)
    step.run(q, k, v, do)
    ws = sas.workspace(sas.SAS_OP_SELECTOR_BWD, w.B, w.Hq, w.Hkv, w.N, w.D, w.block, -1,
                       sas.SAS_BF16 if w.torch_dtype == torch.bfloat16 else sas.SAS_F32)

    def one():
        sas.sas_selector_bwd(q, step.kbar, step.ds, step.dq, step.dk, w.block, w.scale, accumulate=True,
                             workspace=ws)

    one()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        one()
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    sas.sas_profile_read()
    sas.sas_profile_enable(True)
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    sas.sas_profile_enable(False)
    kernels = {name: round(t / cnt, 4) for name, (t, cnt) in sas.sas_profile_read().items()}
    C = w.N // w.block
    entries = w.B * w.Hq * sum(min(t // w.block, C) for t in range(w.N))
    flops = 4 * w.D * entries
    return {"ms": round(ms, 4), "kernels_ms": kernels, "score_entries": entries,
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "note": "NEXT-row kernel, timed on its own; not part of the step above"}


def bench_gate_variants(torch, w, steps):
    """The pages' gate ablations (sigmoid gate, raw logit, outer gate, STE hard
    gate; the STE backward visits every history block) through
    sas_gated_attn_fwd_gate / _bwd_gate on one step's scores and selection,
    timed on their own: forward + backward per gate (the rewrite of the scores
    included), priced with the step's algorithmic work, 14 D flops per
    attended pair."""
    from trainable_block_sparse_sas_amd.inputs import training_inputs
    from trainable_block_sparse_sas_amd.pipeline import TrainStep
    from trainable_block_sparse_sas_amd import binding as sas

    q, k, v, do = training_inputs(w, device="cuda")
    step = TrainStep(w.B, w.Hq, w.Hkv, w.N, w.D, w.block, w.topk, w.torch_dtype)
    step.run(q, k, v, do)
    sdt = sas.SAS_BF16 if w.torch_dtype == torch.bfloat16 else sas.SAS_F32
    tk = -1 if w.topk is None else w.topk
    wsf = sas.workspace(sas.SAS_OP_FWD_GATE, w.B, w.Hq, w.Hkv, w.N, w.D, w.block, tk, sdt)
    wsb = sas.workspace(sas.SAS_OP_BWD_GATE, w.B, w.Hq, w.Hkv, w.N, w.D, w.block, tk, sdt)
    flops = 14 * w.D * attended_pairs(w.N, w.block, w.topk, w.Hq, w.B)
    out = {}
    for name, g in (("sigmoid", sas.SAS_GATE_SIGMOID), ("raw", sas.SAS_GATE_RAW), ("outer", sas.SAS_GATE_OUTER),
                    ("ste", sas.SAS_GATE_STE)):
        def one():
            sas.sas_gated_attn_fwd_gate(q, k, v, step.scores, step.idx, step.o, step.lse, step.lse_s, w.block,
                                        w.scale, g, wsf)
            sas.sas_gated_attn_bwd_gate(q, k, v, step.o, do, step.scores, step.idx, step.lse, step.lse_s, step.dq,
                                        step.dk, step.dv, step.ds, w.block, w.scale, g, wsb)

        one()
        torch.cuda.synchronize()
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(steps):
            one()
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / steps
        out[name] = {"ms_fwd_bwd": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    del wsf, wsb
    out["note"] = "NEXT-row entry points, timed on their own; not part of the step above"
    return out


def copy_probe(torch):
    """One plain streaming kernel over 1 GiB (bitwise not of 2^28 int32: 1 GiB
    read, 1 GiB written); its counter readings calibrate FETCH_SIZE and
    WRITE_SIZE."""
    src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _threads():
    try:
        import threadpoolctl
        return max(p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:
        return os.cpu_count()


def oracle_train_ops(ws, seed):
    """Wall-clock seconds of the oracle's training ops on workload ws (one run
    each): pool + score, Top-K (sparse scope), forward, backward."""
    import numpy as np
    import torch

    from oracle import sas_oracle as orc
    from trainable_block_sparse_sas_amd.inputs import training_inputs

    q, k, v, do = training_inputs(ws, device="cpu", seed=seed)
    f = lambda t: t.to(torch.float64).numpy()
    q, k, v, do = f(q), f(k), f(v), f(do)
    ops = {}
    t0 = time.perf_counter()
    kbar = orc.pool_block_keys(k, ws.block)
    pos = np.broadcast_to(np.arange(ws.N), (ws.B, ws.N))
    s = orc.block_scores(q, kbar, ws.block, ws.scale, pos)
    t1 = time.perf_counter()
    idx = None
    if ws.topk is not None:
        idx = orc.topk_select(s.astype(np.float32), ws.Hq // ws.Hkv, pos // ws.block, ws.topk)
    t2 = time.perf_counter()
    orc.gated_attention_forward(q, k, v, s, idx, ws.block, ws.scale)
    t3 = time.perf_counter()
    orc.gated_attention_backward(q, k, v, do, s, idx, ws.block, ws.scale)
    t4 = time.perf_counter()
    ops = {"pool_score": t1 - t0, "topk": t2 - t1, "fwd": t3 - t2, "bwd": t4 - t3}
    return ops, t4 - t0


def cpu_baseline(w):
    """The oracle, as it stands, on a bounded prefix sample of the workload."""
    n_s = 16384
    ws = w.with_(N=n_s, Hq=w.Hq // w.Hkv, Hkv=1, B=1)
    ops, dt = oracle_train_ops(ws, 1000 + w.index)
    pairs = attended_pairs(n_s, ws.block, ws.topk, ws.Hq, 1)
    flops = 14 * ws.D * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "seconds": dt, "seconds_per_op": {k: round(v, 3) for k, v in ops.items()},
            "sample": f"fp64 oracle pool+score+Top-K+fwd+bwd on the first {n_s} tokens of one KV-head "
                      f"group ({ws.Hq} query heads) of the same seeded inputs, Top-K {ws.topk}"}


def cpu_baseline_tiny(w):
    """The oracle on the whole small fp32 workload (full scope), all threads and
    one thread (after one untimed run)."""
    oracle_train_ops(w, 1000 + w.index)
    ops, dt = oracle_train_ops(w, 1000 + w.index)
    try:
        import threadpoolctl
        with threadpoolctl.threadpool_limits(1):
            ops1, dt1 = oracle_train_ops(w, 1000 + w.index)
    except Exception:
        ops1, dt1 = None, None
    pairs = attended_pairs(w.N, w.block, w.topk, w.Hq, w.B)
    return {"value": 14 * w.D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "seconds": dt, "seconds_per_op": {k: round(v, 4) for k, v in ops.items()},
            "seconds_1_thread": dt1,
            "seconds_per_op_1_thread": None if ops1 is None else {k: round(v, 4) for k, v in ops1.items()},
            "sample": f"fp64 oracle pool+score+fwd+bwd, whole {w.name} workload"}


def decode_entry(r, topk):
    gbs = r["step_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    return {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_step": round(r["ms_step"], 4),
            "ms_step_separate_calls": round(r["ms_separate"], 4),
            "ms_step_after_write_flush": round(r["ms_step_write_flush"], 4),
            "step_bytes": r["step_bytes"], "kv_bytes": r["kv_bytes"], "kbar_bytes": r["kbar_bytes"],
            "step_GBps": round(gbs, 1), "step_frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "ms_event_pair_floor": round(r["ms_event_floor"], 4),
            "timing": "median of 50 HIP-event spans of sas_decode_step, 1 GiB read flush before each span "
                      "(each span includes the event-pair floor)",
            "kernels_ms": {k: round(v, 5) for k, v in sorted(r["kernels"].items(), key=lambda kv: -kv[1])},
            "topk": topk}


def bench_decodes(torch, wmap):
    dec = {}
    for name, topks in (("decode-128k-b8", (16, 32)), ("decode-512k-b1", (32,))):
        dec[name] = {}
        for topk in topks:
            wd = wmap[name].with_(topk=topk)
            r = bench_decode(torch, wd, 50, 10)
            ent = decode_entry(r, topk)
            ent["roofline"] = decode_roofline(r, wd)
            ent["paged"] = bench_paged_decode(torch, wd, 50, 10)
            dec[name][f"k{topk}"] = ent
            torch.cuda.empty_cache()
            if name == "decode-512k-b1":
                rd = bench_decode(torch, wd, 20, 3, dense=True)
                dec[name]["dense_ms"] = round(rd["ms_step"], 4)
                dec[name]["dense_GBps"] = round(rd["attend_gbs"], 1)
                dec[name]["speedup_vs_dense"] = round(rd["ms_step"] / r["ms_step"], 2)
                dec[name]["pages_speedup_context"] = ("5.6x end-to-end Qwen3-4B decode at 512K, batch 1, "
                                                      "unnamed GPU")
    return dec


def cpu_baseline_decode(w):
    """The oracle's decode step (group scores from the pooled keys, Top-K,
    sparse attention; pooled keys precomputed, as on the GPU) on the same seeded
    cache as the GPU run, all threads and one thread."""
    import numpy as np
    import torch

    from oracle import sas_oracle as orc
    from trainable_block_sparse_sas_amd.inputs import decode_inputs

    q, kc, vc, lens = decode_inputs(w, device="cpu")
    f = lambda t: t.to(torch.float64).numpy()
    q64, kc64, vc64, lens_np = f(q), f(kc), f(vc), lens.numpy()
    del kc, vc
    kbar = orc.pool_block_keys(kc64, w.block)

    def one():
        u = orc.decode_scores(q64, kbar, lens_np, w.N, w.block, w.scale, True)
        c = orc.decode_candidates(lens_np, w.N, w.block)
        idx = orc.topk_select(u[:, :, None, :], 1, c[:, None], w.topk)[:, :, 0, :]
        orc.sparse_decode(q64, kc64, vc64, lens_np, idx, w.block, w.scale)

    def timed():
        one()
        t0 = time.perf_counter()
        n = 3
        for _ in range(n):
            one()
        return (time.perf_counter() - t0) / n

    try:
        import threadpoolctl
        cores = _threads()
        dt = timed()
        with threadpoolctl.threadpool_limits(1):
            dt1 = timed()
    except Exception:
        cores, dt, dt1 = os.cpu_count(), timed(), None
    return {"value": w.B / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "seconds_per_step": dt,
            "seconds_per_step_1_thread": dt1,
            "sample": f"fp64 oracle decode step ({w.name}, Top-K {w.topk}: scores from precomputed pooled "
                      f"keys, Top-K, sparse attention), whole workload"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); the multi-GPU path is a "
              f"design, not a built component.", file=sys.stderr)
        sys.exit(2)
    import torch

    from trainable_block_sparse_sas_amd.inputs import WORKLOADS

    wmap = {w.name: w for w in WORKLOADS}
    w = wmap[args.workload]
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(torch)
    if args.decode_only:
        print(json.dumps({"decode": bench_decodes(torch, wmap)}))
        return
    if args.full_only:
        full = bench_train(torch, w, args.steps, args.warmup, scope_topk=None)
        print(json.dumps({"full_scope_same_shape": {
            "ms_step": round(full["ms_step"], 3),
            "tflops": round((full["flops_fwd"] + full["flops_bwd"]) / (full["ms_step"] * 1e-3) / 1e12, 3),
            "kernels_ms": {k: round(v[0], 4) for k, v in sorted(full["kernels"].items(), key=lambda kv: -kv[1][0])}}}))
        return
    tr = bench_train(torch, w, args.steps, args.warmup)
    tflops = (tr["flops_fwd"] + tr["flops_bwd"]) / (tr["ms_step"] * 1e-3) / 1e12
    out = {
        "metric": "gated attn fwd+bwd TFLOP/s @32K (sparse scope, Top-K 32)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tr["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v, dO)",
        "config": {"workload": w.name, "batch": w.B, "seq_len": w.N, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "block": w.block, "topk": w.topk,
                   "step": "pool+score -> topk -> gated fwd -> gated bwd"},
        "stages_ms": {"select": round(tr["ms_select"], 4), "fwd": round(tr["ms_fwd"], 4),
                      "bwd": round(tr["ms_bwd"], 4)},
        "attended_pairs": tr["pairs"],
        "kernels_ms": {k: round(v[0], 4) for k, v in sorted(tr["kernels"].items(), key=lambda kv: -kv[1][0])},
        "roofline": roofline(tr["kernels"], tr["pairs"], w.D, w.name),
    }
    if not args.quick:
        full = bench_train(torch, w, max(2, args.steps // 2), 1, scope_topk=None)
        out["full_scope_same_shape"] = {
            "ms_step": round(full["ms_step"], 3),
            "tflops": round((full["flops_fwd"] + full["flops_bwd"]) / (full["ms_step"] * 1e-3) / 1e12, 3),
            "fwd_tflops": round(full["flops_fwd"] / (full["ms_fwd"] * 1e-3) / 1e12, 3),
            "bwd_tflops": round(full["flops_bwd"] / (full["ms_bwd"] * 1e-3) / 1e12, 3)}
        w8 = wmap["train-8k-full"]
        t8 = bench_train(torch, w8, max(3, args.steps), 2)
        out["train_8k_full"] = {
            "ms_step": round(t8["ms_step"], 4),
            "tflops": round((t8["flops_fwd"] + t8["flops_bwd"]) / (t8["ms_step"] * 1e-3) / 1e12, 3),
            "fwd_tflops": round(t8["flops_fwd"] / (t8["ms_fwd"] * 1e-3) / 1e12, 3),
            "bwd_tflops": round(t8["flops_bwd"] / (t8["ms_bwd"] * 1e-3) / 1e12, 3),
            "step": "pool+score -> gated fwd -> gated bwd, full scope (8192 tokens, 32/8 heads, D 128)"}
        del t8
        w0 = wmap["tiny-f32-full"]
        t0w = bench_train(torch, w0, 20, 3)
        out["train_tiny_f32"] = {
            "ms_step": round(t0w["ms_step"], 4),
            "step": "pool+score -> gated fwd -> gated bwd, full scope, fp32 (512 tokens, 2/1 heads, D 64; "
                    "the oracle-sized parity case, timed for the record)"}
        torch.cuda.empty_cache()
        out["decode"] = bench_decodes(torch, wmap)
        out["selector_bwd"] = bench_selector_bwd(torch, w, 5)
        out["gate_variants"] = bench_gate_variants(torch, w, 3)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
        if not args.quick:
            out["cpu_baseline_decode"] = cpu_baseline_decode(wmap["decode-512k-b1"])
            out["cpu_baseline_decode_128k"] = cpu_baseline_decode(wmap["decode-128k-b8"])
            out["cpu_baseline_tiny"] = cpu_baseline_tiny(wmap["tiny-f32-full"])
    print(json.dumps(out))


if __name__ == "__main__":
    main()
