"""C ABI contract checks that need no GPU: the library loads, exports every
function include/sas.h declares, and rejects invalid arguments on the host
(before any HIP call) with the documented status codes."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")

sas = pytest.importorskip("trainable_block_sparse_sas_amd.binding")
L = sas._lib
N = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == {"sas_score_blocks", "sas_score_blocks_lse", "sas_topk_select", "sas_topk_select_gated",
                          "sas_gated_attn_fwd", "sas_gated_attn_fwd_lse", "sas_gated_attn_fwd_ctx",
                          "sas_gated_attn_bwd_ctx",
                          "sas_gated_attn_bwd", "sas_gated_attn_fwd_gate", "sas_gated_attn_bwd_gate",
                          "sas_sparse_decode", "sas_selector_bwd", "sas_pool_pages",
                          "sas_paged_decode", "sas_sparse_decode_noalloc", "sas_decode_step", "sas_prefill_paged", "sas_workspace_bytes",
                          "sas_last_error", "sas_abi_version", "sas_profile_enable",
                          "sas_profile_read"}
    for n in names:
        assert hasattr(L, n), n
        assert n in sas.EXPORTED


def test_version_and_workspace_sizes():
    assert sas.sas_abi_version() == 106
    assert sas.sas_workspace_bytes(sas.SAS_OP_SCORE, 1, 32, 8, 8192, 128, 64, -1, 1) == 0
    assert sas.sas_workspace_bytes(sas.SAS_OP_BWD, 1, 32, 8, 8192, 128, 64, -1, 1) >= 32 * 8192 * 4
    assert sas.sas_workspace_bytes(sas.SAS_OP_DECODE, 8, 32, 8, 131072, 128, 64, 16, 1) > 0
    assert sas.sas_workspace_bytes(sas.SAS_OP_FWD, 1, 3, 2, 64, 128, 64, -1, 1) == ctypes.c_size_t(-1).value
    assert sas.sas_workspace_bytes(99, 1, 4, 2, 64, 128, 64, -1, 1) == ctypes.c_size_t(-1).value
    # selector backward: fp32 partials of dK̄ per 1024-token chunk (bf16), one chunk (fp32)
    assert sas.sas_workspace_bytes(sas.SAS_OP_SELECTOR_BWD, 1, 32, 8, 32768, 128, 64, -1, 1) == \
        32 * 8 * 512 * 128 * 4
    assert sas.sas_workspace_bytes(sas.SAS_OP_SELECTOR_BWD, 1, 4, 2, 512, 64, 64, -1, 0) == 2 * 8 * 64 * 4
    assert sas.sas_workspace_bytes(sas.SAS_OP_SELECTOR_BWD, 1, 4, 2, 512, 96, 64, -1, 1) == \
        ctypes.c_size_t(-1).value


def fwd(B=1, Hq=4, Hkv=2, N_=128, D=128, block=64, topk=0, dtype=1, ptr=1, idx=None, ws=None, wsb=0,
        scale=0.1):
    p = ctypes.c_void_p(ptr) if ptr else None
    return L.sas_gated_attn_fwd(p, p, p, p, idx, p, p, p, B, Hq, Hkv, N_, D, block, topk, scale, dtype,
                                ws, wsb, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(Hq=3, Hkv=2), sas.SAS_EINVAL, "multiple"),
    (dict(Hkv=0), sas.SAS_EINVAL, "Hkv"),
    (dict(B=-1), sas.SAS_EINVAL, "non-negative"),
    (dict(block=0), sas.SAS_EINVAL, "block"),
    (dict(dtype=7), sas.SAS_EINVAL, "dtype"),
    (dict(D=96), sas.SAS_EUNSUPPORTED, "head dim"),
    (dict(ptr=0), sas.SAS_EINVAL, "non-NULL"),
    (dict(idx=ctypes.c_void_p(8), topk=-1), sas.SAS_EINVAL, "topk"),
    (dict(idx=ctypes.c_void_p(8), topk=300), sas.SAS_EUNSUPPORTED, "topk"),
    (dict(scale=0.0), sas.SAS_EINVAL, "scale"),
    (dict(scale=-0.5), sas.SAS_EINVAL, "scale"),
    (dict(scale=float("nan")), sas.SAS_EINVAL, "scale"),
    (dict(scale=float("inf")), sas.SAS_EINVAL, "scale"),
])
def test_fwd_rejects(kw, code, msg):
    assert fwd(**kw) == code
    assert msg in sas.sas_last_error()


def test_empty_calls_succeed_without_gpu():
    assert fwd(N_=0) == 0
    assert fwd(B=0) == 0
    assert L.sas_topk_select(N, N, N, 1, 2, 4, 16, 8, 64, 0, N, 0, N) == 0


def test_other_entry_points_reject():
    v = ctypes.c_void_p(8)
    # score: training mode needs Nq == L
    assert L.sas_score_blocks(v, v, v, v, N, 1, 4, 2, 100, 128, 128, 64, 0.1, 0, 1, N) == sas.SAS_EINVAL
    # score: decode mode needs Nq == 1 and at most 16 heads per KV head
    assert L.sas_score_blocks(v, N, v, v, v, 1, 4, 2, 2, 128, 128, 64, 0.1, 1, 1, N) == sas.SAS_EINVAL
    assert L.sas_score_blocks(v, N, v, v, v, 1, 34, 2, 1, 128, 128, 64, 0.1, 1, 1, N) == sas.SAS_EUNSUPPORTED
    # topk: heads_per_row, sizes, limits
    assert L.sas_topk_select(v, v, N, 1, 2, 0, 16, 8, 64, 4, N, 0, N) == sas.SAS_EINVAL
    assert L.sas_topk_select(v, v, N, 1, 2, 4, 16, 8, 64, -2, N, 0, N) == sas.SAS_EINVAL
    assert L.sas_topk_select(v, v, N, 1, 2, 4, 16, 20000, 64, 4, N, 0, N) == sas.SAS_EUNSUPPORTED
    assert L.sas_topk_select(v, v, N, 1, 2, 4, 16, 8, 64, 257, N, 0, N) == sas.SAS_EUNSUPPORTED
    assert L.sas_topk_select(v, v, v, 1, 2, 1, 3, 8, 64, 4, N, 0, N) == sas.SAS_EINVAL
    assert L.sas_topk_select(N, v, N, 1, 2, 1, 3, 8, 64, 4, N, 0, N) == sas.SAS_EINVAL
    # bwd: workspace required
    args = [v] * 13 + [1, 4, 2, 128, 128, 64, 0, 0.1, 1]
    assert L.sas_gated_attn_bwd(*args, N, 0, N) == sas.SAS_EWORKSPACE
    assert "workspace" in sas.sas_last_error()
    # decode: workspace, cache_len and head-group limits
    dargs = [v, v, v, v, N, v, N, 2, 8, 2, 1024, 128, 64, 4, 0.1, 1]
    assert L.sas_sparse_decode(*dargs, N, 0, N) == sas.SAS_EWORKSPACE
    dargs2 = [v, v, v, N, N, v, N, 2, 8, 2, 1024, 128, 64, 4, 0.1, 1]
    assert L.sas_sparse_decode(*dargs2, v, 1 << 30, N) == sas.SAS_EINVAL
    dargs3 = [v, v, v, v, N, v, N, 2, 40, 2, 1024, 128, 64, 4, 0.1, 1]
    assert L.sas_sparse_decode(*dargs3, v, 1 << 30, N) == sas.SAS_EUNSUPPORTED


def test_scale_checked_by_every_scaled_call():
    v = ctypes.c_void_p(8)
    assert L.sas_score_blocks(v, v, v, v, N, 1, 4, 2, 128, 128, 128, 64, -1.0, 0, 1, N) == sas.SAS_EINVAL
    args = [v] * 13 + [1, 4, 2, 128, 128, 64, 0, 0.0, 1]
    assert L.sas_gated_attn_bwd(*args, v, 1 << 30, N) == sas.SAS_EINVAL
    dargs = [v, v, v, v, N, v, N, 2, 8, 2, 1024, 128, 64, 4, float("nan"), 1]
    assert L.sas_sparse_decode(*dargs, v, 1 << 30, N) == sas.SAS_EINVAL
    assert "scale" in sas.sas_last_error()


def test_profile_api_without_launches():
    sas.sas_profile_enable(True)
    sas.sas_profile_enable(False)
    assert sas.sas_profile_read() == {}
    names = ctypes.create_string_buffer(8)
    ms = (ctypes.c_double * 1)()
    cnt = (ctypes.c_int * 1)()
    assert L.sas_profile_read(-1, names, 8, ms, cnt) == sas.SAS_EINVAL
    assert L.sas_profile_read(1, names, 0, ms, cnt) == sas.SAS_EINVAL
    assert L.sas_profile_read(1, None, 8, ms, cnt) == sas.SAS_EINVAL


def test_errors_are_thread_local():
    import threading
    assert fwd(Hq=3, Hkv=2) == sas.SAS_EINVAL
    seen = {}

    def other():
        seen["msg"] = sas.sas_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "multiple" in sas.sas_last_error()


def test_selector_bwd_host_checks():
    v = ctypes.c_void_p(8)
    base = [v, v, v, v, v, N]

    def call(B=1, Hq=4, Hkv=2, N_=128, D=128, block=64, scale=0.1, acc=0, dtype=1, ws=v, wsb=1 << 30, ptrs=None):
        return L.sas_selector_bwd(*(ptrs or base), B, Hq, Hkv, N_, D, block, scale, acc, dtype, ws, wsb, N)

    assert call(Hq=3) == sas.SAS_EINVAL
    assert call(D=96) == sas.SAS_EUNSUPPORTED
    assert call(block=0) == sas.SAS_EINVAL
    assert call(scale=0.0) == sas.SAS_EINVAL
    assert call(acc=2) == sas.SAS_EINVAL
    assert call(ptrs=[v, N, v, v, v, N]) == sas.SAS_EINVAL
    assert "non-NULL" in sas.sas_last_error()
    assert call(ws=N, wsb=0) == sas.SAS_EWORKSPACE
    assert call(B=0, ptrs=[N] * 6) == sas.SAS_OK


def test_paged_decode_host_checks():
    v = ctypes.c_void_p(8)

    def call(maxb=16, topk=4, B=2, Hq=8, Hkv=2, D=128, block=64, scale=0.1, dtype=1, ptrs=None, ws=v, wsb=1 << 30):
        p = ptrs or [v, v, v, v, v]
        return L.sas_paged_decode(*p, maxb, v, topk, v, N, N, B, Hq, Hkv, D, block, scale, dtype, ws, wsb, N)

    assert call(dtype=0) == sas.SAS_EUNSUPPORTED
    assert call(topk=-1) == sas.SAS_EINVAL
    assert call(topk=300) == sas.SAS_EUNSUPPORTED
    assert call(Hq=40) == sas.SAS_EUNSUPPORTED
    assert call(maxb=20000) == sas.SAS_EUNSUPPORTED
    assert call(maxb=-1) == sas.SAS_EINVAL
    assert call(D=96) == sas.SAS_EUNSUPPORTED
    assert call(ptrs=[v, v, v, v, N]) == sas.SAS_EINVAL
    assert call(ws=N, wsb=0) == sas.SAS_EWORKSPACE
    assert call(B=0, ptrs=[N] * 5) == sas.SAS_OK
    need = sas.sas_workspace_bytes(sas.SAS_OP_PAGED_DECODE, 2, 8, 2, 16 * 64, 128, 64, 4, 1)
    assert need >= 2 * 2 * 16 * 4 + sas.sas_workspace_bytes(sas.SAS_OP_DECODE, 2, 8, 2, 16 * 64, 128, 64, 4, 1)
    assert call(wsb=need - 1) == sas.SAS_EWORKSPACE
    assert L.sas_pool_pages(v, v, v, -1, 2, 128, 64, 1, N) == sas.SAS_EINVAL
    assert L.sas_pool_pages(v, v, N, 3, 2, 128, 64, 1, N) == sas.SAS_EINVAL
    assert L.sas_pool_pages(N, N, N, 0, 2, 128, 64, 1, N) == sas.SAS_OK


def test_gate_variant_host_checks():
    """Gate variants: an unknown gate is rejected before any GPU work, empty
    calls succeed, the workspace grows by the rewritten scores (fp32
    [B,Hq,N,C]) and, for the backward, a zero LSE_s per row; the softmax gate
    needs exactly the plain call's workspace."""
    p = ctypes.c_void_p(1)
    args = (p, p, p, p, None, p, p, p, 1, 4, 2, 128, 128, 64, 0, 0.1, 1)
    assert L.sas_gated_attn_fwd_gate(*args, 7, None, 0, None) == sas.SAS_EINVAL
    assert L.sas_gated_attn_fwd_gate(*args, 5, None, 0, None) == sas.SAS_EINVAL
    assert "gate" in sas._lib.sas_last_error().decode()
    assert L.sas_gated_attn_fwd_gate(*args[:8], 0, *args[9:], 1, None, 0, None) == sas.SAS_OK
    bargs = (p,) * 13 + (1, 4, 2, 128, 128, 64, 0, 0.1, 1)
    assert L.sas_gated_attn_bwd_gate(*bargs, -1, None, 0, None) == sas.SAS_EINVAL
    # the backward of a non-softmax gate does not read lse_s: NULL is fine for the host checks
    nb = list(bargs)
    nb[8] = None
    nb[13] = 0  # B = 0: an empty call
    assert L.sas_gated_attn_bwd_gate(*nb, 2, None, 0, None) == sas.SAS_OK
    # the outer gate reads lse_s: NULL is refused
    nb[13] = 1
    assert L.sas_gated_attn_bwd_gate(*nb, 3, None, 0, None) == sas.SAS_EINVAL
    # and needs no workspace beyond the softmax gate's
    assert sas.sas_workspace_bytes(sas.SAS_OP_FWD, 1, 4, 2, 128, 128, 64, -1, 1) > 0
    B, Hq, Hkv, N, D, blk = 1, 32, 8, 8192, 128, 64
    rows, C = B * Hq * N, N // blk
    f0 = sas.sas_workspace_bytes(sas.SAS_OP_FWD, B, Hq, Hkv, N, D, blk, -1, 1)
    fg = sas.sas_workspace_bytes(sas.SAS_OP_FWD_GATE, B, Hq, Hkv, N, D, blk, -1, 1)
    assert fg >= f0 + rows * C * 4
    b0 = sas.sas_workspace_bytes(sas.SAS_OP_BWD, B, Hq, Hkv, N, D, blk, 32, 1)
    bg = sas.sas_workspace_bytes(sas.SAS_OP_BWD_GATE, B, Hq, Hkv, N, D, blk, 32, 1)
    assert bg >= b0 + rows * C * 4 + rows * 4
    # a workspace big enough for the softmax gate only is refused on the host
    small = sas.sas_workspace_bytes(sas.SAS_OP_FWD, 1, 4, 2, 128, 128, 64, -1, 1)
    assert small < sas.sas_workspace_bytes(sas.SAS_OP_FWD_GATE, 1, 4, 2, 128, 128, 64, -1, 1)
    assert L.sas_gated_attn_fwd_gate(*args, 1, p, small, None) == sas.SAS_EWORKSPACE


def test_noalloc_decode_validation_on_the_host():
    """The allocation-free decode validates like sas_sparse_decode and refuses
    sizes whose partials exceed its fixed 8 MiB scratch, all before any HIP
    call (dummy pointers are never dereferenced)."""
    vp = ctypes.c_void_p
    d = vp(256)
    f = ctypes.c_float
    # dense decode, 16 query heads on one KV head, 1M tokens: more than 8 MiB of partials
    need = sas.sas_workspace_bytes(sas.SAS_OP_DECODE, 1, 16, 1, 1 << 20, 128, 64, -1, sas.SAS_BF16)
    assert need > (8 << 20)
    assert L.sas_sparse_decode_noalloc(d, d, d, d, N, d, N, 1, 16, 1, 1 << 20, 128, 64, 0, f(0.1),
                                       sas.SAS_BF16, N) == sas.SAS_EUNSUPPORTED
    assert "scratch" in sas.sas_last_error()
    assert L.sas_sparse_decode_noalloc(N, d, d, d, N, d, N, 1, 4, 2, 1024, 128, 64, 0, f(0.1),
                                       sas.SAS_BF16, N) == sas.SAS_EINVAL
    assert L.sas_sparse_decode_noalloc(d, d, d, d, d, d, N, 1, 4, 2, 1024, 128, 64, -1, f(0.1),
                                       sas.SAS_BF16, N) == sas.SAS_EINVAL
    assert L.sas_sparse_decode_noalloc(d, d, d, d, N, d, N, 1, 4, 2, 1024, 96, 64, 0, f(0.1),
                                       sas.SAS_BF16, N) == sas.SAS_EUNSUPPORTED
    assert L.sas_sparse_decode_noalloc(d, d, d, d, N, d, N, 0, 4, 2, 1024, 128, 64, 0, f(0.1),
                                       sas.SAS_BF16, N) == sas.SAS_OK


def test_decode_step_validation_on_the_host():
    """sas_decode_step validates on the host, before any HIP call, through the
    Python binding's argument list (so the binding's signature is exercised)."""
    vp = ctypes.c_void_p
    d = vp(256)
    f = ctypes.c_float
    ws_need = sas.sas_workspace_bytes(sas.SAS_OP_DECODE_STEP, 2, 8, 2, 4096, 128, 64, 16, sas.SAS_BF16)
    assert 0 < ws_need < (1 << 30)
    call = L.sas_decode_step
    # workspace missing / too small
    assert call(d, d, d, d, d, 16, d, N, N, 2, 8, 2, 4096, 128, 64, f(0.1), sas.SAS_BF16, N, 0, N) == sas.SAS_EWORKSPACE
    assert call(d, d, d, d, d, 16, d, N, N, 2, 8, 2, 4096, 128, 64, f(0.1), sas.SAS_BF16, d, ws_need - 1,
                N) == sas.SAS_EWORKSPACE
    # bad arguments
    assert call(N, d, d, d, d, 16, d, N, N, 2, 8, 2, 4096, 128, 64, f(0.1), sas.SAS_BF16, d, ws_need,
                N) == sas.SAS_EINVAL
    assert call(d, d, d, d, d, -1, d, N, N, 2, 8, 2, 4096, 128, 64, f(0.1), sas.SAS_BF16, d, ws_need,
                N) == sas.SAS_EINVAL
    assert call(d, d, d, d, d, 300, d, N, N, 2, 8, 2, 4096, 128, 64, f(0.1), sas.SAS_BF16, d, 1 << 40,
                N) == sas.SAS_EUNSUPPORTED
    assert call(d, d, d, d, d, 16, d, N, N, 2, 40, 2, 4096, 128, 64, f(0.1), sas.SAS_BF16, d, 1 << 40,
                N) == sas.SAS_EUNSUPPORTED
    assert call(d, d, d, d, d, 16, d, N, N, 2, 8, 2, 4096, 128, 64, f(-1.0), sas.SAS_BF16, d, 1 << 40,
                N) == sas.SAS_EINVAL
    assert call(d, d, d, d, d, 16, d, N, N, 0, 8, 2, 4096, 128, 64, f(0.1), sas.SAS_BF16, N, 0, N) == sas.SAS_OK


def test_prefill_validation_on_the_host():
    vp = ctypes.c_void_p
    d = vp(256)
    f = ctypes.c_float
    need = sas.sas_workspace_bytes(sas.SAS_OP_PREFILL, 2, 8, 2, 640, 128, 64, 0, sas.SAS_BF16)
    assert 0 < need < (1 << 30)
    call = L.sas_prefill_paged
    args = (d, d, d, d, d, N, d, d, d, d)
    assert call(*args, 10, 2, 8, 2, 640, 128, 64, f(0.1), sas.SAS_BF16, d, need - 1, N) == sas.SAS_EWORKSPACE
    assert call(*args, 9, 2, 8, 2, 640, 128, 64, f(0.1), sas.SAS_BF16, d, need + (1 << 20), N) == sas.SAS_EINVAL
    assert call(*args, 10, 2, 8, 2, 640, 96, 64, f(0.1), sas.SAS_BF16, d, need, N) == sas.SAS_EUNSUPPORTED
    assert call(N, d, d, d, d, N, d, d, d, d, 10, 2, 8, 2, 640, 128, 64, f(0.1), sas.SAS_BF16, d, 1 << 40,
                N) == sas.SAS_EINVAL
    assert call(*args, 10, 0, 8, 2, 640, 128, 64, f(0.1), sas.SAS_BF16, N, 0, N) == sas.SAS_OK


def test_fused_gate_normaliser_validation_on_the_host():
    """sas_score_blocks_lse and sas_gated_attn_fwd_lse: argument checks run
    before any launch (no call here reaches the GPU)."""
    d = ctypes.c_void_p(256)
    f = ctypes.c_float
    call = L.sas_score_blocks_lse
    # lse_s missing, scale invalid, head dims unsupported, Hq % Hkv != 0
    assert call(d, N, d, d, N, 1, 4, 2, 256, 128, 64, f(0.1), sas.SAS_BF16, N) == sas.SAS_EINVAL
    assert "lse_s" in sas.sas_last_error()
    assert call(d, N, d, d, d, 1, 4, 2, 256, 128, 64, f(-1.0), sas.SAS_BF16, N) == sas.SAS_EINVAL
    assert call(d, N, d, d, d, 1, 4, 2, 256, 96, 64, f(0.1), sas.SAS_BF16, N) == sas.SAS_EUNSUPPORTED
    assert call(d, N, d, d, d, 1, 5, 2, 256, 128, 64, f(0.1), sas.SAS_BF16, N) == sas.SAS_EINVAL
    # empty sizes are no-ops even with NULL tensors
    assert call(N, N, N, N, N, 0, 4, 2, 256, 128, 64, f(0.1), sas.SAS_BF16, N) == sas.SAS_OK
    fwd = L.sas_gated_attn_fwd_lse
    need = sas.sas_workspace_bytes(sas.SAS_OP_FWD, 1, 8, 2, 512, 128, 64, 4, sas.SAS_BF16)
    assert need > 0
    assert fwd(d, d, d, d, d, d, d, d, 1, 8, 2, 512, 128, 64, 4, f(0.1), sas.SAS_BF16, d, need - 1,
               N) == sas.SAS_EWORKSPACE
    assert fwd(d, d, d, d, d, N, d, d, 1, 8, 2, 512, 128, 64, 4, f(0.1), sas.SAS_BF16, d, need,
               N) == sas.SAS_EINVAL
    assert fwd(d, d, d, d, d, d, d, d, 1, 8, 2, 512, 128, 64, 300, f(0.1), sas.SAS_BF16, d, 1 << 40,
               N) == sas.SAS_EUNSUPPORTED


def test_saved_context_sizes_and_validation_on_the_host():
    """sas_gated_attn_fwd_ctx / _bwd_ctx: the context size, and a missing or
    short context refused before any launch."""
    d = ctypes.c_void_p(256)
    f = ctypes.c_float
    bf, f32 = sas.SAS_BF16, sas.SAS_F32
    n = sas.sas_workspace_bytes(sas.SAS_OP_CTX, 1, 8, 2, 512, 128, 64, 4, bf)
    assert n > 0
    # used only at sparse scope on the matrix cores
    assert sas.sas_workspace_bytes(sas.SAS_OP_CTX, 1, 8, 2, 512, 128, 64, -1, bf) == 0
    assert sas.sas_workspace_bytes(sas.SAS_OP_CTX, 1, 8, 2, 512, 128, 64, 4, f32) == 0
    assert sas.sas_workspace_bytes(sas.SAS_OP_CTX, 1, 8, 2, 512, 128, 32, 4, bf) == 0
    wf = sas.sas_workspace_bytes(sas.SAS_OP_FWD, 1, 8, 2, 512, 128, 64, 4, bf)
    wb = sas.sas_workspace_bytes(sas.SAS_OP_BWD, 1, 8, 2, 512, 128, 64, 4, bf)
    fwd, bwd = L.sas_gated_attn_fwd_ctx, L.sas_gated_attn_bwd_ctx
    sizes = (1, 8, 2, 512, 128, 64, 4, f(0.1), bf)
    assert fwd(d, d, d, d, d, d, N, d, d, *sizes, N, 0, d, wf, N) == sas.SAS_EWORKSPACE
    assert "context" in sas.sas_last_error()
    assert fwd(d, d, d, d, d, d, N, d, d, *sizes, d, n - 1, d, wf, N) == sas.SAS_EWORKSPACE
    assert fwd(d, d, d, d, d, d, d, d, d, *sizes, d, n, d, wf - 1, N) == sas.SAS_EWORKSPACE
    # given log gates belong to a selection: not at full scope
    full = (1, 8, 2, 512, 128, 64, 0, f(0.1), bf)
    assert fwd(d, d, d, d, N, d, d, d, d, *full, N, 0, d, 1 << 40, N) == sas.SAS_EINVAL
    assert "idx" in sas.sas_last_error()
    assert bwd(d, d, d, d, d, d, d, d, d, N, 0, d, d, d, d, *sizes, d, wb, N) == sas.SAS_EWORKSPACE
    assert bwd(d, d, d, d, d, d, d, d, d, d, n - 1, d, d, d, d, *sizes, d, wb, N) == sas.SAS_EWORKSPACE
    assert bwd(d, d, d, d, d, d, d, d, d, d, n, d, d, N, d, *sizes, d, wb, N) == sas.SAS_EINVAL


def test_gated_topk_validation_on_the_host():
    """sas_topk_select_gated: argument checks before any launch; its range is the
    one-wave-per-row Top-K (C <= 1024, topk <= 64, heads_per_row 1, 2, 4, 8)."""
    N = None
    v = ctypes.c_void_p(256)
    call = L.sas_topk_select_gated
    # empty sizes and topk 0 are no-ops even with NULL tensors
    assert call(N, N, N, N, 0, 2, 4, 16, 8, 64, 4, N) == sas.SAS_OK
    assert call(N, N, N, N, 1, 2, 4, 16, 8, 64, 0, N) == sas.SAS_OK
    assert call(v, v, v, N, 1, 2, 4, 16, 8, 64, 4, N) == sas.SAS_EINVAL
    assert "gates" in sas.sas_last_error()
    assert call(v, N, v, v, 1, 2, 4, 16, 8, 64, 4, N) == sas.SAS_EINVAL
    assert call(v, v, v, v, 1, 2, 0, 16, 8, 64, 4, N) == sas.SAS_EINVAL
    assert call(v, v, v, v, 1, 2, 4, 16, 8, 0, 4, N) == sas.SAS_EINVAL
    assert call(v, v, v, v, 1, 2, 4, 16, 8, 64, -1, N) == sas.SAS_EINVAL
    assert call(v, v, v, v, 1, 2, 4, 16, 1025, 64, 4, N) == sas.SAS_EUNSUPPORTED
    assert call(v, v, v, v, 1, 2, 4, 16, 8, 64, 65, N) == sas.SAS_EUNSUPPORTED
    assert call(v, v, v, v, 1, 2, 16, 16, 8, 64, 4, N) == sas.SAS_EUNSUPPORTED
    assert call(v, v, v, v, 1, 2, 3, 16, 8, 64, 4, N) == sas.SAS_EUNSUPPORTED
