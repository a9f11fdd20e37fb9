"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def normwise(got, ref, tol, what=""):
    """max|got - ref| <= tol * max|ref| over the finite entries of ref; -inf entries must match."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    inf = ~np.isfinite(ref)
    if inf.any():
        assert np.array_equal(got[inf], ref[inf]), f"{what}: non-finite entries differ"
    fin = ~inf
    if not fin.any():
        return 0.0
    scale = max(np.max(np.abs(ref[fin])), 1e-30)
    err = np.max(np.abs(got[fin] - ref[fin]))
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite output"
    assert err <= tol * scale, f"{what}: max err {err:.3e} > {tol:.1e} * {scale:.3e}"
    return err / scale


def max_abs(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
    return err


def tolerances(dtype):
    """(outputs, gradients, fp32 side outputs) tolerances.

    fp32 tensors: 1e-4 relative (normwise).  bf16 attention output: 2e-2
    absolute.  bf16 gradients and the fp32 ds computed from bf16 tensors: 2e-2
    normwise (a reading: the pages fix no bound for them).
    """
    if dtype == torch.float32:
        return dict(o_abs=None, o_rel=1e-4, grad=1e-4, lse=1e-4, ds=1e-4)
    return dict(o_abs=2e-2, o_rel=None, grad=2e-2, lse=1e-4, ds=2e-2)


def kbar_close(got, ref_rounded, what="kbar"):
    """Pooled keys: the fp32 mean rounded to bf16 may sit one bf16 step from the
    rounded exact mean, plus the fp32 summation error of 64 terms (absolute,
    matters only for means that nearly cancel)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref_rounded, dtype=np.float64)
    bad = np.abs(got - ref) > np.abs(ref) * 2.0 ** -7 + 1e-5
    assert not bad.any(), f"{what}: {bad.sum()} entries off, e.g. {got[bad][:3]} vs {ref[bad][:3]}"
