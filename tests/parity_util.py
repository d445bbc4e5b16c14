"""Helpers for the GPU parity tests: move seeded bf16 inputs to the GPU, run
the library through its binding, and compare with the fp64 oracle."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TOL_O = 2e-2      # max abs error on O (bf16 output, fp32 accumulation)
TOL_LSE = 1e-3    # max abs error on the per-row logsumexp
TOL_GRAD = 5e-2   # max abs error on dQ, dK, dV


def to_gpu_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def bits_to_f64(bits):
    u = np.asarray(bits).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def from_gpu(t) -> np.ndarray:
    """bf16 or fp32 GPU tensor -> float64 numpy."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def err_report(name, got, ref):
    e = np.abs(got - ref)
    fro = np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    return f"{name}: max {e.max():.3e} mean {e.mean():.3e} relfro {fro:.3e}"


def assert_close(name, got, ref, tol):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    e = float(np.abs(got - ref).max()) if got.size else 0.0
    print(err_report(name, got, ref) if got.size else f"{name}: empty", flush=True)
    assert e <= tol, f"{name}: max abs error {e:.3e} > {tol:.1e}"


def map_heads(fn, items, workers=None):
    """fn over items on a thread pool (the oracle's BLAS calls and element-wise
    NumPy work release the GIL), results in order."""
    workers = workers or max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


# Relative form of the gradient bound, for scales other than 1/sqrt(d). The
# stated 5e-2 bound is about 1.4-2.4 % of the largest fp64 gradient at
# 1/sqrt(d) on N(0,1) draws (|dQ|, |dK| <= 2.1, |dV| <= 3.5); larger scales
# give larger gradients, and the kernel's bf16 roundings of P, dS and the
# output scale with them. The check: max abs error <= 2e-2 * max |ref| (and
# never tighter than the absolute bound), and the relative Frobenius error
# <= 1e-2.
REL_GRAD_MAX = 2e-2
REL_GRAD_FRO = 1e-2


def assert_close_rel(name, got, ref):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    print(err_report(name, got, ref), flush=True)
    amax = float(np.abs(ref).max()) if ref.size else 0.0
    e = float(np.abs(got - ref).max()) if got.size else 0.0
    bound = max(TOL_GRAD, REL_GRAD_MAX * amax)
    assert e <= bound, f"{name}: max abs error {e:.3e} > {bound:.3e} (max |ref| {amax:.3e})"
    nref = np.linalg.norm(ref.ravel())
    if nref > 0:
        fro = np.linalg.norm((got - ref).ravel()) / nref
        assert fro <= REL_GRAD_FRO, f"{name}: relative Frobenius error {fro:.3e} > {REL_GRAD_FRO}"
