"""Helpers for the GPU parity tests: move seeded bf16 inputs to the GPU, run
the library through its binding, and compare with the fp64 oracle."""
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
