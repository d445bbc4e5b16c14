"""GPU parity of the unfused comparator (S and P in device memory: library
GEMMs around the hand-written row-softmax kernel) against the fp64 oracle,
through the C ABI. Same tolerances as the fused forward pass: O 2e-2, LSE 1e-3
(max abs)."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_12_amd import inputs as fi
from parity_util import TOL_LSE, TOL_O, assert_close, bits_to_f64, from_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_12_amd import fa as mod
    mod.library()
    return mod


def _check(fa, B, H, N, d, causal, seed, scale=None, kscale=1.0):
    import torch
    print(f"[unfused] B={B} H={H} N={N} d={d} causal={causal} seed={seed}", flush=True)
    shape = (B, H, N, d)
    qb = fi.random_bf16(shape, seed)
    kb = fi.random_bf16(shape, seed + 1, kscale)
    vb = fi.random_bf16(shape, seed + 2)
    scale = 1 / math.sqrt(d) if scale is None else scale
    q, k, v = to_gpu_bf16(qb), to_gpu_bf16(kb), to_gpu_bf16(vb)
    o, lse = fa.unfused_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), scale, causal)
    assert_close("O", from_gpu(o), ro, TOL_O)
    assert_close("LSE", from_gpu(lse), rl, TOL_LSE)


# N % 4 != 0 takes the scalar-load softmax path; N > 1024 several register
# chunks per thread.
SHAPES = [(1, 1, 1), (1, 2, 5), (2, 1, 100), (1, 3, 129), (1, 2, 1000), (1, 1, 1027),
          (1, 2, 4096)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", SHAPES)
def test_unfused_small(fa, B, H, N, d, causal):
    _check(fa, B, H, N, d, causal, seed=5000 + N + d)


def test_unfused_scales_and_peaked_rows(fa):
    _check(fa, 1, 2, 300, 128, True, seed=11, scale=0.0)
    _check(fa, 1, 2, 300, 64, False, seed=12, scale=-0.2)
    _check(fa, 1, 2, 513, 128, True, seed=13, kscale=3.0)


def test_unfused_long_rows(fa):
    """Rows longer than the register path (N > 16384) use the two-pass kernel."""
    _check(fa, 1, 1, 16389, 64, True, seed=14)


def test_unfused_matches_fused_workload_2(fa):
    """Workload 2 (B=4, H=16, N=1024, d=64): unfused vs oracle on every head,
    and unfused vs fused within the sum of their tolerances."""
    import torch
    inp = fi.make_inputs(2)
    w = inp.workload
    q, k, v = to_gpu_bf16(inp.q), to_gpu_bf16(inp.k), to_gpu_bf16(inp.v)
    o_u, l_u = fa.unfused_fwd(q, k, v, causal=w.causal, scale=w.scale)
    o_f, l_f = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    ou, lu = from_gpu(o_u), from_gpu(l_u)
    for b in range(w.B):
        for h in range(w.H):
            ro, rl = oracle.attention_fwd(bits_to_f64(inp.q[b, h]), bits_to_f64(inp.k[b, h]),
                                          bits_to_f64(inp.v[b, h]), w.scale, w.causal)
            assert_close(f"O[{b},{h}]", ou[b, h], ro, TOL_O)
            assert_close(f"LSE[{b},{h}]", lu[b, h], rl, TOL_LSE)
    assert np.abs(ou - from_gpu(o_f)).max() <= 2 * TOL_O
    assert np.abs(lu - from_gpu(l_f)).max() <= 2 * TOL_LSE
