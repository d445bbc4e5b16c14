"""GPU parity of the loop-order comparator (outer loop over key/value tiles,
one workgroup per head, running state in device memory) against the fp64
oracle, through the C ABI. Same tolerances as the fused forward pass: O 2e-2,
LSE 1e-3 (max abs)."""
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
    print(f"[fa1] B={B} H={H} N={N} d={d} causal={causal} seed={seed}", flush=True)
    shape = (B, H, N, d)
    qb = fi.random_bf16(shape, seed)
    kb = fi.random_bf16(shape, seed + 1, kscale)
    vb = fi.random_bf16(shape, seed + 2)
    scale = 1 / math.sqrt(d) if scale is None else scale
    q, k, v = to_gpu_bf16(qb), to_gpu_bf16(kb), to_gpu_bf16(vb)
    # The workspace starts as garbage: the kernel must not read state it has
    # not written.
    ws = torch.full((fa.fa_fa1_workspace_bytes(B, H, N, d) // 4,), float("nan"),
                    device="cuda", dtype=torch.float32)
    o, lse = fa.fa1_fwd(q, k, v, causal=causal, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), scale, causal)
    assert_close("O", from_gpu(o), ro, TOL_O)
    assert_close("LSE", from_gpu(lse), rl, TOL_LSE)


# Ragged in both tile sizes (64 keys, 128 queries), a single row, several
# query tiles whose waves start past a causal key tile.
SHAPES = [(1, 1, 1), (1, 2, 5), (2, 1, 100), (1, 3, 129), (1, 2, 200), (1, 1, 1027),
          (1, 2, 2048)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", SHAPES)
def test_fa1_small(fa, B, H, N, d, causal):
    _check(fa, B, H, N, d, causal, seed=7000 + N + d)


def test_fa1_scales_and_peaked_rows(fa):
    _check(fa, 1, 2, 300, 128, True, seed=21, scale=0.0)
    _check(fa, 1, 2, 300, 64, False, seed=22, scale=-0.2)
    _check(fa, 1, 2, 513, 128, True, seed=23, kscale=3.0)


def test_fa1_matches_fused_workload_3(fa):
    """Workload 3 (B=2, H=32, N=4096, d=128, causal): comparator vs fused on
    every element within the sum of their tolerances, and vs the oracle on
    two heads."""
    import torch
    inp = fi.make_inputs(3)
    w = inp.workload
    q, k, v = to_gpu_bf16(inp.q), to_gpu_bf16(inp.k), to_gpu_bf16(inp.v)
    o_1, l_1 = fa.fa1_fwd(q, k, v, causal=w.causal, scale=w.scale)
    o_f, l_f = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o1, l1 = from_gpu(o_1), from_gpu(l_1)
    assert np.abs(o1 - from_gpu(o_f)).max() <= 2 * TOL_O
    assert np.abs(l1 - from_gpu(l_f)).max() <= 2 * TOL_LSE
    for b, h in [(0, 0), (1, 31)]:
        ro, rl = oracle.attention_fwd(bits_to_f64(inp.q[b, h]), bits_to_f64(inp.k[b, h]),
                                      bits_to_f64(inp.v[b, h]), w.scale, w.causal)
        assert_close(f"O[{b},{h}]", o1[b, h], ro, TOL_O)
        assert_close(f"LSE[{b},{h}]", l1[b, h], rl, TOL_LSE)
