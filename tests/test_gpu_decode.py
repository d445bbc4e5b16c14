"""GPU parity of decode attention (Nq <= 32 query rows against an Nk-row KV
cache, keys split over workgroups and merged) against the fp64 oracle,
through the C ABI. Same tolerances as the forward pass: O 2e-2, LSE 1e-3."""
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


def _check(fa, B, H, Nq, Nk, d, causal, seed, scale=None, kscale=1.0):
    import torch
    print(f"[decode] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} seed={seed}", flush=True)
    qb = fi.random_bf16((B, H, Nq, d), seed)
    kb = fi.random_bf16((B, H, Nk, d), seed + 1, kscale)
    vb = fi.random_bf16((B, H, Nk, d), seed + 2)
    scale = 1 / math.sqrt(d) if scale is None else scale
    q, k, v = to_gpu_bf16(qb), to_gpu_bf16(kb), to_gpu_bf16(vb)
    o, lse = fa.decode_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_decode(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), scale,
                                     causal)
    assert_close("O", from_gpu(o), ro, TOL_O)
    assert_close("LSE", from_gpu(lse), rl, TOL_LSE)


# Nk spans one split and many (a split is >= 256 keys; B*H small -> many
# splits), ragged key tails (Nk % 32 != 0) and Nq from 1 to 32.
SHAPES = [(1, 1, 1, 1), (1, 2, 1, 37), (2, 3, 4, 300), (1, 1, 16, 1000), (1, 2, 32, 777),
          (2, 2, 1, 8192), (1, 1, 7, 5003)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Nq,Nk", SHAPES)
def test_decode_small(fa, B, H, Nq, Nk, d, causal):
    _check(fa, B, H, Nq, Nk, d, causal, seed=9000 + Nq + Nk + d)


def test_decode_scales_and_peaked_keys(fa):
    _check(fa, 1, 2, 4, 600, 128, True, seed=21, scale=0.0)
    _check(fa, 1, 2, 3, 600, 64, False, seed=22, scale=-0.3)
    _check(fa, 2, 2, 8, 2100, 128, True, seed=23, kscale=3.0)


def test_decode_equals_last_rows_of_fused_forward(fa):
    """The causal decode of the last Nq rows equals the fused forward's last
    rows on the same sequence (both against the oracle's tolerance)."""
    import torch
    B, H, N, d, nq = 1, 4, 1500, 128, 5
    qb, kb, vb = (fi.random_bf16((B, H, N, d), 31 + i) for i in range(3))
    q, k, v = to_gpu_bf16(qb), to_gpu_bf16(kb), to_gpu_bf16(vb)
    o_f, l_f = fa.fwd(q, k, v, causal=True)
    o_d, l_d = fa.decode_fwd(q[:, :, N - nq:].contiguous(), k, v, causal=True)
    torch.cuda.synchronize()
    assert np.abs(from_gpu(o_d) - from_gpu(o_f)[:, :, N - nq:]).max() <= 2 * TOL_O
    assert np.abs(from_gpu(l_d) - from_gpu(l_f)[:, :, N - nq:]).max() <= 2 * TOL_LSE


def test_decode_deterministic(fa):
    import torch
    q, k, v = (to_gpu_bf16(fi.random_bf16((2, 4, n, 128), 50 + i))
               for i, n in enumerate((4, 4096, 4096)))
    o1, l1 = fa.decode_fwd(q, k, v, causal=True)
    o2, l2 = fa.decode_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_long_cache_many_splits(fa):
    """A 500000-key cache on one head: about 2000 key splits merged."""
    _check(fa, 1, 1, 4, 500000, 128, True, seed=61)
