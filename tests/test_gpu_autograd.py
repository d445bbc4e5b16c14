"""fa.attention, the autograd operation over fa_fwd / fa_bwd: its forward
output is fa_fwd's O, and the gradients that autograd delivers for a loss
sum(O * dO) are exactly fa_bwd's dQ, dK, dV for that dO (the same kernels on
the same tensors), and within the stated bounds of the fp64 oracle's."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_12_amd import inputs as fi
from parity_util import TOL_GRAD, TOL_O, assert_close, bits_to_f64, from_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_12_amd import fa as mod
    mod.library()
    return mod


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 300, 128, True), (2, 1, 257, 64, False)])
def test_autograd_matches_entry_points_and_oracle(fa, B, H, N, d, causal):
    import torch
    print(f"[autograd] B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    shape = (B, H, N, d)
    seed = 9500 + N + d
    qb, kb, vb, dob = (fi.random_bf16(shape, seed + i) for i in range(4))
    q, k, v = (to_gpu_bf16(x).requires_grad_(True) for x in (qb, kb, vb))
    do = to_gpu_bf16(dob)
    scale = 1 / math.sqrt(d)

    o = fa.attention(q, k, v, causal=causal)
    (o.float() * do.float()).sum().backward()

    qd, kd, vd = (t.detach() for t in (q, k, v))
    o_ref, lse_ref = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o_ref, do, lse_ref, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for name, g, r in (("dQ", q.grad, dq), ("dK", k.grad, dk), ("dV", v.grad, dv)):
        assert g is not None and g.dtype == torch.bfloat16, name
        assert torch.equal(g, r), f"{name}: autograd gradient differs from fa_bwd"

    fq, fk, fv, fdo = (bits_to_f64(x) for x in (qb, kb, vb, dob))
    for b in range(B):
        for h in range(H):
            ro, _ = oracle.attention_fwd(fq[b, h], fk[b, h], fv[b, h], scale, causal)
            assert_close(f"O[{b},{h}]", from_gpu(o.detach())[b, h], ro, TOL_O)
            rg = oracle.attention_bwd(fq[b, h], fk[b, h], fv[b, h], fdo[b, h], scale, causal)
            for i, (name, g) in enumerate((("dQ", q.grad), ("dK", k.grad), ("dV", v.grad))):
                assert_close(f"{name}[{b},{h}]", from_gpu(g)[b, h], np.asarray(rg[i]), TOL_GRAD)


def test_autograd_gradient_of_other_dtype(fa):
    # An fp32 upstream gradient is converted to bf16 before fa_bwd.
    import torch
    shape = (1, 1, 130, 64)
    q, k, v = (to_gpu_bf16(fi.random_bf16(shape, 9700 + i)).requires_grad_(True)
               for i in range(3))
    w = torch.randn(shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(3))
    o = fa.attention(q, k, v, causal=True)
    (o.float() * w).sum().backward()
    o2, lse = fa.fwd(q.detach(), k.detach(), v.detach(), causal=True)
    dq, dk, dv = fa.bwd(q.detach(), k.detach(), v.detach(), o2, w.bfloat16(), lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
