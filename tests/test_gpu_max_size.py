"""GPU parity at the largest sizes the entry points accept.

fa_fwd and fa_bwd take B*H*N*d up to 2^31 - 1 elements, i.e. tensors of up to
4 GiB, where head and row offsets leave the 32-bit signed range in bytes.
Every head below holds one of P seeded blocks (head h: block h % P, so heads
with the same inputs lie 4 GiB apart), which makes every head checkable:
  * every head's O, LSE, dQ, dK and dV are bit-identical to those of the
    first head that holds the same block (no head interacts with another, so
    any difference would be an addressing fault);
  * the first P heads and the last P heads are compared with the fp64 oracle
    to the stated tolerances (O 2e-2, LSE 1e-3, gradients 5e-2 max abs).
The persistent-grid forward must give the fused forward's O and LSE bit for
bit at the same size.
"""
import math

import pytest

import oracle
from exact_io_aware_12_amd import inputs as fi
from parity_util import (TOL_GRAD, TOL_LSE, TOL_O, assert_close, bits_to_f64, from_gpu,
                         to_gpu_bf16)

pytestmark = pytest.mark.gpu

P = 7   # distinct head blocks (prime, so blocks do not line up with the 8-XCD grouping)

# (B, H, N, d, causal): B*H*N*d = 2^31 - 128, the largest at d = 128 (ragged N,
# B*H odd: heads in plain order); 2^31 - 32768 with B*H a multiple of 8 (heads
# grouped per XCD); 2^31 - 64, the largest at d = 64.
MAX_CASES = [
    (21, 3133, 255, 128, True),
    (8, 8224, 255, 128, False),
    (31, 1801, 601, 64, True),
]


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_12_amd import fa as mod
    mod.library()
    return mod


@pytest.mark.parametrize("B,H,N,d,causal", MAX_CASES)
def test_max_size_fwd_bwd(fa, B, H, N, d, causal):
    import torch
    BH = B * H
    assert 0 <= 2**31 - 1 - BH * N * d < 32768   # at most 32768 elements below the limit
    print(f"[max size] B={B} H={H} N={N} d={d} causal={causal} elements={BH * N * d} "
          f"fwd={fa.fa_fwd_kernel_name(B, H, N, d, causal)} "
          f"bwd={fa.fa_bwd_kernel_name(B, H, N, d, causal)}", flush=True)
    seed = 31000 + N + d
    blocks = [fi.random_bf16((P, N, d), seed + i) for i in range(4)]   # Q, K, V, dO
    idx = torch.arange(BH, device="cuda") % P

    def spread(bits):
        return to_gpu_bf16(bits)[idx].view(B, H, N, d)

    q, k, v, do = (spread(b) for b in blocks)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    op, lsep = fa.fwd_persistent(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    del q, k, v, do

    outs = {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}
    for name, t in outs.items():
        flat = t.view(BH, -1)
        assert torch.equal(flat, flat[:P][idx]), \
            f"{name}: some head differs from the first head with the same inputs"
    assert torch.equal(op, o) and torch.equal(lsep, lse), "persistent forward differs"
    del op, lsep

    fq, fk, fv, fdo = (bits_to_f64(b) for b in blocks)
    ro, rl = oracle.attention_fwd(fq, fk, fv, scale, causal)
    rg = [oracle.attention_bwd(fq[m], fk[m], fv[m], fdo[m], scale, causal) for m in range(P)]
    heads = list(range(P)) + list(range(BH - P, BH))
    for h in heads:
        m = h % P
        got = {name: from_gpu(t.view(BH, *t.shape[2:])[h]) for name, t in outs.items()}
        assert_close(f"O[{h}]", got["O"], ro[m], TOL_O)
        assert_close(f"LSE[{h}]", got["LSE"], rl[m], TOL_LSE)
        for i, name in enumerate(("dQ", "dK", "dV")):
            assert_close(f"{name}[{h}]", got[name], rg[m][i], TOL_GRAD)


# Decode at the largest single-head cache: Nk = 2^24 - 1 keys at d = 128 and
# 2^25 - 1 at d = 64 (4 GiB per K and V tensor), so the key offsets within
# one head reach 4 GiB. The cache repeats a seeded block of pk keys c times
# (Nk = c * pk). Every distinct key then carries c times the weight of its
# single copy, so the softmax weights of the block, and O, are unchanged, and
# the LSE is the block's plus ln c: the oracle computes the block's O and LSE.
@pytest.mark.parametrize("d,pk", [(128, 255), (64, 601)])
def test_max_size_decode(fa, d, pk):
    import torch
    nk = (2**31 - 1) // d
    assert nk % pk == 0 and nk * d > 2**31 - 1 - d
    c, nq = nk // pk, 8
    print(f"[max size decode] Nq={nq} Nk={nk} d={d} block={pk} copies={c}", flush=True)
    seed = 32000 + d
    qb = fi.random_bf16((1, 1, nq, d), seed)
    kb = fi.random_bf16((1, 1, pk, d), seed + 1)
    vb = fi.random_bf16((1, 1, pk, d), seed + 2)
    idx = torch.arange(nk, device="cuda") % pk
    k = to_gpu_bf16(kb)[:, :, idx]
    v = to_gpu_bf16(vb)[:, :, idx]
    scale = 1 / math.sqrt(d)
    o, lse = fa.decode_fwd(to_gpu_bf16(qb), k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_decode(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), scale,
                                     False)
    assert_close("O", from_gpu(o), ro, TOL_O)
    assert_close("LSE", from_gpu(lse), rl + math.log(c), TOL_LSE)
