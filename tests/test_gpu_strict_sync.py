"""Race check of the LDS staging: the normal library against its race-check
build (libfa355_strict.so, compiled with FA_STRICT_SYNC: every global -> LDS
copy is awaited by its wave as soon as it is issued, so copies never overlap
any later instruction). Both builds compute the same arithmetic in the same
order, so their outputs must be bit-identical; a copy racing with a read of
its buffer in the normal build would show as a difference. Shapes cover every
kernel variant (asserted by name) and ragged tails."""
import ctypes
import math
import os

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRICT = os.path.join(ROOT, "exact_io_aware_12_amd", "libfa355_strict.so")


@pytest.fixture(scope="module")
def libs():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_12_amd import fa
    assert os.path.exists(STRICT), "libfa355_strict.so is missing: build first"
    return fa, fa.library(), fa.load_build(STRICT)


def _rand(shape, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda").bfloat16()


def _fwd(lib, q, k, v, causal, scale):
    import torch
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    s = torch.cuda.current_stream().cuda_stream
    rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N,
                    d, scale, int(causal), s)
    assert rc == 0, rc
    return o, lse


def _bwd(lib, fa, q, k, v, o, do, lse, causal, scale):
    import torch
    B, H, N, d = q.shape
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), device=q.device, dtype=torch.uint8)
    g = [torch.empty_like(q) for _ in range(3)]
    s = torch.cuda.current_stream().cuda_stream
    rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                    lse.data_ptr(), g[0].data_ptr(), g[1].data_ptr(), g[2].data_ptr(), ws.data_ptr(),
                    ws.numel(), B, H, N, d, scale, int(causal), s)
    assert rc == 0, rc
    return g


@pytest.mark.parametrize("B,H,N,d,causal,fwd_kernel", [
    (2, 16, 2048, 128, True, "fa_fwd_kernel"),                                      # workload 5
    (1, 3, 1000, 64, False, "fa_fwd_kernel"),                                       # ragged, d = 64
    (1, 16, 8200, 128, True, "fa_fwd_pp_kernel"),                                   # two-group kernel
    (1, 2, 3000, 128, True, "fa_fwd_pp_kernel (keys split between the groups)"),
    (1, 9, 4100, 128, True,
     "fa_fwd_pp_kernel (keys split between the groups, two query tiles per workgroup)"),
    (1, 2, 3000, 64, False, "fa_fwd_kernel (keys split between two groups)"),
    (4, 33, 500, 128, True, "fa_fwd_kernel"),                                       # unsplit causal dQ
    (1, 33, 1000, 64, False, "fa_fwd_kernel"),                                      # unsplit non-causal dQ
])
def test_strict_build_is_bit_identical(libs, B, H, N, d, causal, fwd_kernel):
    import torch
    fa, lib, strict = libs
    assert fa.fa_fwd_kernel_name(B, H, N, d, causal) == fwd_kernel
    print(f"[strict] B={B} H={H} N={N} d={d} causal={causal} fwd={fwd_kernel} "
          f"bwd={fa.fa_bwd_kernel_name(B, H, N, d, causal)}", flush=True)
    shape = (B, H, N, d)
    q, k, v, do = (_rand(shape, 100 * N + d + i) for i in range(4))
    scale = 1 / math.sqrt(d)
    o1, l1 = _fwd(lib, q, k, v, causal, scale)
    o2, l2 = _fwd(strict, q, k, v, causal, scale)
    g1 = _bwd(lib, fa, q, k, v, o1, do, l1, causal, scale)
    g2 = _bwd(strict, fa, q, k, v, o1, do, l1, causal, scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "forward differs between builds"
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        assert torch.equal(a, b), f"{name} differs between builds"


def test_strict_build_decode_is_bit_identical(libs):
    import torch
    fa, lib, strict = libs
    B, H, Nq, Nk, d = 2, 4, 8, 20000, 128
    q, k, v = _rand((B, H, Nq, d), 1), _rand((B, H, Nk, d), 2), _rand((B, H, Nk, d), 3)
    outs = []
    for L in (lib, strict):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), device="cuda", dtype=torch.float32)
        ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d), device="cuda", dtype=torch.uint8)
        rc = L.fa_decode_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             ws.data_ptr(), ws.numel(), B, H, Nq, Nk, d, 1 / math.sqrt(d), 1,
                             torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
