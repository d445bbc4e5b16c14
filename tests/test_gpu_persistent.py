"""GPU parity of the persistent-grid forward comparator (fa_fwd_persistent:
at most two resident workgroups per CU looping over the query tiles in a
static snake order) against the fp64 oracle, and bit-for-bit against fa_fwd
on shapes where fa_fwd runs the same 128-row kernel (same arithmetic, same
order)."""
import math

import pytest

import oracle
from exact_io_aware_12_amd import inputs as fi
from parity_util import TOL_LSE, TOL_O, assert_close, bits_to_f64, from_gpu, map_heads, to_gpu_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_12_amd import fa as mod
    mod.library()
    return mod


def _inputs(B, H, N, d, seed):
    shape = (B, H, N, d)
    return [fi.random_bf16(shape, seed + i) for i in range(3)]


# Items = 128-row query tiles x heads. Fewer than 512 items: one per
# workgroup; more: several rounds of the snake. Heads a multiple of 8: the
# snake runs within each XCD's heads; otherwise over all items.
@pytest.mark.parametrize("B,H,N,d,causal,scale", [
    (1, 1, 1, 64, True, None),
    (1, 3, 200, 128, False, None),
    (2, 4, 511, 64, True, 0.37),
    (1, 2, 1000, 128, True, -0.2),
    (1, 2, 300, 64, False, 0.0),
    (2, 8, 4100, 128, True, None),      # 33 x 16 = 528 items: two rounds, heads grouped by XCD
    (1, 5, 13000, 64, False, None),     # 102 x 5 = 510 items, heads not grouped
])
def test_persistent_matches_oracle(fa, B, H, N, d, causal, scale):
    import torch
    print(f"[persistent] B={B} H={H} N={N} d={d} causal={causal} scale={scale}", flush=True)
    qb, kb, vb = _inputs(B, H, N, d, 9000 + N + d)
    sc = 1 / math.sqrt(d) if scale is None else scale
    q, k, v = (to_gpu_bf16(x) for x in (qb, kb, vb))
    o, lse = fa.fwd_persistent(q, k, v, causal=causal, scale=sc)
    torch.cuda.synchronize()
    o_np, l_np = from_gpu(o), from_gpu(lse)
    fq, fk, fv = (bits_to_f64(x) for x in (qb, kb, vb))
    heads = [(b, h) for b in range(B) for h in range(H)]
    for (b, h), (ro, rl) in zip(heads, map_heads(
            lambda bh: oracle.attention_fwd(fq[bh], fk[bh], fv[bh], sc, causal), heads)):
        assert_close(f"O[{b},{h}]", o_np[b, h], ro, TOL_O)
        assert_close(f"LSE[{b},{h}]", l_np[b, h], rl, TOL_LSE)


# Shapes where fa_fwd itself runs "fa_fwd_kernel" (one 128-row workgroup per
# query tile): the comparator computes each tile with the same code, so the
# outputs are identical. Includes several rounds per workgroup, with and
# without the per-XCD head grouping, and a ragged last tile.
@pytest.mark.parametrize("B,H,N,d,causal", [
    (2, 32, 4096, 128, True),     # the causal workload-3 shape: 2048 items, 4 per workgroup
    (1, 5, 16400, 64, True),      # 645 items, heads not grouped by XCD
    (4, 16, 2000, 128, False),    # 1024 items
    # One-round causal grids, where fa_fwd places a heavy and a light tile on
    # each CU (the dispatch order differs from the comparator's): every tile
    # of every head must still be computed exactly once.
    (2, 16, 2048, 128, True),     # 512 items
    (1, 24, 2000, 128, True),     # 384 items: a partial second pass
    (3, 8, 1500, 64, True),       # 288 items, d = 64
])
def test_persistent_equals_fused_forward(fa, B, H, N, d, causal):
    import torch
    assert fa.fa_fwd_kernel_name(B, H, N, d, causal) == "fa_fwd_kernel"
    print(f"[persistent=fwd] B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(N + d)
    q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").bfloat16() for _ in range(3))
    o1, l1 = fa.fwd(q, k, v, causal=causal)
    o2, l2 = fa.fwd_persistent(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
