"""The seeded input generator: determinism, shapes and bf16 rounding."""
import numpy as np
import pytest

from exact_io_aware_12_amd import inputs as fi


def test_bf16_rounding_matches_torch_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000, dtype=np.float32) * 5,
                        np.array([1.0, -2.5, 3.0039062, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                  65504.0, 1e-30, -0.0], dtype=np.float32)])
    ours = fi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # Widening is exact.
    back = fi.bf16_bits_to_f64(ours)
    assert np.array_equal(back.astype(np.float32), torch.from_numpy(x).bfloat16().float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: even is 1.
    b = fi.f32_to_bf16_bits(np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32))
    assert fi.bf16_bits_to_f64(b).tolist() == [1.0, 1.0 + 2 ** -6]


@pytest.mark.parametrize("idx", [1, 2, 5])
def test_workload_draws_are_deterministic(idx):
    a = fi.make_inputs(idx)
    b = fi.make_inputs(idx)
    w = fi.WORKLOADS[idx]
    for name in ("q", "k", "v"):
        assert getattr(a, name).shape == w.shape
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert (a.do is not None) == w.backward


def test_key_scale_applied_before_rounding():
    w = fi.Workload("t", 1, 1, 64, 8, True, key_scale=3.0, seed=7)
    inp = fi.make_inputs(w, keep_f32=True)
    rng = np.random.default_rng(7)
    rng.standard_normal(w.shape, dtype=np.float32)
    k = rng.standard_normal(w.shape, dtype=np.float32) * np.float32(3.0)
    assert np.array_equal(inp.k, fi.f32_to_bf16_bits(k))


def test_flop_counts():
    w3 = fi.WORKLOADS[3]
    assert w3.fwd_flops() == pytest.approx(274.877906944e9)
    w5 = fi.WORKLOADS[5]
    assert w5.fwd_flops() == pytest.approx(34.359738368e9)
    assert w5.bwd_flops() == pytest.approx(85.89934592e9)


def test_decode_inputs_are_seeded():
    small = fi.DecodeWorkload("t", 1, 2, 3, 40, 64, True, seed=5)
    a = fi.make_decode_inputs(small)
    b = fi.make_decode_inputs(small)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert a[0].shape == (1, 2, 3, 64) and a[1].shape == (1, 2, 40, 64)
    assert a[0].dtype == np.uint16
    for w in fi.DECODE_WORKLOADS.values():
        assert w.Nq <= 32 and (not w.causal or w.Nq <= w.Nk)
