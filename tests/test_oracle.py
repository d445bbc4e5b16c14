"""Pins of the fp64 oracle against values fixed by the pages and by mathematics.

None of these re-types the oracle's formula: each compares it with a closed
form, the pages' worked example, an invariant of softmax attention, scalar
brute force, central finite differences or a library route (torch's CPU
softmax + autograd). The last group plants plausible mistakes in copies of
the oracle and checks that some pin rejects each one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- worked example
def test_worked_example_online_stream(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    # The fixture's decimals are the closed forms it states.
    e = math.exp
    assert g["after_block_1"]["l"] == pytest.approx(1 + e(-1), abs=1e-15)
    assert g["alpha_block_2"]["value"] == pytest.approx(e(-2), abs=1e-15)
    assert g["final"]["lse"] == pytest.approx(4 + math.log(1 + e(-1) + e(-2) + e(-3)), abs=1e-15)
    hist, p = oracle.online_softmax_stream(g["row_scores"], g["blocks"])
    (m1, l1, _), (m2, l2, a2) = hist
    assert m1 == g["after_block_1"]["m"]
    assert abs(l1 - g["after_block_1"]["l"]) <= 1e-15
    assert abs(a2 - g["alpha_block_2"]["value"]) <= 1e-15
    assert m2 == g["final"]["m"]
    assert abs(l2 - g["final"]["l"]) <= 1e-15
    assert np.abs(p - np.array(g["final"]["p"])).max() <= 1e-15
    # One-shot softmax of the whole row gives the same probabilities.
    s = np.array(g["row_scores"])
    one_shot = np.exp(s) / np.exp(s).sum()
    assert np.abs(p - one_shot).max() <= 1e-15


def test_worked_example_as_attention(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    n, d = 4, 64
    q = np.zeros((n, d)); q[0, 0] = 1.0
    for i in range(1, n):
        q[i, 0] = i + 1.0
    k = np.zeros((n, d))
    for j in range(n):
        k[j, 0] = j + 1.0
    v = np.zeros((n, d))
    for j in range(n):
        v[j, j] = 1.0
    for fn in (oracle.attention_fwd,
               lambda *a: oracle.attention_tiled(*a, q_tile=1, k_tile=2)):
        o, lse = fn(q, k, v, 1.0, False)
        assert abs(lse[0] - g["final"]["lse"]) <= 1e-14
        assert np.abs(o[0, :4] - np.array(g["final"]["p"])).max() <= 1e-15
        assert np.abs(o[0, 4:]).max() == 0.0
        # Row i has scores (i+1)(j+1): a closed form per row.
        for i in range(n):
            sc = np.array([(i + 1.0) * (j + 1.0) for j in range(n)])
            ref = np.exp(sc - sc.max()); ref /= ref.sum()
            assert np.abs(o[i, :4] - ref).max() <= 1e-14


# ---------------------------------------------------------------- tiled == untiled
def test_simulator_check_pattern(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "simulator_check.json")))
    rng = np.random.default_rng(g["seed"])
    Q = rng.normal(size=g["shape"]); K = rng.normal(size=g["shape"]); V = rng.normal(size=g["shape"])
    scale = 1.0 / math.sqrt(g["shape"][1])
    o, _ = oracle.attention_fwd(Q, K, V, scale)
    t, _ = oracle.attention_tiled(Q, K, V, scale, q_tile=g["q_tile"], k_tile=g["k_tile"])
    assert np.abs(o - t).max() < g["max_abs_diff_below"]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", [(4, 4), (5, 7), (32, 64), (128, 13), (1, 128)])
def test_tiled_equals_untiled(causal, tiles):
    n, d = 128, 64
    q, k, v = _rand((n, d), 1), _rand((n, d), 2, 3.0), _rand((n, d), 3)
    o, lse = oracle.attention_fwd(q, k, v, 0.125, causal, row_block=40)
    t, tl = oracle.attention_tiled(q, k, v, 0.125, causal, *tiles)
    assert np.abs(o - t).max() <= 1e-12
    assert np.abs(lse - tl).max() <= 1e-12


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k = _rand((97, 16), 4), _rand((97, 16), 5, 3.0)
    p = oracle.attention_probs(q, k, 0.25, causal)
    assert np.abs(p.sum(axis=1) - 1).max() <= 1e-14
    assert (p >= 0).all()
    if causal:
        assert (np.triu(p, 1) == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_identical_key_rows_give_mean_of_v(causal):
    n, d = 50, 8
    q = _rand((n, d), 6)
    k = np.tile(_rand((1, d), 7), (n, 1))
    v = _rand((n, d), 8)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, causal)
    if causal:
        ref = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
        cnt = np.arange(1, n + 1)
    else:
        ref = np.broadcast_to(v.mean(axis=0), v.shape)
        cnt = np.full(n, n)
    assert np.abs(o - ref).max() <= 1e-14
    s0 = 0.3 * (q @ k[0])
    assert np.abs(lse - (s0 + np.log(cnt))).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_o(causal):
    n, d = 64, 16
    q, k = _rand((n, d), 9), _rand((n, d), 10, 3.0)
    c = _rand((1, d), 11)
    o, _ = oracle.attention_fwd(q, k, np.tile(c, (n, 1)), 0.25, causal)
    assert np.abs(o - c).max() <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_closed_form(causal):
    n, d = 70, 8
    q, k, v = _rand((n, d), 12), _rand((n, d), 13), _rand((n, d), 14)
    o, lse = oracle.attention_fwd(q, k, v, 0.0, causal, row_block=16)
    if causal:
        assert np.abs(o - np.cumsum(v, 0) / np.arange(1, n + 1)[:, None]).max() <= 1e-14
        assert np.abs(lse - np.log(np.arange(1, n + 1))).max() <= 1e-14
    else:
        assert np.abs(o - v.mean(0)).max() <= 1e-14
        assert np.abs(lse - math.log(n)).max() <= 1e-14


def test_causal_row_zero_single_key():
    q, k, v = _rand((33, 8), 15), _rand((33, 8), 16), _rand((33, 8), 17)
    o, lse = oracle.attention_fwd(q, k, v, 0.7, True)
    assert np.abs(o[0] - v[0]).max() == 0.0
    assert abs(lse[0] - 0.7 * float(q[0] @ k[0])) <= 1e-15


def test_causal_last_row_equals_noncausal_last_row():
    q, k, v = _rand((40, 8), 18), _rand((40, 8), 19), _rand((40, 8), 20)
    oc, lc = oracle.attention_fwd(q, k, v, 0.5, True)
    on, ln = oracle.attention_fwd(q, k, v, 0.5, False)
    assert np.abs(oc[-1] - on[-1]).max() <= 1e-14 and abs(lc[-1] - ln[-1]) <= 1e-14


def test_key_permutation_invariance():
    n, d = 60, 8
    q, k, v = _rand((n, d), 21), _rand((n, d), 22), _rand((n, d), 23)
    perm = np.random.default_rng(24).permutation(n)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.4, False)
    o2, l2 = oracle.attention_fwd(q, k[perm], v[perm], 0.4, False)
    assert np.abs(o1 - o2).max() <= 1e-14 and np.abs(l1 - l2).max() <= 1e-14


def test_batched_heads_match_single_heads():
    q, k, v = _rand((2, 3, 20, 8), 25), _rand((2, 3, 20, 8), 26), _rand((2, 3, 20, 8), 27)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, True)
    for b in range(2):
        for h in range(3):
            o1, l1 = oracle.attention_fwd(q[b, h], k[b, h], v[b, h], 0.3, True)
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], l1)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (7, 5), (16, 8)])
def test_forward_matches_brute_force(causal, n, d):
    q, k, v = _rand((n, d), 30 + n), _rand((n, d), 31 + n, 3.0), _rand((n, d), 32 + n)
    o, lse = oracle.attention_fwd(q, k, v, 0.35, causal, row_block=3)
    ob, lb = oracle.attention_fwd_brute(q, k, v, 0.35, causal)
    assert np.abs(o - ob).max() <= 1e-13
    assert np.abs(lse - lb).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (7, 5), (12, 8)])
def test_backward_matches_brute_force(causal, n, d):
    q, k, v, do = (_rand((n, d), 40 + i) for i in range(4))
    g = oracle.attention_bwd(q, k, v, do, 0.35, causal, row_block=5)
    gb = oracle.attention_bwd_brute(q, k, v, do, 0.35, causal)
    for a, b in zip(g, gb):
        assert np.abs(a - b).max() <= 1e-13


# ---------------------------------------------------------------- finite differences
def _fd_grads(fwd, q, k, v, do, scale, causal, h=1e-6):
    def loss(qq, kk, vv):
        return float((fwd(qq, kk, vv, scale, causal)[0] * do).sum())
    out = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(g.shape):
            plus = [x.copy() for x in base]; minus = [x.copy() for x in base]
            plus[which][idx] += h; minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        out.append(g)
    return out


def _fd_error(bwd, causal, n=7, d=5, scale=0.45):
    q, k, v, do = (_rand((n, d), 50 + i) for i in range(4))
    fd = _fd_grads(oracle.attention_fwd, q, k, v, do, scale, causal)
    an = bwd(q, k, v, do, scale, causal)
    return max(np.abs(a - b).max() for a, b in zip(an, fd))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    assert _fd_error(oracle.attention_bwd, causal) <= 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    n, d = 80, 16
    q, k, v, do = (_rand((n, d), 60 + i) for i in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.25, causal, row_block=24)
    o, _ = oracle.attention_fwd(q, k, v, 0.25, causal)
    # Softmax rows sum to one, so shifting every key by the same vector leaves
    # every output unchanged: the key gradients sum to zero.
    assert np.abs(dk.sum(axis=0)).max() <= 1e-12
    # Columns of P summed over keys give one per query: sum_j dV_j = sum_i dO_i.
    assert np.abs(dv.sum(axis=0) - do.sum(axis=0)).max() <= 1e-12
    # Shifting all queries by t changes row scores by scale*t.k_j: dQ is
    # orthogonal to nothing in particular, but scaling Q by (1+e) gives
    # d/de sum(O*dO) = sum(dQ * Q) (directional derivative, checked by FD).
    f = lambda s: float((oracle.attention_fwd(q * s, k, v, 0.25, causal)[0] * do).sum())
    dir_fd = (f(1 + 1e-6) - f(1 - 1e-6)) / 2e-6
    assert abs(dir_fd - float((dq * q).sum())) <= 1e-6


def test_backward_D_equals_dO_dot_O():
    n, d = 50, 8
    q, k, v, do = (_rand((n, d), 70 + i) for i in range(4))
    p = oracle.attention_probs(q, k, 0.3, True)
    o, _ = oracle.attention_fwd(q, k, v, 0.3, True)
    dp = do @ v.T
    assert np.abs((p * dp).sum(1) - (do * o).sum(1)).max() <= 1e-13


# ---------------------------------------------------------------- library route
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_cpu_softmax_autograd(causal):
    torch = pytest.importorskip("torch")
    n, d = 33, 16
    q, k, v, do = (_rand((2, n, d), 80 + i) for i in range(4))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = 0.2 * tq @ tk.transpose(-1, -2)
    if causal:
        mask = torch.ones(n, n, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    lse = torch.logsumexp(s, dim=-1)
    (o * torch.tensor(do)).sum().backward()
    oo, ll = oracle.attention_fwd(q, k, v, 0.2, causal)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.2, causal)
    assert np.abs(oo - o.detach().numpy()).max() <= 1e-12
    assert np.abs(ll - lse.detach().numpy()).max() <= 1e-12
    for a, t in zip((dq, dk, dv), (tq, tk, tv)):
        assert np.abs(a - t.grad.numpy()).max() <= 1e-12


# ---------------------------------------------------------------- planted mistakes
def _bwd_per_tile_rowsum(q, k, v, do, scale, causal, tile=2):
    """Planted mistake: the row sum of P*dP taken per key tile (the literal
    reading of page 1's per-tile listing) instead of over the whole row."""
    p = oracle.attention_probs(q, k, scale, causal)
    dp = do @ v.T
    ds = np.zeros_like(p)
    for j0 in range(0, p.shape[1], tile):
        sl = slice(j0, j0 + tile)
        ds[:, sl] = p[:, sl] * (dp[:, sl] - (p[:, sl] * dp[:, sl]).sum(1, keepdims=True))
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _bwd_missing_scale_in_dk(q, k, v, do, scale, causal):
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    return dq, dk / scale, dv


def _bwd_transposed_dv(q, k, v, do, scale, causal):
    p = oracle.attention_probs(q, k, scale, causal)
    dq, dk, _ = oracle.attention_bwd(q, k, v, do, scale, causal)
    return dq, dk, p @ do


@pytest.mark.parametrize("mutant", [_bwd_per_tile_rowsum, _bwd_missing_scale_in_dk,
                                    _bwd_transposed_dv])
def test_planted_backward_mistakes_fail_finite_differences(mutant):
    assert _fd_error(mutant, True) > 1e-3


def test_planted_missing_rescale_fails_tiled_pin(monkeypatch):
    real_exp = np.exp
    # Planted mistake: the correction factor alpha forced to 1 (old terms never
    # rescaled when the running max grows).
    def tiled_no_rescale(q, k, v, scale, causal, q_tile, k_tile):
        n, d = q.shape
        out = np.empty_like(q)
        for i0 in range(0, n, q_tile):
            qi = q[i0:i0 + q_tile]
            m = np.full(qi.shape[0], -np.inf); l = np.zeros(qi.shape[0]); acc = np.zeros((qi.shape[0], d))
            for j0 in range(0, n, k_tile):
                s = scale * qi @ k[j0:j0 + k_tile].T
                m_new = np.maximum(m, s.max(1))
                p = real_exp(s - m_new[:, None])
                l = l + p.sum(1); acc = acc + p @ v[j0:j0 + k_tile]; m = m_new
            out[i0:i0 + q_tile] = acc / l[:, None]
        return out
    q, k, v = _rand((16, 8), 90), _rand((16, 8), 91, 3.0), _rand((16, 8), 92)
    o, _ = oracle.attention_fwd(q, k, v, 0.35, False)
    assert np.abs(tiled_no_rescale(q, k, v, 0.35, False, 4, 4) - o).max() > 1e-3


def test_planted_wrong_mask_fails_row_zero_pin():
    # Planted mistake: causal mask off by one (j < i): row 0 would have no key.
    q, k = _rand((8, 4), 93), _rand((8, 4), 94)
    s = 0.5 * q @ k.T
    wrong = np.where(np.arange(8)[None, :] < np.arange(8)[:, None] + 2, s, -np.inf)  # j <= i+1
    p = np.exp(wrong - wrong.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    assert abs(p[0, 0] - 1.0) > 1e-3  # the pin demands p[0,0] == 1 (O_0 == V_0)


# ---------------------------------------------------------------- decode (Nq x Nk)
@pytest.mark.parametrize("nq", [1, 3, 16])
def test_decode_rows_are_the_last_rows_of_causal_attention(nq):
    """Causal decode of the last Nq queries equals the last Nq rows of the
    full (square, pinned) causal attention over the same sequence."""
    rng = np.random.default_rng(70 + nq)
    n, d = 40, 8
    q, k, v = (rng.standard_normal((2, n, d)) for _ in range(3))
    o_full, l_full = oracle.attention_fwd(q, k, v, 0.4, causal=True)
    o, l = oracle.attention_decode(q[:, n - nq:], k, v, 0.4, causal=True)
    assert np.abs(o - o_full[:, n - nq:]).max() < 1e-12
    assert np.abs(l - l_full[:, n - nq:]).max() < 1e-12


def test_decode_noncausal_matches_scalar_loops():
    """Rectangular non-causal case against scalar loops over every key."""
    rng = np.random.default_rng(71)
    nq, nk, d = 3, 11, 5
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    o, l = oracle.attention_decode(q, k, v, 0.7, causal=False)
    for i in range(nq):
        s = [0.7 * sum(float(q[i, c]) * float(k[j, c]) for c in range(d)) for j in range(nk)]
        mx = max(s)
        tot = sum(math.exp(x - mx) for x in s)
        assert abs(l[i] - (mx + math.log(tot))) < 1e-12
        for c in range(d):
            ref = sum(math.exp(s[j] - mx) / tot * float(v[j, c]) for j in range(nk))
            assert abs(o[i, c] - ref) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_decode_scale_zero_closed_form(causal):
    """scale = 0: every admissible key has weight 1/count, so O is the mean of
    the admissible V rows and LSE = ln(count); query i of Nq (causal) admits
    keys 0 .. Nk - Nq + i."""
    rng = np.random.default_rng(72)
    nq, nk, d = 4, 9, 3
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    o, l = oracle.attention_decode(q, k, v, 0.0, causal=causal)
    for i in range(nq):
        cnt = (nk - nq + i + 1) if causal else nk
        assert np.abs(o[i] - v[:cnt].mean(axis=0)).max() < 1e-12
        assert abs(l[i] - math.log(cnt)) < 1e-12


def test_planted_decode_offset_mistake_fails_last_rows_pin(monkeypatch):
    """A query offset one position off (row0 = Nk - Nq + 1) must fail the
    last-rows pin."""
    orig = oa._scores

    def shifted(q, k, scale, causal, row0=0):
        return orig(q, k, scale, causal, row0=row0 + 1 if q.shape[0] != k.shape[0] else row0)

    monkeypatch.setattr(oa, "_scores", shifted)
    with pytest.raises(AssertionError):
        test_decode_rows_are_the_last_rows_of_causal_attention(3)
