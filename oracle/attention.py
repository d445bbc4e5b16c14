"""Plain fp64 attention (forward, backward, online recurrence) on the CPU.

Test infrastructure only; see the package docstring for who may call it.

Conventions shared by every function here:

* q, k, v, do are float64 arrays shaped [..., N, d] (leading batch/head axes
  are looped over one head at a time). They are the exact bf16 input values
  widened to float64.
* ``scale`` multiplies the raw dot products (page 1, section 4 writes the
  fixed 1/sqrt(d); here it is a parameter so scale = 0 can serve as a pin).
* ``causal``: query i may attend key j iff j <= i. The pages do not define a
  mask; this is the reading used throughout, with masked probabilities exactly
  zero.
* LSE is the natural-log logsumexp of the scaled, masked scores of a row,
  i.e. m + ln l with m the row max and l the sum of exp(s - m) (the two
  per-row statistics that page 1 section 5 keeps for the backward, folded
  into one number).
"""
from __future__ import annotations

import math

import numpy as np

_NEG_INF = -np.inf


def _heads(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x.reshape((-1,) + x.shape[-2:])


def _scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
            row0: int = 0) -> np.ndarray:
    """S = scale * q k^T for query rows row0.., with masked entries -inf.

    Page 1 section 1 (the N x N matrix S) and section 4 (S_ij = Q_i K_j^T
    scaled)."""
    s = scale * (q @ k.T)
    if causal:
        qi = np.arange(row0, row0 + q.shape[0])[:, None]
        kj = np.arange(k.shape[0])[None, :]
        s = np.where(kj <= qi, s, _NEG_INF)
    return s


def _row_lse(s: np.ndarray) -> np.ndarray:
    """ln sum_j exp(s_ij), computed around the row max (page 3, section
    19.12's stable softmax subtracts the row max before exp)."""
    m = s.max(axis=1)
    return m + np.log(np.exp(s - m[:, None]).sum(axis=1))


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float,
                    causal: bool) -> np.ndarray:
    """P = softmax(S) per row for one head (page 1 section 1's P)."""
    s = _scores(np.asarray(q, np.float64), np.asarray(k, np.float64), scale, causal)
    return np.exp(s - _row_lse(s)[:, None])


def _fwd_one_head(q, k, v, scale, causal, row_block):
    n = q.shape[0]
    o = np.empty_like(q)
    lse = np.empty(n)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        # Rows are independent: a block of rows sees every key it may attend
        # (for causal rows, keys up to its last row), so this is still the
        # plain definition, evaluated a slab of rows at a time.
        kend = r1 if causal else n
        s = _scores(q[r0:r1], k[:kend], scale, causal, row0=r0)
        l_rows = _row_lse(s)
        p = np.exp(s - l_rows[:, None])
        o[r0:r1] = p @ v[:kend]
        lse[r0:r1] = l_rows
    return o, lse


def attention_fwd(q, k, v, scale: float, causal: bool = False,
                  row_block: int = 1024):
    """Exact attention O = softmax(scale Q K^T) V and its per-row LSE.

    Page 1 section 1 / page 3 section 19.1 define O; page 1 section 5 keeps a
    per-row statistic instead of P. Returns (O [..., N, d], LSE [..., N])."""
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    lead = np.shape(q)[:-2]
    o = np.empty_like(qh)
    lse = np.empty(qh.shape[:2])
    for h in range(qh.shape[0]):
        o[h], lse[h] = _fwd_one_head(qh[h], kh[h], vh[h], scale, causal, row_block)
    return o.reshape(lead + qh.shape[1:]), lse.reshape(lead + (qh.shape[1],))


def attention_decode(q, k, v, scale: float, causal: bool = False):
    """Attention of Nq query rows against Nk key/value rows (a KV cache).

    The plain definition of page 1 section 1 with a rectangular S (Nq x Nk);
    the interview answer's bonus point names this use (inference with a KV
    cache). ``causal``: the queries are the last Nq positions of the
    sequence, so query i (position Nk - Nq + i) may attend key j iff
    j <= Nk - Nq + i; with Nq = Nk this is the square causal mask above.
    q: [..., Nq, d]; k, v: [..., Nk, d]. Returns (O [..., Nq, d], LSE [..., Nq])."""
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    lead = np.shape(q)[:-2]
    nq, nk = qh.shape[1], kh.shape[1]
    if causal and nq > nk:
        raise ValueError("causal decode needs Nq <= Nk")
    o = np.empty_like(qh)
    lse = np.empty(qh.shape[:2])
    for h in range(qh.shape[0]):
        s = _scores(qh[h], kh[h], scale, causal, row0=nk - nq)
        l_rows = _row_lse(s)
        o[h] = np.exp(s - l_rows[:, None]) @ vh[h]
        lse[h] = l_rows
    return o.reshape(lead + qh.shape[1:]), lse.reshape(lead + (nq,))


def _bwd_one_head(q, k, v, do, scale, causal, row_block):
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        kend = r1 if causal else n
        s = _scores(q[r0:r1], k[:kend], scale, causal, row0=r0)
        p = np.exp(s - _row_lse(s)[:, None])           # recomputed P (page 1 s.5)
        dov = do[r0:r1]
        dv[:kend] += p.T @ dov                          # dV = P^T dO
        dp = dov @ v[:kend].T                           # dP = dO V^T
        # Softmax backward: the row sum of P*dP runs over the WHOLE row of the
        # probability matrix (a per-tile sum, read literally from page 1's
        # per-tile listing, would not be the gradient).
        drow = (p * dp).sum(axis=1)
        ds = p * (dp - drow[:, None])
        dq[r0:r1] = scale * (ds @ k[:kend])             # dQ = scale dS K
        dk[:kend] += scale * (ds.T @ q[r0:r1])          # dK = scale dS^T Q
    return dq, dk, dv


def attention_bwd(q, k, v, do, scale: float, causal: bool = False,
                  row_block: int = 1024):
    """Gradients (dQ, dK, dV) of sum(O * dO) for O = attention_fwd(...)[0].

    Page 1 section 5: dV = P^T dO, dP = dO V^T, dS = P o (dP - rowsum(dP o P))
    times the scale, dQ = dS K, dK = dS^T Q."""
    qh, kh, vh, doh = _heads(q), _heads(k), _heads(v), _heads(do)
    outs = [np.empty_like(qh), np.empty_like(kh), np.empty_like(vh)]
    for h in range(qh.shape[0]):
        r = _bwd_one_head(qh[h], kh[h], vh[h], doh[h], scale, causal, row_block)
        for t, x in zip(outs, r):
            t[h] = x
    shp = np.shape(q)
    return tuple(t.reshape(shp) for t in outs)


def online_softmax_stream(row_scores, block_sizes):
    """Run the online-softmax recurrence over one row of raw scores.

    The row is consumed in consecutive blocks of the given sizes; after each
    block the running max m and running sum l are updated as page 2 ("2.
    Online Softmax") and page 3 (section 19.5) state:
    m_new = max(m, max of block), l = l * exp(m - m_new) + sum exp(block - m_new).
    Returns the list of (m, l, alpha) after each block and the final
    probabilities exp(s - m) / l."""
    s = np.asarray(row_scores, dtype=np.float64)
    m, l = -math.inf, 0.0
    hist = []
    pos = 0
    for b in block_sizes:
        blk = s[pos:pos + b]
        pos += b
        m_new = max(m, float(blk.max()))
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        l = l * alpha + float(np.exp(blk - m_new).sum())
        m = m_new
        hist.append((m, l, alpha))
    assert pos == s.size, "blocks must cover the row"
    return hist, np.exp(s - m) / l


def attention_tiled(q, k, v, scale: float, causal: bool = False,
                    q_tile: int = 4, k_tile: int = 4):
    """Tiled attention with the online-softmax recurrence, in fp64.

    Outer loop over query tiles, inner loop over key/value tiles (page 1
    section 4, "FlashAttention-2 style"; page 3 section 19.4). Per tile pair:
    scores, new running max, correction factor alpha = exp(m_old - m_new),
    p = exp(s - m_new) (the single-exponential form of page 2 and page 3
    section 19.12), l = alpha*l + rowsum p, acc = alpha*acc + p V_j. The
    output is normalised once per query tile. Returns (O, LSE)."""
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    lead = np.shape(q)[:-2]
    n, d = qh.shape[1:]
    out = np.empty_like(qh)
    lse = np.empty(qh.shape[:2])
    for h in range(qh.shape[0]):
        for i0 in range(0, n, q_tile):
            qi = qh[h, i0:i0 + q_tile]
            rows = qi.shape[0]
            m = np.full(rows, -np.inf)
            l = np.zeros(rows)
            acc = np.zeros((rows, d))
            for j0 in range(0, n, k_tile):
                kj, vj = kh[h, j0:j0 + k_tile], vh[h, j0:j0 + k_tile]
                s = scale * (qi @ kj.T)
                if causal:
                    ii = np.arange(i0, i0 + rows)[:, None]
                    jj = np.arange(j0, j0 + kj.shape[0])[None, :]
                    s = np.where(jj <= ii, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                # A row with no allowed key so far keeps m = -inf: take its
                # correction factor as 1 and its exponentials as 0.
                live = m_new > -np.inf
                m_sub = np.where(live, m_new, 0.0)
                alpha = np.where(live, np.exp(np.where(live, m - m_sub, 0.0)), 1.0)
                p = np.where(live[:, None], np.exp(s - m_sub[:, None]), 0.0)
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + p @ vj
                m = m_new
            out[h, i0:i0 + rows] = acc / l[:, None]
            lse[h, i0:i0 + rows] = m + np.log(l)
    return out.reshape(lead + qh.shape[1:]), lse.reshape(lead + (n,))


def attention_fwd_brute(q, k, v, scale: float, causal: bool = False):
    """Scalar-loop forward for tiny single-head inputs (no BLAS, no numpy
    reductions): for each row, the allowed scores, their max, the exp sum, the
    LSE and the weighted sum of value rows."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    o = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        allowed = [j for j in range(n) if (not causal or j <= i)]
        s = {}
        for j in allowed:
            acc = 0.0
            for c in range(d):
                acc += float(q[i, c]) * float(k[j, c])
            s[j] = scale * acc
        mx = max(s.values())
        tot = 0.0
        for j in allowed:
            tot += math.exp(s[j] - mx)
        lse[i] = mx + math.log(tot)
        for j in allowed:
            pj = math.exp(s[j] - lse[i])
            for c in range(d):
                o[i][c] += pj * float(v[j, c])
    return np.array(o), np.array(lse)


def attention_bwd_brute(q, k, v, do, scale: float, causal: bool = False):
    """Scalar-loop gradient for tiny single-head inputs, by the chain rule
    through S -> P -> O written element by element: dP_ij = dO_i . V_j,
    dS_ij = sum_t dP_it * dP_it/dS_ij with dP_it/dS_ij = P_it (delta_tj - P_ij),
    then dQ_i = scale sum_j dS_ij K_j, dK_j = scale sum_i dS_ij Q_i,
    dV_j = sum_i P_ij dO_i."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    n, d = q.shape
    _, lse = attention_fwd_brute(q, k, v, scale, causal)
    P = [[0.0] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            if causal and j > i:
                continue
            acc = 0.0
            for c in range(d):
                acc += float(q[i, c]) * float(k[j, c])
            P[i][j] = math.exp(scale * acc - lse[i])
    dq = [[0.0] * d for _ in range(n)]
    dk = [[0.0] * d for _ in range(n)]
    dv = [[0.0] * d for _ in range(n)]
    for i in range(n):
        dP = [0.0] * n
        for t in range(n):
            acc = 0.0
            for c in range(d):
                acc += float(do[i, c]) * float(v[t, c])
            dP[t] = acc
        for j in range(n):
            # Jacobian of one softmax row: dP_t/dS_j = P_t (delta_tj - P_j).
            g = 0.0
            for t in range(n):
                g += dP[t] * P[i][t] * ((1.0 if t == j else 0.0) - P[i][j])
            for c in range(d):
                dq[i][c] += scale * g * float(k[j, c])
                dk[j][c] += scale * g * float(q[i, c])
                dv[j][c] += P[i][j] * float(do[i, c])
    return np.array(dq), np.array(dk), np.array(dv)
