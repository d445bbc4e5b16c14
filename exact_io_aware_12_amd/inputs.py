"""Seeded synthetic inputs for fused exact attention.

This module holds no attention arithmetic. It draws the Q, K, V (and dO)
tensors of the five benchmark workloads and rounds them to bfloat16, so the
HIP path and the fp64 oracle see bit-identical input values. Nothing here
knows how attention is computed; both sides import it, neither side is
imported by it.

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream per workload):
draw Q, then K, then V, then dO (backward workloads only), each as
``standard_normal([B, H, N, d], dtype=float32)``; multiply K by the workload's
key scale in float32 (3.0 for the long-sequence workload, which makes the
softmax rows peaked); round every tensor to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    key_scale: float = 1.0
    backward: bool = False
    seed: int = 0

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def fwd_flops(self) -> float:
        """4*B*H*N^2*d, halved when causal (two N x N x d contractions)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """10*B*H*N^2*d, halved when causal (five N x N x d contractions)."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


# The five workloads, seeded with their index.
WORKLOADS = {
    1: Workload("fwd_b1h1_n128_d64", 1, 1, 128, 64, False, seed=1),
    2: Workload("fwd_b4h16_n1024_d64", 4, 16, 1024, 64, False, seed=2),
    3: Workload("fwd_causal_b2h32_n4096_d128", 2, 32, 4096, 128, True, seed=3),
    4: Workload("fwd_causal_b1h16_n16384_d128_k3", 1, 16, 16384, 128, True,
                key_scale=3.0, seed=4),
    5: Workload("fwdbwd_causal_b2h16_n2048_d128", 2, 16, 2048, 128, True,
                backward=True, seed=5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return uint16 bits.

    Finite inputs only (the generators draw normals)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float64."""
    u = b.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    u = b.astype(np.uint32) << 16
    return u.view(np.float32)


@dataclass
class Inputs:
    """bf16 bit patterns (uint16, [B,H,N,d]) plus the float32 draws."""
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    q32: np.ndarray | None = None
    k32: np.ndarray | None = None
    v32: np.ndarray | None = None

    def as_f64(self, name: str) -> np.ndarray:
        return bf16_bits_to_f64(getattr(self, name))


def make_inputs(workload: Workload | int, *, keep_f32: bool = False,
                with_do: bool | None = None, N: int | None = None,
                seed: int | None = None) -> Inputs:
    """Draw the seeded inputs of ``workload`` (an index 1..5 or a Workload).

    ``N`` / ``seed`` override the sequence length and seed (for ragged and
    edge-case shapes that reuse a workload's recipe)."""
    w = WORKLOADS[workload] if isinstance(workload, int) else workload
    if N is not None or seed is not None:
        w = Workload(w.name, w.B, w.H, N if N is not None else w.N, w.d, w.causal,
                     w.key_scale, w.backward, seed if seed is not None else w.seed)
    rng = np.random.default_rng(w.seed)
    shape = w.shape
    q32 = rng.standard_normal(shape, dtype=np.float32)
    k32 = rng.standard_normal(shape, dtype=np.float32)
    if w.key_scale != 1.0:
        k32 = (k32 * np.float32(w.key_scale)).astype(np.float32)
    v32 = rng.standard_normal(shape, dtype=np.float32)
    want_do = w.backward if with_do is None else with_do
    do = None
    if want_do:
        do = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    inp = Inputs(w, f32_to_bf16_bits(q32), f32_to_bf16_bits(k32),
                 f32_to_bf16_bits(v32), do)
    if keep_f32:
        inp.q32, inp.k32, inp.v32 = q32, k32, v32
    return inp


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Seeded N(0, scale^2) draw rounded to bf16 bits (edge-case tests)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    return f32_to_bf16_bits(x)


@dataclass(frozen=True)
class DecodeWorkload:
    """Nq query rows against an Nk-row key/value cache per (batch, head)."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def kv_bytes(self) -> int:
        """Bytes of K and V (bf16): what one call must read at least."""
        return 2 * self.B * self.H * self.Nk * self.d * 2

    def flops(self) -> float:
        """4*B*H*Nq*Nk*d (two Nq x Nk x d contractions; the causal mask of the
        last Nq positions removes a negligible triangle)."""
        return 4.0 * self.B * self.H * self.Nq * self.Nk * self.d


# Decode workloads (the pages give none; these stand for one or eight new
# tokens per sequence against an 8192-token cache, 8 sequences x 32 heads).
DECODE_WORKLOADS = {
    "d1": DecodeWorkload("decode_b8h32_q1_k8192_d128", 8, 32, 1, 8192, 128, True, seed=11),
    "d8": DecodeWorkload("decode_b8h32_q8_k8192_d128", 8, 32, 8, 8192, 128, True, seed=12),
}


def make_decode_inputs(w: DecodeWorkload):
    """Seeded draws for a decode workload: Q [B,H,Nq,d], then K and V
    [B,H,Nk,d], each standard normal float32 rounded to bf16 bits."""
    rng = np.random.default_rng(w.seed)
    q = f32_to_bf16_bits(rng.standard_normal((w.B, w.H, w.Nq, w.d), dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((w.B, w.H, w.Nk, w.d), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((w.B, w.H, w.Nk, w.d), dtype=np.float32))
    return q, k, v
