"""Seeded synthetic inputs for the attention forward pass.

Shared by the tests, the benchmark and the smoke check: both the HIP path and
the CPU oracle receive exactly the arrays made here.  This module holds no
attention arithmetic; it only draws Gaussian values and rounds them to
bfloat16 bit patterns.

Recipe (the pages fix the shapes, not the generator; see the workload table
in the 5090 benchmark of "Flash Attention на 5090 в CUDA C++" and the 4K/8K/16K
shapes of the B200 article):
  * ``numpy.random.default_rng(seed)`` (PCG64);
  * Q, then K, then V drawn with ``standard_normal(dtype=float32)`` in C order
    over ``[B, H, N, d]``;
  * optional: K multiplied by ``k_scale``; then, per (b, h) in C order,
    ``round(offset_frac * Nk)`` distinct key rows chosen with the same
    generator (no replacement) get ``+offset`` on every element;
  * one round-to-nearest-even conversion of each fp32 value to bf16.

Arrays are returned as ``uint16`` bf16 bit patterns, layout ``[B, H, N, d]``,
C-contiguous.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits.

    NaN inputs are not expected from the generator and are not special-cased.
    """
    x = np.asarray(x, dtype=np.float32)
    u = np.ascontiguousarray(x).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16).reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.asarray(b, dtype=np.uint16)
    return (np.ascontiguousarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(b.shape)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int = HEAD_DIM
    seed: int = 0
    k_scale: float = 1.0
    offset_frac: float = 0.0
    offset: float = 0.0
    dv: int | None = None   # value head size; None: equal to d

    @property
    def d_v(self) -> int:
        return self.d if self.dv is None else self.dv

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d) as the float32 value a caller passes."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> int:
        """Two dense products per (query, key) pair: 2*B*H*Nq*Nk*(d + d_v)
        (4*B*H*Nq*Nk*d when d_v = d)."""
        return 2 * self.B * self.H * self.Nq * self.Nk * (self.d + self.d_v)

    def describe(self) -> str:
        dv = "" if self.dv is None else f" d_v={self.dv}"
        s = f"B={self.B} H={self.H} Nq={self.Nq} Nk={self.Nk} d={self.d}{dv} seed={self.seed}"
        if self.k_scale != 1.0 or self.offset_frac:
            s += f" K*{self.k_scale:g} +{self.offset:g} on {self.offset_frac:.0%} of rows"
        return s


# The workloads: a tiny case, the RTX 5090 benchmark shape (bs=1, heads=8,
# q=4096, kv=8192), and 16K tokens at 4K/8K/16K sequence length with 16
# heads of size 128 (the 16K one stresses large logits and running-max
# jumps); then head sizes 64 and 256 at 8K, and query/key head size 192 with
# value head size 128 (the split of multi-head latent attention's prefill).
WORKLOADS = {
    "tiny_256": Workload("tiny_256", 1, 1, 256, 256, seed=1001),
    "rtx5090_q4096_kv8192": Workload("rtx5090_q4096_kv8192", 1, 8, 4096, 8192, seed=1002),
    "b4_h16_n4096": Workload("b4_h16_n4096", 4, 16, 4096, 4096, seed=1003),
    "b2_h16_n8192": Workload("b2_h16_n8192", 2, 16, 8192, 8192, seed=1004),
    "b1_h16_n16384_koffset": Workload(
        "b1_h16_n16384_koffset", 1, 16, 16384, 16384, seed=1005,
        k_scale=4.0, offset_frac=0.01, offset=8.0),
    # other head sizes at the same hidden size H*d = 2048 and 16K tokens
    "b2_h32_n8192_d64": Workload("b2_h32_n8192_d64", 2, 32, 8192, 8192, d=64, seed=1006),
    "b2_h8_n8192_d256": Workload("b2_h8_n8192_d256", 2, 8, 8192, 8192, d=256, seed=1007),
    "b2_h16_n8192_d192_dv128": Workload("b2_h16_n8192_d192_dv128", 2, 16, 8192, 8192, d=192, seed=1008, dv=128),
}
WORKLOAD_ORDER = list(WORKLOADS)


def offset_row_count(Nk: int, frac: float) -> int:
    return int(round(frac * Nk))


def make_qkv(B: int, H: int, Nq: int, Nk: int, d: int = HEAD_DIM, seed: int = 0,
             k_scale: float = 1.0, offset_frac: float = 0.0, offset: float = 0.0,
             dv: int | None = None):
    """Draw Q [B,H,Nq,d], K [B,H,Nk,d], V [B,H,Nk,dv] as bf16 bits (uint16)."""
    dv = d if dv is None else dv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, Nk, dv), dtype=np.float32)
    if k_scale != 1.0:
        k *= np.float32(k_scale)
    n_off = offset_row_count(Nk, offset_frac)
    if n_off:
        for b in range(B):
            for h in range(H):
                idx = rng.choice(Nk, size=n_off, replace=False)
                k[b, h, idx, :] += np.float32(offset)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_workload(w: Workload):
    return make_qkv(w.B, w.H, w.Nq, w.Nk, w.d, w.seed, w.k_scale, w.offset_frac, w.offset, dv=w.dv)


def sample_rows(B: int, H: int, Nq: int, n: int, seed: int) -> np.ndarray:
    """Flat row indices into [B*H*Nq] for sampled parity checks.

    Always includes the first and last row of every head and the rows around
    the 128-row tile edges, then fills up with seeded random rows.
    """
    rng = np.random.default_rng(seed + 7919)
    rows = set()
    for bh in range(B * H):
        base = bh * Nq
        rows.update({base, base + Nq - 1})
    for r in (127, 128, 255, 256):
        if r < Nq:
            rows.add(r)
    total = B * H * Nq
    while len(rows) < min(n, total):
        rows.add(int(rng.integers(0, total)))
    return np.array(sorted(rows), dtype=np.int64)
