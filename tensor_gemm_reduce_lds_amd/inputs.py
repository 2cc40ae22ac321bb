"""Seeded synthetic workloads for the fused GEMM + reduce-scatter path.

This module only makes input data and names the five workloads.  It holds
none of the method's arithmetic: no GEMM, no epilogue, no reduction, no tile
map.  Tests and the benchmark feed the same arrays to the HIP library and to
the CPU oracle, so both sides see the exact same bits.

Workloads (FFN down-projection shards, from the page "flux实现：sm80
gemm+rs", opening paragraph, and the Llama-3 7B/70B and decode cases on the
page "通信 overlap 实现", sections on the async-TP numbers and on the cost
limits of overlap):

* ``tiny_f32``     W=2, A_r[128,512], B_r[512,256], U[-1,1], fp32 in/out.
* ``llama8b``      W=8, A_r[4096,1792], B_r[1792,4096], bf16.
* ``llama70b``     W=8, A_r[8192,3584], B_r[3584,8192], bf16, beta=1 with a
                   bf16 bias row broadcast down the rows (std 0.02).
* ``decode``       W=8, A_r[64,3584], B_r[3584,8192], bf16 (m <= 64 case).
* ``ragged_2lvl``  W=8 as 2 groups of 4, A_r[8000,3584], alpha=0.5, bf16,
                   M not a multiple of the tile height.

Value recipe: A ~ N(0,1) "activations", B ~ N(0, (1/sqrt(K))^2) "weights"
(standard deviation 1/sqrt(K)), bias ~ N(0, 0.02^2).  Each tensor of each
rank is drawn from its own PCG64 stream seeded by
``SeedSequence([seed, workload_index, kind, rank])`` with kind A=0, B=1,
C=2, drawn in float32 and converted to bfloat16 by torch's CPU cast
(round to nearest even).  bf16 tensors are returned as their raw uint16
bits; fp32 tensors as float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

KIND_A, KIND_B, KIND_C = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    W: int
    M: int
    N: int
    K: int
    dtype: str            # "bf16" or "f32"
    alpha: float
    beta: float
    has_c: bool
    ldc: int              # 0: bias row broadcast down the rows; N: full matrix
    order: str            # "flat" or "two_level"
    groups: int           # sub-groups for the two-level order (1 for flat)
    tile_m: int           # 0 lets the library choose
    tile_n: int
    dist: str             # "normal" or "uniform"
    c_std: float = 0.0

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs of one pass: W partial GEMMs of 2*M*N*K."""
        return self.W * 2 * self.M * self.N * self.K

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 0, W=2, M=128, N=256, K=512, dtype="f32",
                         alpha=1.0, beta=0.0, has_c=False, ldc=0,
                         order="flat", groups=1, tile_m=64, tile_n=64,
                         dist="uniform"),
    "llama8b": Workload("llama8b", 1, W=8, M=4096, N=4096, K=1792,
                        dtype="bf16", alpha=1.0, beta=0.0, has_c=False, ldc=0,
                        order="flat", groups=1, tile_m=0, tile_n=0,
                        dist="normal"),
    "llama70b": Workload("llama70b", 2, W=8, M=8192, N=8192, K=3584,
                         dtype="bf16", alpha=1.0, beta=1.0, has_c=True, ldc=0,
                         order="flat", groups=1, tile_m=0, tile_n=0,
                         dist="normal", c_std=0.02),
    "decode": Workload("decode", 3, W=8, M=64, N=8192, K=3584, dtype="bf16",
                       alpha=1.0, beta=0.0, has_c=False, ldc=0, order="flat",
                       groups=1, tile_m=0, tile_n=0, dist="normal"),
    "ragged_2lvl": Workload("ragged_2lvl", 4, W=8, M=8000, N=8192, K=3584,
                            dtype="bf16", alpha=0.5, beta=0.0, has_c=False,
                            ldc=0, order="two_level", groups=2, tile_m=0,
                            tile_n=0, dist="normal"),
}


def _rng(seed: int, index: int, kind: int, rank: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, index, kind, rank])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16) through torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (h.astype(np.uint32) << 16).view(np.float32)


def _draw(g: np.random.Generator, shape, dist: str, scale: float) -> np.ndarray:
    if dist == "normal":
        x = g.standard_normal(size=shape, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        return x
    if dist == "uniform":
        return g.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "ternary":
        # entries in {-1, 0, 1}: every product and partial sum is a small
        # integer, exact in fp32
        return g.integers(-1, 2, size=shape).astype(np.float32)
    raise ValueError(dist)


def make_inputs(w: Workload, seed: int = 0, dist: Optional[str] = None,
                c_dist: Optional[str] = None):
    """Return dict(A=[W,M,K], B=[W,K,N], C=[N] | [M,N] | None).

    ``dist`` overrides the A/B value distribution ("normal", "uniform",
    "ternary").  With "normal", B gets standard deviation 1/sqrt(K).
    ``c_dist`` overrides the bias distribution ("normal" with w.c_std, or
    "ternary").
    """
    dist = dist or w.dist
    A = np.empty((w.W, w.M, w.K), dtype=np.float32)
    B = np.empty((w.W, w.K, w.N), dtype=np.float32)
    b_scale = 1.0 / np.sqrt(w.K) if dist == "normal" and w.K > 0 else 1.0
    for r in range(w.W):
        A[r] = _draw(_rng(seed, w.index, KIND_A, r), (w.M, w.K), dist, 1.0)
        B[r] = _draw(_rng(seed, w.index, KIND_B, r), (w.K, w.N), dist, b_scale)
    C = None
    if w.has_c:
        c_shape = (w.N,) if w.ldc == 0 else (w.M, w.ldc)
        cd = c_dist or "normal"
        C = _draw(_rng(seed, w.index, KIND_C, 0), c_shape, cd,
                  w.c_std if cd == "normal" else 1.0)
    if w.dtype == "bf16":
        A = to_bf16_bits(A)
        B = to_bf16_bits(B)
        if C is not None:
            C = to_bf16_bits(C)
    return {"A": A, "B": B, "C": C}


def with_shape(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (for smaller cases)."""
    return dataclasses.replace(w, **kw)


# ---- all-gather + GEMM inputs -------------------------------------------------
# FFN up-projection shard of a Llama-3-70B-like layer (hidden 8192, intermediate
# 28672 split over W=8 ranks): X is sequence-sharded by rows across the ranks,
# each rank's weight shard B_r is [K, N] with N = 28672 / 8.
AG_WORKLOADS = {
    "llama70b_up": dict(index=5, W=8, M=8192, N=3584, K=8192),
}


def make_ag_inputs(M: int, N: int, K: int, W: int, index: int = 5, seed: int = 0,
                   dist: str = "normal"):
    """Return dict(X=[W, M/W, K], B=[W, K, N]) as bfloat16 bits.

    Rank d's row shard X[d] is rows [d*M/W, (d+1)*M/W) of the full input.
    X ~ N(0,1), B ~ N(0, (1/sqrt(K))^2) with "normal"; "ternary" draws both
    from {-1, 0, 1}.  Streams as in ``make_inputs`` (kind A for X, B for B).
    """
    Mc = M // W
    X = np.empty((W, Mc, K), dtype=np.float32)
    B = np.empty((W, K, N), dtype=np.float32)
    b_scale = 1.0 / np.sqrt(K) if dist == "normal" else 1.0
    for r in range(W):
        X[r] = _draw(_rng(seed, index, KIND_A, r), (Mc, K), dist, 1.0)
        B[r] = _draw(_rng(seed, index, KIND_B, r), (K, N), dist, b_scale)
    return dict(X=to_bf16_bits(X).reshape(X.shape), B=to_bf16_bits(B).reshape(B.shape))
