"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the contractions themselves: it only draws
seeded random operands and describes shapes and layouts.  Both the oracle
side and the GPU side receive the very same bf16 bit patterns from here.

Recipe: a torch CPU ``Generator`` seeded per operand; uniform [lo, hi] is
``lo + (hi - lo) * torch.rand`` in fp32, normal is ``torch.randn`` in fp32;
both are rounded to bf16 (round-to-nearest-even, torch's conversion).  An
operand is drawn in its STORAGE order (a column-major matrix is drawn as its
row-major transpose), so the bits depend only on (seed, shape, distribution).

The five contraction workloads and the attention-forward workload are dense,
unstructured matrices; the pages measure no public dataset, so nothing here
stands in for one.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "gemm" or "sscore"
    batch: int
    M: int                    # rows of C  (Lq for sscore)
    N: int                    # cols of C  (Lk for sscore)
    K: int                    # contraction length (head dim d for sscore)
    a_major: str              # "row" (K contiguous) or "col" (M contiguous)
    b_major: str              # "row" (N contiguous) or "col" (K contiguous); sscore: K[b,j,d] rows
    dist: str                 # "uniform" or "normal"
    lo: float
    hi: float
    seeds: Tuple[int, int]
    out: str                  # "f32" or "bf16"
    description: str

    @property
    def flop(self) -> float:
        return 2.0 * self.batch * self.M * self.N * self.K

    @property
    def a_storage_shape(self) -> Tuple[int, ...]:
        if self.kind == "sscore":
            return (self.batch, self.M, self.K)
        return (self.K, self.M) if self.a_major == "col" else (self.M, self.K)

    @property
    def b_storage_shape(self) -> Tuple[int, ...]:
        if self.kind == "sscore":
            return (self.batch, self.N, self.K)
        return (self.N, self.K) if self.b_major == "col" else (self.K, self.N)

    def a_strides(self) -> Tuple[int, int, int]:
        """(row, col, batch) element strides of the logical A[b, i, k]."""
        if self.kind == "sscore":
            return (self.K, 1, self.M * self.K)
        return (1, self.M, 0) if self.a_major == "col" else (self.K, 1, 0)

    def b_strides(self) -> Tuple[int, int, int]:
        """(row, col, batch) element strides of the logical B[b, k, j] (sscore: of K[b, j, d])."""
        if self.kind == "sscore":
            return (self.K, 1, self.N * self.K)
        return (1, self.K, 0) if self.b_major == "col" else (self.N, 1, 0)

    @property
    def bytes_a(self) -> int:
        return 2 * int(np.prod(self.a_storage_shape))

    @property
    def bytes_b(self) -> int:
        return 2 * int(np.prod(self.b_storage_shape))

    @property
    def bytes_c(self) -> int:
        return (4 if self.out == "f32" else 2) * self.batch * self.M * self.N


WORKLOADS: Dict[str, Workload] = {
    "gemm512": Workload(
        "gemm512", "gemm", 1, 512, 512, 512, "row", "row", "uniform", -1.0, 1.0, (101, 102), "f32",
        "bf16 GEMM C=A.B, M=N=K=512, row-major A and B, U[-1,1], fp32 out"),
    "sscore32x2048": Workload(
        "sscore32x2048", "sscore", 32, 2048, 2048, 128, "row", "row", "normal", 0.0, 1.0, (201, 202), "f32",
        "attention scores S=Q.K^T, 32 slices of Q,K [2048,128], N(0,1), fp32 S [32,2048,2048]"),
    "gemm8192": Workload(
        "gemm8192", "gemm", 1, 8192, 8192, 8192, "row", "row", "uniform", -1.0, 1.0, (301, 302), "bf16",
        "square bf16 GEMM M=N=K=8192, row-major, U[-1,1], bf16 out"),
    "gemm65536x256x4096": Workload(
        "gemm65536x256x4096", "gemm", 1, 65536, 256, 4096, "row", "row", "normal", 0.0, 1.0, (401, 402),
        "f32", "tall-skinny bf16 GEMM M=65536 N=256 K=4096, N(0,1), fp32 out"),
    "gemm16384x8192x2048_colA": Workload(
        "gemm16384x8192x2048_colA", "gemm", 1, 16384, 8192, 2048, "col", "row", "uniform", -0.5, 0.5,
        (501, 502), "bf16", "bf16 GEMM M=16384 N=8192 K=2048, A column-major, B row-major, U[-0.5,0.5], bf16 out"),
    "gemm4096x2048x8192": Workload(
        "gemm4096x2048x8192", "gemm", 1, 4096, 2048, 8192, "row", "row", "uniform", -1.0, 1.0, (311, 312), "bf16",
        "one GPU's share of the 8192^3 GEMM on a 2 x 4 grid of 8 GPUs: M=4096, N=2048, K=8192, row-major, "
        "U[-1,1], bf16 out (128 tiles of 256^2: split K)"),
}
ORDER = ["gemm512", "sscore32x2048", "gemm8192", "gemm65536x256x4096", "gemm16384x8192x2048_colA",
         "gemm4096x2048x8192"]


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """Attention forward O = softmax(scale Q K^T) V over `batch` slices;
    Q [Lq, d], K [Lk, d], V [Lk, dv], O [Lq, dv], all with the last
    dimension contiguous."""
    name: str
    batch: int
    Lq: int
    Lk: int
    d: int
    dv: int
    dist: str
    lo: float
    hi: float
    seeds: Tuple[int, int, int]   # Q, K, V
    scale: float
    out: str                      # "f32" or "bf16"
    description: str
    causal: bool = False          # query i sees keys j <= i + Lk - Lq only
    kv_group: int = 1             # query slice b reads K/V slice b // kv_group

    @property
    def flop(self) -> float:
        """Q.K^T and P.V over the visible (query, key) pairs: 2*(d + dv) each."""
        if self.causal:
            off = self.Lk - self.Lq
            pairs = self.Lq * (off + 1) + self.Lq * (self.Lq - 1) / 2.0
        else:
            pairs = float(self.Lq) * self.Lk
        return 2.0 * self.batch * pairs * (self.d + self.dv)

    def strides(self):
        """(row, col, batch) element strides of Q, K, V and O."""
        return ((self.d, 1, self.Lq * self.d), (self.d, 1, self.Lk * self.d),
                (self.dv, 1, self.Lk * self.dv), (self.dv, 1, self.Lq * self.dv))

    @property
    def kv_batch(self) -> int:
        return self.batch // self.kv_group

    @property
    def bytes_in(self) -> int:
        return 2 * (self.batch * self.Lq * self.d + self.kv_batch * (self.Lk * self.d + self.Lk * self.dv))

    @property
    def bytes_out(self) -> int:
        return (4 if self.out == "f32" else 2) * self.batch * self.Lq * self.dv


# The attention forward consumes the score workload's very Q and K (same
# seeds, shapes and distribution) plus a V drawn alike.
ATTN_WORKLOADS: Dict[str, AttnWorkload] = {
    "attn32x2048": AttnWorkload(
        "attn32x2048", 32, 2048, 2048, 128, 128, "normal", 0.0, 1.0, (201, 202, 203), 128 ** -0.5, "bf16",
        "attention forward O=softmax(Q.K^T/sqrt(128)).V, 32 slices of Q,K,V [2048,128], N(0,1), bf16 O"),
    "attn32x2048_causal": AttnWorkload(
        "attn32x2048_causal", 32, 2048, 2048, 128, 128, "normal", 0.0, 1.0, (201, 202, 203), 128 ** -0.5, "bf16",
        "causal attention forward (query i sees keys 0..i), 32 slices of Q,K,V [2048,128], N(0,1), bf16 O",
        causal=True),
    "attn32x2048_gqa8_causal": AttnWorkload(
        "attn32x2048_gqa8_causal", 32, 2048, 2048, 128, 128, "normal", 0.0, 1.0, (201, 202, 203), 128 ** -0.5,
        "bf16", "causal attention forward with grouped key/value heads: 32 query slices [2048,128] over 4 K,V "
        "slices (8 query slices per K,V), N(0,1), bf16 O", causal=True, kv_group=8),
}


def attn_operands(w: AttnWorkload):
    """(Q, K, V) bf16 CPU tensors [batch, L, d] for attention workload ``w``."""
    Q = draw((w.batch, w.Lq, w.d), w.dist, w.lo, w.hi, w.seeds[0])
    K = draw((w.kv_batch, w.Lk, w.d), w.dist, w.lo, w.hi, w.seeds[1])
    V = draw((w.kv_batch, w.Lk, w.dv), w.dist, w.lo, w.hi, w.seeds[2])
    return Q, K, V


def draw(shape, dist: str, lo: float, hi: float, seed: int) -> torch.Tensor:
    """Seeded bf16 tensor (CPU) in storage order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    if dist == "uniform":
        x = torch.rand(tuple(shape), generator=g, dtype=torch.float32)
        x.mul_(hi - lo).add_(lo)
    elif dist == "normal":
        x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    elif dist == "int":
        # integers in [lo, hi], exactly representable in bf16
        x = torch.randint(int(lo), int(hi) + 1, tuple(shape), generator=g, dtype=torch.int32).to(torch.float32)
    else:
        raise ValueError(dist)
    return x.to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy array of its bit patterns (CPU copy if needed)."""
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def operands(w: Workload, dist: Optional[str] = None, lo: Optional[float] = None, hi: Optional[float] = None):
    """(A, B) bf16 CPU tensors in storage order for workload ``w``."""
    d = dist or w.dist
    l = w.lo if lo is None else lo
    h = w.hi if hi is None else hi
    A = draw(w.a_storage_shape, d, l, h, w.seeds[0])
    B = draw(w.b_storage_shape, d, l, h, w.seeds[1])
    return A, B


def sample_points(batch: int, M: int, N: int, n: int, seed: int, edges: bool = True) -> np.ndarray:
    """Seeded (b, i, j) sample of output positions, plus the tile-edge corners when ``edges``."""
    rng = np.random.default_rng(seed)
    pts = np.stack([rng.integers(0, batch, n), rng.integers(0, M, n), rng.integers(0, N, n)], axis=1)
    if edges:
        corners = []
        for b in {0, batch - 1}:
            for i in {0, M - 1, M // 2}:
                for j in {0, N - 1, N // 2}:
                    corners.append((b, i, j))
        pts = np.concatenate([pts, np.array(corners, dtype=np.int64)], axis=0)
    return pts.astype(np.int64)
