"""Seeded synthetic inputs for the attention forward: the one module shared by the
oracle side and the GPU side.

It holds shapes, seeds and random draws only, none of the attention arithmetic.
Every workload is dense, non-causal and i.i.d. Gaussian; Q, K and V are drawn in
fp32 and rounded to bfloat16 with round-to-nearest-even, which is what torch's
``Tensor.to(torch.bfloat16)`` does on the CPU.

Recipe (one ``torch.Generator('cpu')`` per workload, seeded with ``seed``):
    Q = bf16(sigma_qk * randn(B,H,N,d)),  K = bf16(sigma_qk * randn(B,H,N,d)),
    V = bf16(sigma_v  * randn(B,H,N,d))      -- drawn in that order.
Query rows checked on the large workloads come from ``sample_rows``: distinct flat
(b, h, i) indices drawn without replacement by ``numpy.random.default_rng``, with
the first and the last row always included.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    full_rows: bool = True  # False: check ``n_sample_rows`` sampled rows instead
    n_sample_rows: int = 4096

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Dense forward FLOPs, 2 contractions of 2*N*N*d each per (b, h)."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d

    @property
    def min_hbm_bytes(self) -> int:
        """Read Q, K, V once and write O (bf16) and LSE (fp32) once."""
        return self.B * self.H * self.N * (8 * self.d + 4)


# The five graded workloads. Seeds: the first states seed 0; the others use their
# index in this list. The last one has Q, K ~ N(0, 2.5^2) so scores span a wide range.
WORKLOADS = (
    Workload("b1h1_n256_d64", 1, 1, 256, 64, seed=0),
    Workload("b4h16_n1024_d64", 4, 16, 1024, 64, seed=1),
    Workload("b2h16_n4096_d128", 2, 16, 4096, 128, seed=2),
    Workload("b1h32_n8192_d128", 1, 32, 8192, 128, seed=3, full_rows=False),
    Workload("b1h8_n30001_d128_wide", 1, 8, 30001, 128, seed=4, sigma_qk=2.5, full_rows=False),
)
WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS}
HEADLINE = WORKLOADS[3]


def make_qkv(B: int, H: int, N: int, d: int, seed: int, sigma_qk: float = 1.0,
             sigma_v: float = 1.0):
    """Return (q, k, v) as contiguous CPU bfloat16 tensors of shape [B, H, N, d]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, d)
    q = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    k = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    v = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_v).to(torch.bfloat16)
    return q.contiguous(), k.contiguous(), v.contiguous()


def make_workload(w: Workload):
    return make_qkv(w.B, w.H, w.N, w.d, w.seed, w.sigma_qk, w.sigma_v)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Decode shape: Nq query rows per head against Nk key/value rows."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    check_heads: int = 0  # 0: check every head; else this many sampled (b, h) heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        return 4.0 * self.B * self.H * self.Nq * self.Nk * self.d

    @property
    def min_hbm_bytes(self) -> int:
        """Read Q, K, V once; write O (bf16) and LSE (fp32) once."""
        return self.B * self.H * (4 * self.Nk * self.d + self.Nq * (4 * self.d + 4))


# Decode workloads: a batch of sequences each adding one token (or a few) against
# its cached keys and values. The first is the benchmark shape (16 sequences at 8K
# context with the heads and head size of the prefill benchmark); the second one
# long sequence; the others vary Nq, d, a ragged Nk and a wide score range.
DECODE_WORKLOADS = (
    DecodeWorkload("dec_b16h32_q1_k8192_d128", 16, 32, 1, 8192, 128, seed=100, check_heads=24),
    DecodeWorkload("dec_b1h32_q1_k131072_d128", 1, 32, 1, 131072, 128, seed=101, check_heads=6),
    DecodeWorkload("dec_b4h16_q4_k4096_d64", 4, 16, 4, 4096, 64, seed=102),
    DecodeWorkload("dec_b2h8_q16_k30001_d128_wide", 2, 8, 16, 30001, 128, seed=103, sigma_qk=2.5),
    DecodeWorkload("dec_b16h32_q16_k8192_d128", 16, 32, 16, 8192, 128, seed=104, check_heads=24),
)
DECODE_BY_NAME = {w.name: w for w in DECODE_WORKLOADS}
DECODE_HEADLINE = DECODE_WORKLOADS[0]


def make_decode_qkv(B: int, H: int, Nq: int, Nk: int, d: int, seed: int, sigma_qk: float = 1.0,
                    sigma_v: float = 1.0):
    """Return q [B,H,Nq,d] and k, v [B,H,Nk,d] as contiguous CPU bfloat16 tensors,
    drawn Q, K, V in that order from one generator seeded with ``seed``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = (torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    k = (torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    v = (torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * sigma_v).to(torch.bfloat16)
    return q.contiguous(), k.contiguous(), v.contiguous()


def make_decode_workload(w: DecodeWorkload):
    return make_decode_qkv(w.B, w.H, w.Nq, w.Nk, w.d, w.seed, w.sigma_qk, w.sigma_v)


def sample_heads(B: int, H: int, count: int, seed: int) -> list:
    """Sorted distinct (b, h) pairs, the first and the last head always included."""
    total = B * H
    if count <= 0 or count >= total:
        return [(i // H, i % H) for i in range(total)]
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(total, size=count, replace=False).tolist()) | {0, total - 1}
    return [(i // H, i % H) for i in sorted(picks)]


def sample_rows(B: int, H: int, N: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct flat row indices (b*H + h)*N + i, first and last included."""
    total = B * H * N
    if count >= total:
        return np.arange(total, dtype=np.int64)
    rng = np.random.default_rng(seed)
    picks = rng.choice(total, size=count, replace=False).astype(np.int64)
    picks = np.unique(np.concatenate([picks, [0, total - 1]]))
    if picks.size > count:  # keep the two forced rows, drop extras
        keep = [0, total - 1]
        rest = [p for p in picks.tolist() if p not in (0, total - 1)]
        picks = np.array(sorted(keep + rest[: count - 2]), dtype=np.int64)
    return picks


def rows_for(w: Workload) -> np.ndarray:
    """The rows a parity check compares for workload ``w``."""
    if w.full_rows:
        return np.arange(w.B * w.H * w.N, dtype=np.int64)
    return sample_rows(w.B, w.H, w.N, w.n_sample_rows, 1000 + WORKLOADS.index(w))


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bfloat16 tensor to a float64 numpy array."""
    return t.to(torch.float64).numpy()
