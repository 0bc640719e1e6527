"""Seeded synthetic workloads for the SageSLA attention path.

This module only draws inputs. It holds none of the method's arithmetic, so
both the HIP path and the CPU oracle may consume what it produces.

The shapes stand in for the latent token grids of the video models the
TurboDiffusion pages benchmark (page 5, "Performance Benchmarks": Wan2.1 1.3B
at 480p, Wan 14B at 720p), whose weights and prompts are not available here:

* 21 x 30 x 52 = 32760 tokens with 12 heads (1.3B, 480p),
* 21 x 45 x 80 = 75600 tokens with 40 heads (14B, 720p),
* 33 x 68 x 120 = 269280 tokens with 40 heads (1080p-like stress shape).

Head dimension is 128 throughout. ``topk`` is the fraction of key blocks kept
per query block, the meaning the pages give ``--sla_topk`` (page 5, "Hands-On
Tutorial": 0.1 keeps 10%, i.e. 90% sparsity).

Recipe (per workload, one ``torch.Generator`` seeded with ``seed``):

1. if ``spikes``: ``idx = randperm(N)[: N // 100]`` (token positions shared by
   every head);
2. for each (b, h) in row-major order: ``q = randn(N, D)``, ``k = randn(N, D)``,
   ``v = randn(N, D)``, ``off = 3 * randn(D)``; ``k += off`` (a per-channel
   offset with standard deviation 3, shared by all tokens: outlier channels);
   if ``spikes``: ``k[idx] *= 20`` (after the offset);
3. every draw is fp32 and is cast to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    topk: float | None  # None: dense (every key block kept, linear branch off)
    spikes: bool = False
    seed: int = 0

    @property
    def dense(self) -> bool:
        return self.topk is None


# Named by what they are; the first is the small case the oracle finishes in
# seconds, the fourth is the 14B / 720p shape that throughput is quoted on and
# the fifth the same inputs at the larger keep fraction the pages suggest for
# quality (page 5, "Hands-On Tutorial": 0.15).
WORKLOADS = {
    w.name: w
    for w in (
        Workload("dense_h1_n1024", 1, 1, 1024, 128, None),
        Workload("dense_h12_n32760", 1, 12, 32760, 128, None),
        Workload("sla10_h12_n32760", 1, 12, 32760, 128, 0.1),
        Workload("sla10_h40_n75600", 1, 40, 75600, 128, 0.1),
        Workload("sla15_h40_n75600", 1, 40, 75600, 128, 0.15),
        Workload("sla5_spikes_h40_n269280", 1, 40, 269280, 128, 0.05, spikes=True),
    )
}

BENCH_WORKLOAD = "sla10_h40_n75600"


def make_qkv(B: int, H: int, N: int, D: int, seed: int = 0, spikes: bool = False,
             offset_std: float = 3.0):
    """Return bf16 CPU tensors q, k, v of shape [B, H, N, D] (recipe above)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.empty((B, H, N, D), dtype=torch.bfloat16)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    idx = torch.randperm(N, generator=g)[: N // 100] if spikes else None
    for b in range(B):
        for h in range(H):
            qf = torch.randn((N, D), generator=g)
            kf = torch.randn((N, D), generator=g)
            vf = torch.randn((N, D), generator=g)
            off = offset_std * torch.randn((D,), generator=g)
            kf += off
            if idx is not None:
                kf[idx] *= 20.0
            q[b, h] = qf.to(torch.bfloat16)
            k[b, h] = kf.to(torch.bfloat16)
            v[b, h] = vf.to(torch.bfloat16)
    return q, k, v


def make_workload(w: Workload | str):
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_qkv(w.B, w.H, w.N, w.D, seed=w.seed, spikes=w.spikes)


def bf16_bits(x: torch.Tensor):
    """View a contiguous bf16 tensor as a numpy uint16 array (no copy)."""
    return x.contiguous().view(torch.int16).numpy().view("uint16")


# ---------------------------------------------------------------------------
# W8A8 linear layer (page 5, Pillar Three). The benchmarked shape is a linear
# layer of the 14B / 720p model on one frame sequence: 75600 tokens of width
# H * D = 40 * 128 = 5120, mapped 5120 -> 5120.
#
# Recipe (one torch.Generator seeded with ``seed``): x = randn(M, K); then
# w = randn(N, K) / sqrt(K) (the scale of a default-initialised linear layer);
# if ``outliers``: 1% of the K channels of x (randperm(K)[: K // 100]) are
# multiplied by 20 after drawing (the activation outlier channels block
# quantization meets). Every draw is fp32, cast to bf16 with round-to-nearest-even.

@dataclass(frozen=True)
class LinearWorkload:
    name: str
    M: int
    N: int
    K: int
    outliers: bool = False
    seed: int = 0


LINEAR_WORKLOADS = {
    w.name: w
    for w in (
        LinearWorkload("w8a8_m1000_k512_n384", 1000, 384, 512, outliers=True),
        LinearWorkload("w8a8_m75600_k5120_n5120", 75600, 5120, 5120, outliers=True),
    )
}

LINEAR_BENCH_WORKLOAD = "w8a8_m75600_k5120_n5120"


def make_linear(M: int, N: int, K: int, seed: int = 0, outliers: bool = False):
    """Return bf16 CPU tensors x [M][K] and w [N][K] (recipe above)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    w = torch.randn((N, K), generator=g) / (K ** 0.5)
    if outliers:
        idx = torch.randperm(K, generator=g)[: max(1, K // 100)]
        x[:, idx] *= 20.0
    return x.to(torch.bfloat16), w.to(torch.bfloat16)


def make_linear_workload(w: LinearWorkload):
    return make_linear(w.M, w.N, w.K, w.seed, w.outliers)
