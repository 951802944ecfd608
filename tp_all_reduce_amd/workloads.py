"""Seeded synthetic inputs for the fused W-way reduce + residual add + RMSNorm
epilogue, shared by the tests, the smoke check and the benchmark.

This module only draws random numbers; it holds none of the method's
arithmetic.  The five workloads are the decode/prefill shapes of the tensor-
parallel layer epilogue (W partial-sum buffers of [T, H] tokens x hidden):

  c1  W=2, T=8, H=1024, standard RMSNorm, eps 1e-6
  c2  W=4, H=4096, Gemma RMSNorm (weight applied as 1 + w), eps 1e-6,
      T in {1, 2, 4, 8, 16, 21, 22, 32, 64, 80} (decode window)
  c3  W=8, H=8192, eps 1e-5, T in {1024, 8192, 16384} (prefill, bandwidth-bound)
  c4  W=4, T=256, H=7168, FP8-e4m3 per-group (128) quant epilogue
  c5  QK-norm, W=4 shards of [T=64, 1536 q + 256 k + 256 v]

Every tensor is drawn as ``randn(float32) * std + mean`` and then rounded to the
16-bit format, from a generator seeded with ``1000 * config + T`` on the device
the tensor lives on.  Draw order: partials rank 0..W-1, then the residual, then
the weight(s).  ``N(a, b)`` below means mean a, standard deviation b.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                      # 1-based; part of the seed
    W: int
    H: int
    Ts: tuple
    eps: float
    gemma: bool = False
    partial_std: float = 1.0
    residual_std: float = 1.0
    weight_mean: float = 1.0
    weight_std: float = 0.1
    group: int = 0                  # FP8 group size along H (0: no quant epilogue)
    q_size: int = 0                 # QK-norm only
    kv_size: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "c1": Workload("c1", 1, W=2, H=1024, Ts=(8,), eps=1e-6),
    "c2": Workload("c2", 2, W=4, H=4096, Ts=(1, 2, 4, 8, 16, 21, 22, 32, 64, 80), eps=1e-6,
                   gemma=True, partial_std=0.5, weight_mean=0.0, weight_std=0.1),
    "c3": Workload("c3", 3, W=8, H=8192, Ts=(1024, 8192, 16384), eps=1e-5),
    "c4": Workload("c4", 4, W=4, H=7168, Ts=(256,), eps=1e-6, partial_std=2.0, group=128),
    "c5": Workload("c5", 5, W=4, H=2048, Ts=(64,), eps=1e-6, q_size=1536, kv_size=256),
}


def seed_of(wl: Workload, T: int) -> int:
    return 1000 * wl.index + int(T)


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def draw(shape, mean: float, std: float, gen: torch.Generator, dtype=torch.bfloat16,
         device="cpu") -> torch.Tensor:
    """One seeded normal draw, rounded to ``dtype``."""
    x = torch.randn(tuple(shape), dtype=torch.float32, generator=gen, device=device)
    return (x * std + mean).to(dtype)


def make_inputs(wl: Workload, T: int, dtype=torch.bfloat16, device="cpu", seed=None,
                W=None, H=None):
    """Inputs of the reduce + add + RMSNorm workloads (c1..c4).

    Returns dict(partials=[W x [T,H]], residual=[T,H], weight=[H])."""
    W = wl.W if W is None else W
    H = wl.H if H is None else H
    g = generator(seed_of(wl, T) if seed is None else seed, device)
    partials = [draw((T, H), 0.0, wl.partial_std, g, dtype, device) for _ in range(W)]
    residual = draw((T, H), 0.0, wl.residual_std, g, dtype, device)
    weight = draw((H,), wl.weight_mean, wl.weight_std, g, dtype, device)
    return {"partials": partials, "residual": residual, "weight": weight}


def make_qk_inputs(wl: Workload, T: int, dtype=torch.bfloat16, device="cpu", seed=None,
                   W=None, q_size=None, kv_size=None):
    """Inputs of the QK-norm workload (c5).

    Returns dict(shards=[W x [T, q+2kv]], q_weight=[W*q], k_weight=[W*kv])."""
    W = wl.W if W is None else W
    q = wl.q_size if q_size is None else q_size
    kv = wl.kv_size if kv_size is None else kv_size
    g = generator(seed_of(wl, T) if seed is None else seed, device)
    shards = [draw((T, q + 2 * kv), 0.0, wl.partial_std, g, dtype, device) for _ in range(W)]
    q_weight = draw((W * q,), wl.weight_mean, wl.weight_std, g, dtype, device)
    k_weight = draw((W * kv,), wl.weight_mean, wl.weight_std, g, dtype, device)
    return {"shards": shards, "q_weight": q_weight, "k_weight": k_weight}


def bits(t: torch.Tensor):
    """Host numpy view of a 16-bit tensor's bit patterns (uint16)."""
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16).numpy().view("uint16")
