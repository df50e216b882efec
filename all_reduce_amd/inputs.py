"""Seeded synthetic rank inputs for the all-reduce workloads.

Holds none of the all-reduce's arithmetic: it only draws numbers with a CPU
``torch.Generator`` and casts them to the element type with torch's own
round-to-nearest-even ``.to()``.  Tests, the benchmark and the oracle checks
all take their inputs from here, so the GPU path and the oracle always see the
same bits.

The workloads stand in for those on the pages (no dataset is involved):
the SGLang MSCCL++ benchmark sweeps bfloat16 messages of 2^10 .. 2^19
elements ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南",
blog.gitcode.com, section 3.3), and tensor-parallel inference all-reduces the
attention and MLP outputs, tokens x hidden, in every layer (same guide,
section 1).  Recipe, per call of :func:`make`:

* ``g = torch.Generator("cpu").manual_seed(seed)``; one (R, N) float32 draw,
  row r is rank r;
* ``uniform``  -> ``rand * 2 - 1``  (uniform on [-1, 1));
* ``normal``   -> ``randn``;
* ``outliers`` -> ``randn``, then per rank ``floor(0.001 * N)`` positions from
  ``randperm(N)`` multiplied by 1000, before the cast;
* ``int4``     -> ``randint(-4, 5)``, integers -4..4 (their sums are exact);
* cast to the element type with ``.to(dtype)``.
"""
from __future__ import annotations

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def make(nranks: int, count: int, dtype: str, dist: str, seed: int) -> torch.Tensor:
    """(nranks, count) CPU tensor of the element type."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (nranks, count)
    if dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * 2 - 1
    elif dist == "normal":
        x = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "outliers":
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        k = count // 1000
        for r in range(nranks):
            idx = torch.randperm(count, generator=g)[:k]
            x[r, idx] *= 1000.0
    elif dist == "int4":
        x = torch.randint(-4, 5, shape, generator=g, dtype=torch.int64).to(torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.to(DTYPES[dtype])


# The workloads, by name.  Sizes are per rank.
WORKLOADS = {
    # R=8, 1024 bf16 per rank, uniform[-1, 1], seed 0
    "C1": dict(nranks=8, count=1024, dtype="bf16", dist="uniform", seed=0),
    # R=8, 64 tokens x hidden 8192 bf16 per rank (decode activation), N(0, 1), seed 3
    "C3": dict(nranks=8, count=64 * 8192, dtype="bf16", dist="normal", seed=3),
    # R=8, 8192 tokens x hidden 8192 bf16 per rank (prefill), N(0,1) + 0.1% x1000, seed 4
    "C4": dict(nranks=8, count=8192 * 8192, dtype="bf16", dist="outliers", seed=4),
}


def sweep(k: int) -> dict:
    """R=8, 2^k bf16 per rank (k = 10..19: 2 KiB .. 1 MiB), uniform[-1, 1], seed k."""
    return dict(nranks=8, count=1 << k, dtype="bf16", dist="uniform", seed=k)


def integer_case(nranks: int, dtype: str) -> dict:
    """R = 16 or 32 with integer data: 2^18 fp16, or 4096 x 7168 fp32, per rank; seed 5."""
    count = (1 << 18) if dtype == "fp16" else 4096 * 7168
    return dict(nranks=nranks, count=count, dtype=dtype, dist="int4", seed=5)
