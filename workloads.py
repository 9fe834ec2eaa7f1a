"""Seeded synthetic workloads for the virtual-rank collectives.

This module only describes workloads and draws their inputs; it holds none
of the collectives' arithmetic.  Both the HIP path (tests, bench) and the
CPU oracle take their inputs from here.

The workloads follow what the pages exchange: gradient buffers summed by a
data-parallel all-reduce, at the 1/16/128/512 MB sizes of the bandwidth
table (hwcomputing.csdn.net/6a0dc11a10ee7a33f273f7fd.html, "性能参考"), a
[8, 4096] fp16 activation (ai6s.net/6a157e6510ee7a33f27553e9.html,
"代码示例") and attention-head slices gathered across tensor-parallel ranks
(ai6s.net/6a102b5410ee7a33f2746c06.html, "分布式推理中的通信").  No public
dataset is involved.

Values are drawn with torch's generator on the device the caller names
(Philox on the GPU, the CPU generator on the CPU); rank r of a workload with
seed S uses seed S*1000 + r.  The same seed therefore gives the same inputs
on every run of one device type.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

MiB = 1 << 20


@dataclass(frozen=True)
class Workload:
    name: str
    n: int                   # virtual ranks
    shape: tuple             # per-rank input shape
    dtype: str               # int32 | fp32 | fp16 | bf16
    dist: str                # uniform_int | normal | normal_outliers
    seed: int
    sigma: float = 1.0
    collective: str = "allreduce"   # allreduce | all_gather | reduce_scatter
    dim: int = 0                    # concat / scatter dimension
    modes: tuple = ("ring", "fused")
    rtol: float | None = None       # tolerance gate (None: bit-exact)
    note: str = ""
    sweep: tuple = field(default_factory=tuple)  # extra per-rank element counts

    @property
    def count(self) -> int:
        c = 1
        for k in self.shape:
            c *= k
        return c

    @property
    def esize(self) -> int:
        return 4 if self.dtype in ("int32", "fp32") else 2

    def with_count(self, count: int) -> "Workload":
        return Workload(self.name + f"@{count}", self.n, (count,), self.dtype, self.dist, self.seed,
                        self.sigma, self.collective, self.dim, self.modes, self.rtol, self.note)


TORCH_DTYPES = {"int32": torch.int32, "fp32": torch.float32, "fp16": torch.float16,
                "bf16": torch.bfloat16}

WORKLOADS = {
    "allreduce_int32_n4_4099": Workload(
        "allreduce_int32_n4_4099", 4, (4099,), "int32", "uniform_int", 1,
        note="4099 int32 per rank (not divisible by 4), uniform in [-1000, 1000]"),
    "allreduce_fp32_n8_16mib": Workload(
        "allreduce_fp32_n8_16mib", 8, (4194304,), "fp32", "normal", 2, sigma=1.0, rtol=1e-5,
        note="16 MiB fp32 gradient-like N(0,1) per rank"),
    "allreduce_fp16_n8_128mib": Workload(
        "allreduce_fp16_n8_128mib", 8, (67108864,), "fp16", "normal", 3, sigma=1e-2, rtol=1e-2,
        sweep=(524288, 8388608),
        note="128 MiB fp16 gradients N(0, 0.01^2) per rank; sweep at 1 MiB and 16 MiB"),
    "allreduce_bf16_n8_512mib": Workload(
        "allreduce_bf16_n8_512mib", 8, (268435456,), "bf16", "normal_outliers", 4, sigma=1e-2,
        rtol=1e-2, modes=("fused",),
        note="512 MiB bf16 gradients N(0, 0.01^2) per rank, 1% of entries replaced by +-100"),
    "all_gather_fp16_n8_heads": Workload(
        "all_gather_fp16_n8_heads", 8, (1, 5, 4096, 128), "fp16", "normal", 5, sigma=1.0,
        collective="all_gather", dim=1,
        note="attention slice [1, 5 heads, 4096, 128] fp16 per rank, gathered on the head dim"),
    "reduce_scatter_fp16_n8_act": Workload(
        "reduce_scatter_fp16_n8_act", 8, (8, 4096), "fp16", "normal", 6, sigma=1.0, rtol=1e-2,
        collective="reduce_scatter", dim=-1,
        note="[8, 4096] fp16 activation per rank, reduce-scattered along the last dim"),
}

HEADLINE = "allreduce_bf16_n8_512mib"


def make_rank(w: Workload, r: int, device) -> torch.Tensor:
    """Rank r's input for workload w, drawn on `device`."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + r)
    shape = w.shape
    if w.dist == "uniform_int":
        return torch.randint(-1000, 1001, shape, generator=g, device=device, dtype=torch.int32)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.sigma != 1.0:
        x.mul_(w.sigma)
    if w.dist == "normal_outliers":
        hit = torch.rand(shape, generator=g, device=device) < 0.01
        sign = torch.rand(shape, generator=g, device=device) < 0.5
        big = torch.where(sign, torch.full_like(x, 100.0), torch.full_like(x, -100.0))
        x = torch.where(hit, big, x)
        del hit, sign, big
    return x.to(TORCH_DTYPES[w.dtype])


def make_inputs(w: Workload, device) -> list[torch.Tensor]:
    return [make_rank(w, r, device) for r in range(w.n)]


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy in the oracle's representation (bf16 as raw uint16 bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    return t.cpu().numpy().reshape(-1)


def torch_dtype(name: str) -> torch.dtype:
    return TORCH_DTYPES[name]


def random_ranks(n: int, shape, dtype: str, seed: int, device, sigma: float = 1.0) -> list[torch.Tensor]:
    """n ranks of seeded random values (int32 uniform in [-1000, 1000],
    floats N(0, sigma^2)) for parity cases of arbitrary shape."""
    shape = tuple(shape) if not isinstance(shape, int) else (shape,)
    dist = "uniform_int" if dtype == "int32" else "normal"
    w = Workload(f"random_{dtype}", n, shape, dtype, dist, seed, sigma=sigma)
    return make_inputs(w, device)
