"""Helpers for comparing HIP outputs with the oracle (host-side plumbing)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import workloads


def host(ts):
    return [workloads.to_numpy(t) for t in ts]


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).reshape(-1).view(np.uint8)


def assert_bitwise(got: np.ndarray, want: np.ndarray, what: str):
    got = np.ascontiguousarray(got).reshape(-1)
    want = np.ascontiguousarray(want).reshape(-1)
    assert got.dtype == want.dtype, f"{what}: dtype {got.dtype} vs {want.dtype}"
    assert got.size == want.size, f"{what}: size {got.size} vs {want.size}"
    if not np.array_equal(bits(got), bits(want)):
        w = got.view(np.uint8).reshape(got.size, -1)
        v = want.view(np.uint8).reshape(want.size, -1)
        bad = np.nonzero(np.any(w != v, axis=1))[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} elements differ; first at {bad[:8].tolist()}: "
                             f"got {got[bad[:4]].tolist()} want {want[bad[:4]].tolist()}")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def tolerance_gate_torch(ys, xs, rtol: float, what: str, chunk: int = 1 << 24):
    """Gate against the fp64 sum, computed by torch on the device:
    every element |y - s| <= rtol * sum_r |x_r|, and ||y - s|| / ||s|| <= rtol.
    ys may hold fewer elements than xs (reduce-scatter): pass matching views."""
    count = ys[0].numel()
    err2 = torch.zeros((), dtype=torch.float64, device=ys[0].device)
    ref2 = torch.zeros((), dtype=torch.float64, device=ys[0].device)
    worst = 0.0
    for lo in range(0, count, chunk):
        hi = min(count, lo + chunk)
        s = torch.zeros(hi - lo, dtype=torch.float64, device=ys[0].device)
        a = torch.zeros_like(s)
        for x in xs:
            xv = x.reshape(-1)[lo:hi].double()
            s += xv
            a += xv.abs()
        ref2 += (s * s).sum()
        for r, y in enumerate(ys):
            d = (y.reshape(-1)[lo:hi].double() - s).abs()
            if r == 0:
                err2 += (d * d).sum()
            ratio = (d / torch.clamp(a, min=1e-300)).max().item()
            worst = max(worst, ratio)
            ok = bool((d <= rtol * a).all().item())
            assert ok, f"{what}: rank {r} elements [{lo},{hi}) exceed |y-s| <= {rtol}*sum|x| (worst {ratio:.3g})"
    rel = (err2.sqrt() / torch.clamp(ref2.sqrt(), min=1e-300)).item()
    assert rel <= rtol, f"{what}: relative 2-norm error {rel:.3g} > {rtol}"
    return worst, rel


def ranks_identical(ys, what: str):
    """Every rank's output has the same bytes as rank 0's (checked on the device)."""
    b0 = ys[0].contiguous().view(-1).view(torch.uint8)
    for r in range(1, len(ys)):
        assert torch.equal(ys[r].contiguous().view(-1).view(torch.uint8), b0), f"{what}: rank {r} differs from rank 0"


def sample_indices(count: int, n: int, m: int, seed: int) -> np.ndarray:
    """Random indices plus every chunk boundary (+-9), the first and last
    4096 elements, and 16-byte vector edges."""
    rng = np.random.default_rng(seed)
    parts = [rng.integers(0, count, size=m, dtype=np.int64), np.arange(min(count, 4096)),
             np.arange(max(0, count - 4096), count)]
    base = count // n
    for c in range(1, n):
        b = c * base
        parts.append(np.arange(max(0, b - 9), min(count, b + 9)))
    idx = np.unique(np.concatenate(parts))
    return idx[(idx >= 0) & (idx < count)].astype(np.uint64)


def oracle_every_element(at, hx, dtype: str, count: int, slice_elems: int = 1 << 22) -> np.ndarray:
    """All `count` elements of an all-reduce result from one of the oracle's
    per-element forms (`ring_allreduce_at`, `hd_allreduce_at`,
    `fused_allreduce_at`), computed in slices on host threads: the oracle's C
    code runs with the interpreter lock released, so the slices proceed in
    parallel.  The forms are pinned against the full ring simulation by the
    CPU tests."""
    out = np.empty(count, dtype=hx[0].dtype)

    def work(lo):
        hi = min(count, lo + slice_elems)
        out[lo:hi] = at(hx, dtype, np.arange(lo, hi, dtype=np.uint64))

    with ThreadPoolExecutor(max_workers=max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        list(ex.map(work, range(0, count, slice_elems)))
    return out


def equal_to_expected(ys, want: torch.Tensor, what: str):
    """Every rank's output bit for bit equal to `want` (on the device); on a
    mismatch, name the first differing elements."""
    wb = want.reshape(-1).view(torch.uint8)
    esz = want.element_size()
    for r, y in enumerate(ys):
        yb = y.contiguous().reshape(-1).view(torch.uint8)
        if not torch.equal(yb, wb):
            diff = (yb.view(-1, esz) != wb.view(-1, esz)).any(dim=1).nonzero().reshape(-1)
            first = diff[:8].tolist()
            raise AssertionError(f"{what}: rank {r}: {diff.numel()} of {want.numel()} elements differ; "
                                 f"first at {first}")
