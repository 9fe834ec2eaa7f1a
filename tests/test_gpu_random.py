"""Seeded random sweep: every collective, mode and dtype on random rank
counts (1-16), shapes, split dimensions, ragged sizes, element offsets that
misalign the buffers (equal or different per rank) and in-place all-reduce,
compared bit for bit with the oracle; and a smaller sweep above 64 MiB moved,
where the all-reduce and reduce-scatter take their one-wave and flat shapes.
Each case draws from its own seed, so a failure names a reproducible case.
VRC_RANDOM_SEED_BASE (an integer, default 0) moves every case to a fresh
seed family, for longer sweeps run by hand; 0 gives the committed cases."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import assert_bitwise, host
from tests.test_gpu_parity import AG_MODES, DTYPES, HD_FAMILY, MODES, want_ag, want_ar, want_rs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = 120
SEED_BASE = int(os.environ.get("VRC_RANDOM_SEED_BASE", "0"))


def case_rng(seed: int):
    """The generator of one case: its own seed, in the chosen seed family."""
    return np.random.default_rng(seed if SEED_BASE == 0 else [SEED_BASE, seed])


def input_seed(seed: int) -> int:
    return seed + 1_000_003 * SEED_BASE


@pytest.fixture(scope="module")
def vrc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_all_reduce_virtual_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def draw(kind: int, k: int, modes=MODES):
    rng = case_rng(7919 * kind + k)
    dtype = str(rng.choice(DTYPES))
    mode = str(rng.choice(modes))
    n = int(2 ** rng.integers(0, 5)) if mode in HD_FAMILY else int(rng.integers(1, 17))
    return rng, dtype, mode, n


def log_uniform(rng, hi: int) -> int:
    return int(np.exp(rng.uniform(0.0, np.log(hi + 1)))) - 1


def offsets(rng, n: int):
    how = rng.integers(0, 3)
    if how == 0:
        return [0] * n
    if how == 1:
        return [int(rng.integers(1, 8))] * n
    return [int(v) for v in rng.integers(0, 8, n)]


def place(t: torch.Tensor, off: int) -> torch.Tensor:
    """A contiguous copy of t starting `off` elements into a fresh allocation."""
    base = torch.empty(t.numel() + off, dtype=t.dtype, device=t.device)
    v = base[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def empty_at(shape, dtype, off: int) -> torch.Tensor:
    numel = int(np.prod(shape)) if len(shape) else 1
    base = torch.empty(numel + off, dtype=dtype, device=DEV)
    return base[off:off + numel].view(shape)


def ranks(rng, n, shape, dtype, seed):
    xs = workloads.random_ranks(n, shape, dtype, seed=seed, device=DEV)
    return [place(x, o) for x, o in zip(xs, offsets(rng, n))]


@pytest.mark.parametrize("k", range(CASES))
def test_random_allreduce(vrc, orc, k):
    rng, dtype, mode, n = draw(1, k)
    count = log_uniform(rng, 70000)
    xs = ranks(rng, n, (count,), dtype, seed=input_seed(10000 + k))
    in_place = rng.random() < 0.25
    print(f"random allreduce case {k}: {mode} {dtype} n={n} count={count} in_place={in_place}", flush=True)
    hx = host(xs)
    if in_place:
        ys = xs
    else:
        ys = [empty_at((count,), xs[0].dtype, o) for o in offsets(rng, n)]
    vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.synchronize()
    want = want_ar(orc, hx, dtype, mode)
    for r, y in enumerate(host(ys)):
        assert_bitwise(y, want[r], f"case {k} {mode} {dtype} n={n} count={count} rank {r}")


@pytest.mark.parametrize("k", range(CASES))
def test_random_reduce_scatter(vrc, orc, k):
    rng, dtype, mode, n = draw(2, k)
    if rng.random() < 0.5:
        shape, dim, outer = (log_uniform(rng, 70000),), 0, 1
    else:
        nd = int(rng.integers(2, 4))
        dim = int(rng.integers(1, nd))
        shape = [int(rng.integers(2, 9)) for _ in range(nd)]
        shape[dim] = n * int(rng.integers(1, 200))
        shape = tuple(shape)
        outer = int(np.prod(shape[:dim]))
    xs = ranks(rng, n, shape, dtype, seed=input_seed(20000 + k))
    print(f"random reduce_scatter case {k}: {mode} {dtype} n={n} shape={shape} dim={dim}", flush=True)
    shapes = vrc.reduce_scatter_shape(shape, n, dim)
    ys = [empty_at(shapes[c], xs[0].dtype, o) for c, o in enumerate(offsets(rng, n))]
    hx = host(xs)
    vrc.vrc_reduce_scatter(xs, recv=ys, dim=dim, mode=mode)
    torch.cuda.synchronize()
    want = want_rs(orc, hx, dtype, mode, outer)
    for c, y in enumerate(host(ys)):
        assert_bitwise(y, want[c], f"case {k} {mode} {dtype} n={n} shape={shape} dim={dim} chunk {c}")


@pytest.mark.parametrize("k", range(CASES))
def test_random_all_gather(vrc, orc, k):
    rng, dtype, mode, n = draw(3, k, AG_MODES)
    nd = int(rng.integers(1, 4))
    shape = tuple(int(rng.integers(1, 9)) for _ in range(nd - 1)) + (log_uniform(rng, 800) + 1,)
    dim = int(rng.integers(0, nd))
    outer = int(np.prod(shape[:dim])) if dim else 1
    xs = ranks(rng, n, shape, dtype, seed=input_seed(30000 + k))
    print(f"random all_gather case {k}: {mode} {dtype} n={n} shape={shape} dim={dim}", flush=True)
    out_shape = list(shape)
    out_shape[dim] *= n
    ys = [empty_at(tuple(out_shape), xs[0].dtype, o) for o in offsets(rng, n)]
    hx = host(xs)
    vrc.vrc_all_gather(xs, recv=ys, dim=dim, mode=mode)
    torch.cuda.synchronize()
    want = want_ag(orc, hx, dtype, mode, outer)
    for r, y in enumerate(host(ys)):
        assert_bitwise(y, want[r], f"case {k} {mode} {dtype} n={n} shape={shape} dim={dim} rank {r}")


# ---------------------------------------------------------------------------
# Above 64 MiB moved the all-reduce and reduce-scatter take their one-wave
# shapes (and, for flat chunks that vectorize, the flat reduce-scatter
# kernels): a smaller seeded sweep there, single-launch modes, random rank
# counts, dtypes, ragged counts and per-rank element offsets.
# ---------------------------------------------------------------------------
LARGE_CASES = 12
LARGE_AR_MODES = ("fused", "ring_order", "ring_chained", "hd_order")
LARGE_RS_MODES = ("fused", "ring_order", "ring_chained", "hd_order", "hd")


def draw_large(kind: int, k: int, modes):
    rng = case_rng(104729 * kind + k)
    dtype = str(rng.choice(DTYPES))
    mode = str(rng.choice(modes))
    n = int(2 ** rng.integers(1, 5)) if mode in HD_FAMILY else int(rng.integers(2, 17))
    esz = 2 if dtype in ("fp16", "bf16") else 4
    return rng, dtype, mode, n, esz


@pytest.mark.parametrize("k", range(LARGE_CASES))
def test_random_large_allreduce(vrc, orc, k):
    rng, dtype, mode, n, esz = draw_large(4, k, LARGE_AR_MODES)
    moved = int(rng.uniform(64, 160) * (1 << 20))
    count = moved // (2 * n * esz) + int(rng.integers(0, 64))
    if k % 3 != 2:  # one element offset shared by every input and output: the vector path
        off = int(rng.integers(0, 8))
        in_off, out_off = [off] * n, [off] * n
    else:
        in_off, out_off = offsets(rng, n), offsets(rng, n)
    xs = workloads.random_ranks(n, (count,), dtype, seed=input_seed(40000 + k), device=DEV)
    xs = [place(x, o) for x, o in zip(xs, in_off)]
    print(f"random large allreduce case {k}: {mode} {dtype} n={n} count={count} offsets {in_off[0]}/"
          f"{out_off[0]}", flush=True)
    hx = host(xs)
    ys = [empty_at((count,), xs[0].dtype, o) for o in out_off]
    vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.synchronize()
    want = want_ar(orc, hx, dtype, mode)
    for r, y in enumerate(host(ys)):
        assert_bitwise(y, want[r], f"large case {k} {mode} {dtype} n={n} count={count} rank {r}")


@pytest.mark.parametrize("k", range(LARGE_CASES))
def test_random_large_reduce_scatter(vrc, orc, k):
    rng, dtype, mode, n, esz = draw_large(5, k, LARGE_RS_MODES)
    moved = int(rng.uniform(64, 160) * (1 << 20))
    vec = 16 // esz
    base = moved // ((n + 1) * n * esz)
    if k % 4 != 3:
        base = base // vec * vec  # whole 16-byte vectors per chunk: the flat kernels can take it
    count = n * base + int(rng.integers(0, n))
    if k % 3 != 2:  # one element offset shared by every input and output
        off = int(rng.integers(0, 8))
        in_off, out_off = [off] * n, [off] * n
    else:
        in_off, out_off = offsets(rng, n), offsets(rng, n)
    xs = workloads.random_ranks(n, (count,), dtype, seed=input_seed(50000 + k), device=DEV)
    xs = [place(x, o) for x, o in zip(xs, in_off)]
    print(f"random large reduce_scatter case {k}: {mode} {dtype} n={n} count={count} offsets {in_off[0]}/"
          f"{out_off[0]}", flush=True)
    shapes = vrc.reduce_scatter_shape((count,), n, 0)
    ys = [empty_at(shapes[c], xs[0].dtype, o) for c, o in enumerate(out_off)]
    hx = host(xs)
    vrc.vrc_reduce_scatter(xs, recv=ys, mode=mode)
    torch.cuda.synchronize()
    want = want_rs(orc, hx, dtype, mode)
    for c, y in enumerate(host(ys)):
        assert_bitwise(y, want[c], f"large case {k} {mode} {dtype} n={n} count={count} chunk {c}")


# ---------------------------------------------------------------------------
# The realigned single-launch all-reduces: outputs on random offsets within a
# 128-byte line (every byte shift up to 127), inputs on their own offsets,
# above 64 MiB moved, and now and then some ranks in place (which keeps the
# tile kernel); vrc_plan names the kernel each case expects.
# ---------------------------------------------------------------------------
REALIGN_CASES = 12
REALIGN_MODES = ("fused", "hd_order", "ring_order")


@pytest.mark.parametrize("k", range(REALIGN_CASES))
def test_random_realigned_allreduce(vrc, orc, k):
    rng, dtype, mode, n, esz = draw_large(6, k, REALIGN_MODES)
    per_line = 128 // esz
    moved = int(rng.uniform(64, 128) * (1 << 20))
    count = moved // (2 * n * esz) + int(rng.integers(0, 4096))
    in_off = [int(v) for v in rng.integers(0, per_line, n)]
    out_off = [int(v) for v in rng.integers(0, per_line, n)]
    in_place = [bool(v) for v in (rng.random(n) < 0.15)] if k % 4 == 3 else [False] * n
    xs = workloads.random_ranks(n, (count,), dtype, seed=input_seed(60000 + k), device=DEV)
    xs = [place(x, o) for x, o in zip(xs, in_off)]
    ys = [xs[r] if in_place[r] else empty_at((count,), xs[0].dtype, out_off[r]) for r in range(n)]
    addrs = [y.data_ptr() for y in ys]
    share = len({a % 128 for a in addrs}) == 1
    realign = not share and not any(in_place)
    base = {"fused": "fused_allreduce", "hd_order": "butterfly_allreduce" if n > 2 else "fused_allreduce",
            "ring_order": "ring_order_allreduce"}[mode]
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, [x.data_ptr() for x in xs], addrs, count, 1,
                      {"int32": vrc.VRC_INT32, "fp32": vrc.VRC_FP32, "fp16": vrc.VRC_FP16, "bf16": vrc.VRC_BF16}[dtype],
                      vrc.MODES[mode])
    print(f"random realigned allreduce case {k}: {mode} {dtype} n={n} count={count} in {in_off} out {out_off} "
          f"in_place {sum(in_place)} -> {ops[0]['kind']}", flush=True)
    assert [o["kind"] for o in ops] == [base + ("_realigned" if realign else "")]
    hx = host(xs)
    vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.synchronize()
    want = want_ar(orc, hx, dtype, mode)
    for r, y in enumerate(host(ys)):
        assert_bitwise(y, want[r], f"realigned case {k} {mode} {dtype} n={n} count={count} rank {r}")
