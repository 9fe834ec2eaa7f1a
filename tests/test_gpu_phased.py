"""The phased fused all-reduce on the GPU, against the oracle.

Large fused, single-launch halving-doubling and ring-order all-reduces from
6 ranks read and write in phases: one 256-lane workgroup per CU folds K vectors per
lane of every input, the grid meets, then every lane writes its sums.  These
cases are large enough for at least three phases (vrc_plan confirms the
phased launch), and cover every element type, 6 to 16 ranks, all three folds, in
place, a partial last phase, a partial vector and a scalar head; every
element of every output is compared with the oracle's per-element form.
The meetings only shape the timing: runs with them switched off, or with
every workgroup holding the same number of sums, two calls at once on two
streams, and replays of a captured graph give the same bits."""
import os
import subprocess
import sys

import pytest
import torch

import oracle
import workloads
from tests.parity_util import equal_to_expected, host, oracle_every_element

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CUS = 256
CODES = {"int32": 0, "fp32": 1, "fp16": 2, "bf16": 3}
ESZ = {"int32": 4, "fp32": 4, "fp16": 2, "bf16": 2}


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def vrc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_all_reduce_virtual_amd as m
    if torch.cuda.get_device_properties(0).multi_processor_count != CUS:
        pytest.skip("the phase sizes below are for 256 CUs")
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def sums_per_lane(n, dtype, mode):
    if mode == "ring_order":  # registers by element type, plus 40 in LDS
        regs = {"bf16": 32 if n <= 7 else 24 if n <= 9 else 16 if n <= 14 else 0,
                "fp16": 40 if n <= 8 else 32 if n <= 11 else 24 if n <= 15 else 16}.get(dtype, 40)
        return regs + 40
    narrow = mode == "hd_order" and ESZ[dtype] == 2
    return ((32 if n <= 8 else 16) if narrow else (64 if n <= 8 else 32)) + 32


def phased_count(n, dtype, mode, extra):
    """Elements per rank for three whole phases after a scalar head of up to
    one 128-byte line (per chunk for the ring order, whose phases count each
    chunk's tiles), plus `extra` elements."""
    per_vector = 16 // ESZ[dtype]
    heads = n if mode == "ring_order" else 1
    return 3 * CUS * 256 * sums_per_lane(n, dtype, mode) * per_vector + heads * 128 // ESZ[dtype] + extra


def shifted(ts, shift):
    """Copies of `ts` placed `shift` elements past a 256-byte boundary (the
    same shift for every rank keeps the outputs on one 128-byte grid)."""
    out = []
    for t in ts:
        buf = torch.empty(t.numel() + 128, dtype=t.dtype, device=DEV)
        v = buf[shift:shift + t.numel()]
        v.copy_(t)
        out.append(v)
    return out


CASES = [  # (n, dtype, mode, extra elements, head shift in elements, in place)
    (6, "fp32", "fused", 12345, 3, False),
    (7, "bf16", "fused", 777, 5, True),
    (12, "fp16", "fused", 99, 1, False),
    (16, "int32", "fused", 5, 0, True),
    (8, "fp32", "fused", 513, 2, False),
    (8, "bf16", "hd_order", 1000, 7, False),
    (16, "fp32", "hd_order", 3, 2, False),
    (16, "fp16", "hd_order", 4097, 4, True),
    (6, "fp32", "ring_order", 4099, 3, False),
    (8, "bf16", "ring_order", 77, 5, True),
    (12, "fp16", "ring_order", 12345, 1, False),
    (16, "bf16", "ring_order", 31, 0, False),
    (9, "int32", "ring_order", 7, 2, False),
]


@pytest.mark.parametrize("n,dtype,mode,extra,shift,in_place", CASES)
def test_phased_allreduce_every_element(vrc, orc, n, dtype, mode, extra, shift, in_place):
    count = phased_count(n, dtype, mode, extra)
    say(f"phased all-reduce {mode}: n={n} {dtype} count={count} shift={shift} in_place={in_place}")
    xs = workloads.random_ranks(n, count, dtype, seed=7100 + n, device=DEV, sigma=1e-2)
    hx = host(xs)
    vx = shifted(xs, shift)
    vy = vx if in_place else shifted([torch.zeros_like(x) for x in xs], shift)
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, [v.data_ptr() for v in vx], [v.data_ptr() for v in vy], count, 1,
                      CODES[dtype], vrc.MODES[mode])
    kind = {"hd_order": "butterfly", "ring_order": "ring_order"}.get(mode, "fused") + "_allreduce_phased"
    assert [(o["kind"], o["grid_x"], o["block"], o["vectors"]) for o in ops] == [
        (kind, CUS, 256, sums_per_lane(n, dtype, mode))]
    vrc.vrc_allreduce(vx, recv=vy, mode=mode)
    torch.cuda.synchronize()
    at = {"hd_order": orc.hd_allreduce_at, "ring_order": orc.ring_allreduce_at}.get(mode, orc.fused_allreduce_at)
    want = torch.from_numpy(oracle_every_element(at, hx, dtype, count)).to(DEV)
    equal_to_expected(vy, want, f"phased {mode} n={n} {dtype}")
    del xs, vx, vy, want
    torch.cuda.empty_cache()


def test_two_phased_calls_at_once(vrc, orc):
    """Two phased all-reduces enqueued on two streams at the same time share
    the meeting count: each still finishes, with the oracle's bits."""
    n, dtype = 8, "bf16"
    count = phased_count(n, dtype, "fused", 31)
    say(f"phased all-reduce on two streams: n={n} {dtype} count={count}")
    xa = workloads.random_ranks(n, count, dtype, seed=7201, device=DEV, sigma=1e-2)
    xb = workloads.random_ranks(n, count, dtype, seed=7202, device=DEV, sigma=1e-2)
    ya = [torch.empty_like(x) for x in xa]
    yb = [torch.empty_like(x) for x in xb]
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        vrc.vrc_allreduce(xa, recv=ya, mode="fused", stream=sa)
        vrc.vrc_allreduce(xb, recv=yb, mode="fused", stream=sb)
    torch.cuda.synchronize()
    for xs, ys, tag in ((xa, ya, "stream a"), (xb, yb, "stream b")):
        want = torch.from_numpy(oracle_every_element(orc.fused_allreduce_at, host(xs), dtype, count)).to(DEV)
        equal_to_expected(ys, want, f"phased fused on {tag}")
    del xa, xb, ya, yb
    torch.cuda.empty_cache()


def test_captured_phased_allreduce(vrc, orc):
    """The phased kernel captured into a graph and replayed three times, with
    fresh inputs written eagerly between replays: every replay has the
    oracle's bits (the meeting count lives on the device and needs no reset)."""
    n, dtype = 8, "bf16"
    count = phased_count(n, dtype, "fused", 9)
    say(f"phased all-reduce captured: n={n} {dtype} count={count}")
    xs = workloads.random_ranks(n, count, dtype, seed=7301, device=DEV, sigma=1e-2)
    ys = [torch.empty_like(x) for x in xs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vrc.vrc_allreduce(xs, recv=ys, mode="fused")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vrc.vrc_allreduce(xs, recv=ys, mode="fused")
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = workloads.random_ranks(n, count, dtype, seed=7310 + rep, device=DEV, sigma=1e-2)
        for x, f in zip(xs, fresh):
            x.copy_(f)
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = torch.from_numpy(oracle_every_element(orc.fused_allreduce_at, host(fresh), dtype, count)).to(DEV)
        equal_to_expected(ys, want, f"phased replay {rep}")
    del g, xs, ys
    torch.cuda.empty_cache()


CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import oracle, workloads
import ring_all_reduce_virtual_amd as vrc
from tests.parity_util import equal_to_expected, host, oracle_every_element
n, count = 8, int(sys.argv[2])
xs = workloads.random_ranks(n, count, "bf16", seed=7401, device="cuda:0", sigma=1e-2)
ys = [torch.empty_like(x) for x in xs]
ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, [x.data_ptr() for x in xs], [y.data_ptr() for y in ys], count, 1,
                  vrc.VRC_BF16, vrc.VRC_FUSED)
assert ops[0]["kind"] == "fused_allreduce_phased", ops[0]["kind"]
vrc.vrc_allreduce(xs, recv=ys, mode="fused")
torch.cuda.synchronize()
want = torch.from_numpy(oracle_every_element(oracle.get().fused_allreduce_at, host(xs), "bf16", count)).to("cuda:0")
equal_to_expected(ys, want, "phased, one setting off")
print("ok", flush=True)
"""


@pytest.mark.parametrize("var", ["VRC_PHASE_WAIT", "VRC_PHASE_SKEW"])
def test_phased_without_meetings_or_skew(vrc, var):
    """VRC_PHASE_WAIT=0 (no workgroup ever waits at a meeting) and
    VRC_PHASE_SKEW=0 (every workgroup holds all its sums, so the phases cover
    other vectors): read once per process, so a child process runs each; the
    outputs are the same bits."""
    count = phased_count(8, "bf16", "fused", 4097)
    say(f"phased all-reduce with {var}=0 (child process): count={count}")
    env = dict(os.environ, PYTHONPATH=ROOT)
    env[var] = "0"
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(count)], env=env, capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]
