"""The library's step plans, executed on the CPU and compared with the oracle.

vrc_plan records every add and copy that a ring, halving-doubling or tree
call would launch: operand addresses, rows, width and element strides, in
launch order.  This test runs those operations on host arrays standing in
for the rank buffers (every add through the oracle's storage-type add, each
launch reading all its operands before it writes) and compares the outcome
bit for bit with the oracle's literal simulations of the same collective.
So the host half of the library (chunk partition, step order, which operand
each add takes, column blocks, buckets, the selector's choice at small
sizes) is checked at random rank counts, sizes and dtypes without a GPU.
The kernels behind the single-launch modes are covered by the GPU tests."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import ring_all_reduce_virtual_amd as vrc

DTYPES = {"int32": (vrc.VRC_INT32, 4), "fp32": (vrc.VRC_FP32, 4), "fp16": (vrc.VRC_FP16, 2), "bf16": (vrc.VRC_BF16, 2)}
SPACING = 1 << 24  # bytes between the stand-in base addresses of consecutive rank buffers
SEND0, RECV0 = 1 << 32, 1 << 36


def inputs(n, count, dtype, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        if dtype == "int32":
            out.append(rng.integers(-2**31, 2**31, count, dtype=np.int64).astype(np.int32))
        elif dtype == "fp32":
            out.append(rng.standard_normal(count).astype(np.float32))
        elif dtype == "fp16":
            out.append(rng.standard_normal(count).astype(np.float16))
        else:  # bf16 bits: the upper half of a normal fp32 draw
            out.append((rng.standard_normal(count).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    return out


class Memory:
    """Host arrays at stand-in device addresses."""

    def __init__(self, esize):
        self.esize = esize
        self.bufs = []  # (base, array)

    def add(self, base, arr):
        assert arr.nbytes <= SPACING
        self.bufs.append((base, arr))
        return base

    def locate(self, addr, rows, width, stride):
        for base, arr in self.bufs:
            if base <= addr < base + max(arr.nbytes, 1):
                off = addr - base
                assert off % self.esize == 0, "operand not on an element boundary"
                i0 = off // self.esize
                last = i0 + (rows - 1) * stride + width
                assert last <= arr.size, f"operand runs past its buffer ({last} > {arr.size})"
                return arr, [i0 + r * stride for r in range(rows)]
        raise AssertionError(f"address {addr:#x} is in no buffer")


def execute(ops, mem, dtype):
    orc = oracle.get()
    launches = sorted({o["launch"] for o in ops})
    for launch in launches:
        writes = []
        for o in (o for o in ops if o["launch"] == launch):
            assert o["kind"] in ("add", "copy"), o["kind"]
            if not o["rows"] or not o["width"]:
                continue
            w = o["width"]
            a, ia = mem.locate(o["a"], o["rows"], w, o["stride_a"])
            d, idst = mem.locate(o["d"], o["rows"], w, o["stride_d"])
            if o["kind"] == "add":
                b, ib = mem.locate(o["b"], o["rows"], w, o["stride_b"])
                vals = [orc.add(a[i:i + w].copy(), b[j:j + w].copy(), dtype) for i, j in zip(ia, ib)]
            else:
                vals = [a[i:i + w].copy() for i in ia]
            writes.extend((d, k, v) for k, v in zip(idst, vals))
        for d, k, v in writes:
            d[k:k + v.size] = v


def run_plan(coll, xs, recv_sizes, outer, dtype, mode, in_place=False):
    code, esize = DTYPES[dtype]
    n = len(xs)
    mem = Memory(esize)
    xs = [x.copy() for x in xs]
    send = [mem.add(SEND0 + r * SPACING, x) for r, x in enumerate(xs)]
    if in_place:
        recv, ys = send, xs
    else:
        ys = [np.zeros(sz, dtype=xs[0].dtype) for sz in recv_sizes]
        recv = [mem.add(RECV0 + r * SPACING, y) for r, y in enumerate(ys)]
    count = xs[0].size
    ops, _ = vrc.plan(coll, send, recv, count, outer, code, mode)
    execute(ops, mem, dtype)
    return ys


def same_bits(got, want):
    assert len(got) == len(want)
    for g, w in zip(got, want):
        assert g.shape == w.shape and g.tobytes() == w.tobytes()


dtypes = st.sampled_from(sorted(DTYPES))


@settings(max_examples=300, deadline=None)
@given(n=st.integers(1, 16), count=st.integers(0, 700), dtype=dtypes, in_place=st.booleans(), seed=st.integers(0, 9))
def test_ring_allreduce_plan_runs_the_ring(n, count, dtype, in_place, seed):
    xs = inputs(n, count, dtype, seed)
    got = run_plan(vrc.COLL_ALLREDUCE, xs, [count] * n, 1, dtype, vrc.VRC_RING, in_place)
    same_bits(got, oracle.get().ring_allreduce(xs, dtype))


@settings(max_examples=150, deadline=None)
@given(k=st.integers(0, 4), count=st.integers(0, 700), dtype=dtypes, in_place=st.booleans(), seed=st.integers(0, 9))
def test_hd_allreduce_plan_runs_the_butterfly(k, count, dtype, in_place, seed):
    n = 1 << k
    xs = inputs(n, count, dtype, seed)
    got = run_plan(vrc.COLL_ALLREDUCE, xs, [count] * n, 1, dtype, vrc.VRC_HD, in_place)
    same_bits(got, oracle.get().hd_allreduce(xs, dtype))


@settings(max_examples=100, deadline=None)
@given(n=st.integers(2, 16), count=st.integers(1, 500), dtype=dtypes, seed=st.integers(0, 9))
def test_select_allreduce_plan_runs_what_it_selects(n, count, dtype, seed):
    """At these sizes VRC_SELECT takes halving-doubling at powers of two and
    the ring otherwise: the plan's bits are that algorithm's."""
    xs = inputs(n, count, dtype, seed)
    got = run_plan(vrc.COLL_ALLREDUCE, xs, [count] * n, 1, dtype, vrc.VRC_SELECT)
    orc = oracle.get()
    want = orc.hd_allreduce(xs, dtype) if n & (n - 1) == 0 else orc.ring_allreduce(xs, dtype)
    same_bits(got, want)


@st.composite
def rs_shapes(draw):
    n = draw(st.integers(1, 16))
    if draw(st.booleans()):
        return n, draw(st.integers(0, 700)), 1
    outer = draw(st.integers(2, 9))
    w = draw(st.integers(0, 12))
    return n, outer * n * w, outer


@settings(max_examples=300, deadline=None)
@given(shape=rs_shapes(), dtype=dtypes, seed=st.integers(0, 9))
def test_ring_reduce_scatter_plan_runs_the_ring(shape, dtype, seed):
    n, count, outer = shape
    xs = inputs(n, count, dtype, seed)
    orc = oracle.get()
    got = run_plan(vrc.COLL_REDUCE_SCATTER, xs, [orc.rs_len(count, n, outer, c) for c in range(n)], outer, dtype,
                   vrc.VRC_RING)
    same_bits(got, orc.ring_reduce_scatter(xs, dtype, outer))


@st.composite
def ag_shapes(draw):
    n = draw(st.integers(1, 16))
    outer = draw(st.sampled_from([1, 1, 2, 3, 5]))
    return n, outer * draw(st.integers(0, 150)), outer


@settings(max_examples=300, deadline=None)
@given(shape=ag_shapes(), dtype=dtypes, mode=st.sampled_from(["ring", "tree", "hd", "select"]), seed=st.integers(0, 9))
def test_all_gather_plans_concatenate(shape, dtype, mode, seed):
    n, count, outer = shape
    if mode == "hd" and n & (n - 1):
        n = 1 << (n.bit_length() - 1)
    xs = inputs(n, count, dtype, seed)
    got = run_plan(vrc.COLL_ALL_GATHER, xs, [n * count] * n, outer, dtype, vrc.MODES[mode])
    orc = oracle.get()
    want = {"ring": orc.ring_all_gather, "tree": orc.tree_all_gather, "hd": orc.hd_all_gather}.get(mode)
    want = want(xs, dtype, outer) if want else orc.ring_all_gather(xs, dtype, outer)
    same_bits(got, want)


@settings(max_examples=100, deadline=None)
@given(n=st.integers(1, 16), count=st.integers(0, 900), bucket=st.integers(1, 400), dtype=dtypes,
       mode=st.sampled_from(["ring", "hd"]), seed=st.integers(0, 9))
def test_bucketed_plan_reduces_every_bucket_on_its_own(n, count, bucket, dtype, mode, seed):
    """Bucket k of every rank is an all-reduce of its own element range, with
    the mode's order over that range's own partition."""
    if mode == "hd" and n & (n - 1):
        n = 1 << (n.bit_length() - 1)
    xs = inputs(n, count, dtype, seed)
    got = run_plan(vrc.COLL_ALLREDUCE_BUCKETED, xs, [count] * n, bucket, dtype, vrc.MODES[mode])
    orc = oracle.get()
    fold = orc.ring_allreduce if mode == "ring" else orc.hd_allreduce
    want = [np.empty_like(x) for x in xs]
    for lo in range(0, count, bucket):
        hi = min(count, lo + bucket)
        part = fold([x[lo:hi] for x in xs], dtype)
        for r in range(n):
            want[r][lo:hi] = part[r]
    same_bits(got, want)


def test_the_executor_catches_a_wrong_schedule():
    """The comparison has teeth: executing the ring plan with one step's
    launches dropped, or with two ranks' inputs swapped, changes the bits."""
    n, count, dtype = 5, 103, "fp32"
    xs = inputs(n, count, dtype, 3)
    orc = oracle.get()
    want = orc.ring_allreduce(xs, dtype)
    _, esize = DTYPES[dtype]
    mem = Memory(esize)
    send = [mem.add(SEND0 + r * SPACING, x.copy()) for r, x in enumerate(xs)]
    ys = [np.zeros(count, np.float32) for _ in range(n)]
    recv = [mem.add(RECV0 + r * SPACING, y) for r, y in enumerate(ys)]
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_FP32, vrc.VRC_RING)
    execute([o for o in ops if o["launch"] != 1], mem, dtype)
    with pytest.raises(AssertionError):
        same_bits(ys, want)
    swapped = [xs[1], xs[0]] + xs[2:]
    got = run_plan(vrc.COLL_ALLREDUCE, xs, [count] * n, 1, dtype, vrc.VRC_RING)
    same_bits(got, want)
    with pytest.raises(AssertionError):
        same_bits(got, orc.ring_allreduce(swapped, dtype))
