"""The library's own launch plans, checked on the CPU (vrc_plan launches
nothing): the ring, halving-doubling and binomial-tree schedules against the
hand-derived fixtures, the chunk partition, the algorithmic bytes of each
mode, and that no two operations of one launch race."""
import os

import pytest

import ring_all_reduce_virtual_amd as vrc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
E = 4  # fp32 / int32
SEND_BASE, RECV_BASE, STRIDE = 0x10000000, 0x40000000, 1 << 24  # host-side stand-in addresses


def rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def buffers(n):
    return [SEND_BASE + r * STRIDE for r in range(n)], [RECV_BASE + r * STRIDE for r in range(n)]


def wide_buffers(n):
    """Stand-in addresses 4 GiB apart, for plans of large buffers."""
    return [(1 << 40) + r * (1 << 32) for r in range(n)], [(1 << 41) + r * (1 << 32) for r in range(n)]


def owner(addr, bases):
    """(rank, byte offset) of an address inside one of the rank buffers."""
    for r, b in enumerate(bases):
        if b <= addr < b + STRIDE:
            return r, addr - b
    raise AssertionError(f"address {addr:#x} is in no buffer")


def chunk_of(off_bytes, count, n):
    base = count // n
    return min(off_bytes // E // base, n - 1) if base else n - 1


def test_ring_allreduce_plan_matches_the_walkthrough():
    """N = 4: every reduce-scatter step op reads the partial of the chunk the
    predecessor sent, every all-gather op copies the chunk the predecessor
    relayed -- exactly the message table derived from the pages."""
    n, count = 4, 12
    send, recv = buffers(n)
    ops, launches = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_FP32, vrc.VRC_RING)
    assert launches == 2 * (n - 1)
    got = []
    for op in ops:
        step = op["launch"] % (n - 1)
        phase = "rs" if op["launch"] < n - 1 else "ag"
        dst, doff = owner(op["d"], recv)
        if phase == "rs":
            assert op["kind"] == "add"
            src, aoff = owner(op["a"], send if step == 0 else recv)
            own, boff = owner(op["b"], send)
            assert own == dst and boff == doff == aoff
        else:
            assert op["kind"] == "copy"
            src, aoff = owner(op["a"], recv)
            assert aoff == doff
        got.append((phase, str(step), str(src), str(dst), str(chunk_of(doff, count, n))))
    want = [tuple(r) for r in rows("ring_n4_schedule.txt")]
    assert sorted(got) == sorted(want)


@pytest.mark.parametrize("n,count", [(4, 4099), (8, 100), (3, 2), (16, 1000003)])
def test_ring_plan_uses_the_remainder_partition(n, count):
    send, recv = buffers(n)
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_INT32, vrc.VRC_RING)
    base = count // n
    for op in ops:
        _, off = owner(op["d"], recv)
        c = chunk_of(off, count, n) if op["width"] else None
        if op["width"]:
            assert off == c * base * E
            assert op["width"] == (count - (n - 1) * base if c == n - 1 else base)


def test_hd_allreduce_plan_matches_the_textbook_schedule():
    n, count = 4, 8  # two elements per block
    send, recv = buffers(n)
    ops, launches = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_FP32, vrc.VRC_HD)
    assert launches == 4
    got = []
    for op in ops:
        step = op["launch"] % 2
        phase = "rs" if op["launch"] < 2 else "ag"
        dst, doff = owner(op["d"], recv)
        lo, hi = doff // E // 2, (doff // E + op["width"]) // 2
        if phase == "rs":
            assert op["kind"] == "add"
            own, aoff = owner(op["a"], send if step == 0 else recv)
            src, boff = owner(op["b"], send if step == 0 else recv)
            assert own == dst and aoff == boff == doff
        else:
            assert op["kind"] == "copy"
            src, aoff = owner(op["a"], recv)
            assert aoff == doff
        got.append((phase, str(step), str(src), str(dst), str(lo), str(hi)))
    want = [tuple(r) for r in rows("hd_n4_schedule.txt")]
    assert sorted(got) == sorted(want)


def test_ring_reduce_scatter_plan_keeps_partials_in_the_output():
    """Column blocks of [outer, row]: step s adds rank (c+1+s)'s block c into
    output c, starting from rank c's block."""
    n, outer, row = 4, 3, 8
    count, w = outer * row, row // n
    send, recv = buffers(n)
    ops, launches = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, count, outer, vrc.VRC_FP32, vrc.VRC_RING)
    assert launches == n - 1
    for op in ops:
        s = op["launch"]
        c, doff = owner(op["d"], recv)
        assert doff == 0 and op["rows"] == outer and op["width"] == w and op["stride_d"] == w
        r, boff = owner(op["b"], send)
        assert r == (c + 1 + s) % n and boff == c * w * E and op["stride_b"] == row
        if s == 0:
            assert owner(op["a"], send) == (c, c * w * E) and op["stride_a"] == row
        else:
            assert owner(op["a"], recv) == (c, 0) and op["stride_a"] == w


@pytest.mark.parametrize("mode,kind", [(vrc.VRC_FUSED, "fused_allreduce"), (vrc.VRC_RING_CHAINED, "chain_allreduce"),
                                       (vrc.VRC_RING_ORDER, "ring_order_allreduce"),
                                       (vrc.VRC_HD_ORDER, "butterfly_allreduce")])
def test_single_launch_modes_plan_one_launch(mode, kind):
    send, recv = buffers(8)
    ops, launches = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, 1000, 1, vrc.VRC_BF16, mode)
    assert launches == 1 and [o["kind"] for o in ops] == [kind]


@pytest.mark.parametrize("n", [2, 4, 8, 16])
@pytest.mark.parametrize("mode", [vrc.VRC_RING, vrc.VRC_HD])
def test_step_plans_move_the_algorithmic_bytes(n, mode):
    """Adds read two operands and write one, copies read one and write one:
    both ring and halving-doubling move 5(N-1) S for the all-reduce, in
    2(N-1) and 2 log2 N launches."""
    count = 64 * n
    send, recv = buffers(n)
    ops, launches = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_FP32, mode)
    moved = sum(o["rows"] * o["width"] * E * (3 if o["kind"] == "add" else 2) for o in ops)
    assert moved == 5 * (n - 1) * count * E
    assert launches == (2 * (n - 1) if mode == vrc.VRC_RING else 2 * (n.bit_length() - 1))


def intervals(op, which):
    """Byte intervals touched by operand `which` ('a', 'b' or 'd') of an op."""
    base, stride = op[which], op["stride_" + which]
    return [(base + r * stride * E, base + r * stride * E + op["width"] * E) for r in range(op["rows"])]


def races(ops):
    by_launch = {}
    for op in ops:
        by_launch.setdefault(op["launch"], []).append(op)
    bad = []
    for launch, group in by_launch.items():
        for i, oi in enumerate(group):
            writes = intervals(oi, "d")
            for j, oj in enumerate(group):
                if i == j:
                    continue
                touched = intervals(oj, "a") + intervals(oj, "d") + (intervals(oj, "b") if oj["kind"] == "add" else [])
                for w0, w1 in writes:
                    for t0, t1 in touched:
                        if w0 < t1 and t0 < w1 and w1 > w0 and t1 > t0:
                            bad.append((launch, i, j))
    return bad


@pytest.mark.parametrize("mode", [vrc.VRC_RING, vrc.VRC_HD])
@pytest.mark.parametrize("n,count", [(2, 10), (4, 4099), (8, 1000), (16, 333)])
@pytest.mark.parametrize("in_place", [False, True])
def test_no_two_ops_of_a_launch_race(mode, n, count, in_place):
    send, recv = buffers(n)
    if in_place:
        recv = send
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_FP32, mode)
    assert not races(ops)


@pytest.mark.parametrize("mode", [vrc.VRC_RING, vrc.VRC_HD])
@pytest.mark.parametrize("n,outer,row", [(4, 3, 8), (8, 8, 4096), (2, 5, 6)])
def test_no_races_in_reduce_scatter_and_all_gather_plans(mode, n, outer, row):
    send, recv = buffers(n)
    for coll in (vrc.COLL_REDUCE_SCATTER, vrc.COLL_ALL_GATHER):
        ops, _ = vrc.plan(coll, send, recv, outer * row, outer, vrc.VRC_FP32, mode)
        assert not races(ops)


@pytest.mark.parametrize("n,name", [(4, "tree_n4_schedule.txt"), (5, "tree_n5_schedule.txt")])
def test_tree_all_gather_plan_matches_the_textbook_schedule(n, name):
    """The tree all-gather's copies, read as messages (source rank, receiving
    rank, slab range), are the hand-derived gather and broadcast schedules;
    the first gather launch also places each receiving rank's own slab."""
    count = 6
    send, recv = buffers(n)
    ops, launches = vrc.plan(vrc.COLL_ALL_GATHER, send, recv, count, 1, vrc.VRC_FP32, vrc.VRC_TREE)
    k = (n - 1).bit_length()
    assert launches == 2 * k
    got, own = [], []
    for op in ops:
        assert op["kind"] == "copy"
        dst, doff = owner(op["d"], recv)
        if op["launch"] < k:
            phase, step = "gather", op["launch"]
            lo, hi = doff // (count * E), doff // (count * E) + op["width"] // count
            if op["a"] in send:
                src = send.index(op["a"])
                if src == dst:
                    own.append(dst)
                    continue
            else:
                src, aoff = owner(op["a"], recv)
                assert aoff == doff
        else:
            phase, step = "bcast", op["launch"] - k
            src, aoff = owner(op["a"], recv)
            assert aoff == doff == 0 and op["width"] == n * count
            lo, hi = 0, n
        got.append((phase, str(step), str(src), str(dst), str(lo), str(hi)))
    assert sorted(got) == sorted(tuple(r) for r in rows(name))
    assert own == list(range(0, n, 2))


def tree_slab_copies(n):
    return (n + 1) // 2 + sum(bin(j).count("1") for j in range(n)) + n * (n - 1)


@pytest.mark.parametrize("n", list(range(1, 17)))
def test_tree_plan_moves_the_tree_bytes(n):
    """Each copy reads and writes its slabs once: ceil(N/2) own slabs, slab j
    once per set bit of j in the gather, N slabs to each of the N - 1 other
    ranks in the broadcast."""
    outer, row = 2, 5
    send, recv = buffers(n)
    ops, launches = vrc.plan(vrc.COLL_ALL_GATHER, send, recv, outer * row, outer, vrc.VRC_FP32, vrc.VRC_TREE)
    moved = sum(o["rows"] * o["width"] * E * 2 for o in ops)
    assert moved == 2 * tree_slab_copies(n) * outer * row * E
    assert launches == (2 * (n - 1).bit_length() if n > 1 else 1)


@pytest.mark.parametrize("n", list(range(2, 17)))
@pytest.mark.parametrize("outer,row", [(1, 7), (3, 8)])
def test_no_races_in_tree_all_gather_plans(n, outer, row):
    send, recv = buffers(n)
    ops, _ = vrc.plan(vrc.COLL_ALL_GATHER, send, recv, outer * row, outer, vrc.VRC_FP32, vrc.VRC_TREE)
    assert not races(ops)


def test_tree_is_an_all_gather_mode_only():
    send, recv = buffers(4)
    for coll in (vrc.COLL_ALLREDUCE, vrc.COLL_REDUCE_SCATTER):
        with pytest.raises(vrc.VrcError) as e:
            vrc.plan(coll, send, recv, 100, 1, vrc.VRC_FP32, vrc.VRC_TREE)
        assert e.value.status == vrc.VRC_ERR_UNSUPPORTED


@pytest.mark.parametrize("mode,per_bucket", [(vrc.VRC_FUSED, 1), (vrc.VRC_RING, 14), (vrc.VRC_HD, 6),
                                               (vrc.VRC_RING_ORDER, 1)])
@pytest.mark.parametrize("count,bucket", [(1000, 300), (1000, 1000), (1000, 4096), (999, 111)])
def test_bucketed_plan_runs_each_bucket_on_its_slice(mode, per_bucket, count, bucket):
    """One all-reduce per bucket, in bucket order, each touching only its
    bucket's slice of every rank buffer; the ring and halving-doubling ones
    partition the bucket as a buffer of its own."""
    n = 8
    send, recv = buffers(n)
    ops, launches = vrc.plan(vrc.COLL_ALLREDUCE_BUCKETED, send, recv, count, bucket, vrc.VRC_FP32, mode)
    nb = vrc.bucket_count(count, bucket)
    assert launches == nb * per_bucket
    for k in range(nb):
        lo, hi = k * bucket * E, min(count, (k + 1) * bucket) * E
        want, _ = vrc.plan(vrc.COLL_ALLREDUCE, [a + lo for a in send], [a + lo for a in recv], (hi - lo) // E, 1,
                           vrc.VRC_FP32, mode)
        got = [dict(o, launch=o["launch"] - k * per_bucket) for o in ops if k * per_bucket <= o["launch"] <
               (k + 1) * per_bucket]
        assert got == want
        for o in got:
            for key in ("a", "b", "d"):
                if o[key]:
                    rank, off = owner(o[key], send if o[key] < RECV_BASE else recv)
                    assert lo <= off < hi


def test_bucketed_plan_selects_per_bucket():
    """VRC_SELECT resolves each bucket by its own size: 8 ranks, 80 MiB fp32
    per rank in 40 MiB buckets take halving-doubling (6 launches each);
    the same buffers in one bucket take the ring (14)."""
    n, count = 8, 20 << 20
    send, recv = wide_buffers(n)
    _, halves = vrc.plan(vrc.COLL_ALLREDUCE_BUCKETED, send, recv, count, count // 2, vrc.VRC_FP32, vrc.VRC_SELECT)
    _, whole = vrc.plan(vrc.COLL_ALLREDUCE_BUCKETED, send, recv, count, count, vrc.VRC_FP32, vrc.VRC_SELECT)
    assert (halves, whole) == (12, 14)


def test_bucketed_plan_validates():
    send, recv = buffers(4)
    for bucket, mode, status in ((0, vrc.VRC_FUSED, vrc.VRC_ERR_INVALID_ARG),
                                 (10, vrc.VRC_TREE, vrc.VRC_ERR_UNSUPPORTED)):
        with pytest.raises(vrc.VrcError) as e:
            vrc.plan(vrc.COLL_ALLREDUCE_BUCKETED, send, recv, 100, bucket, vrc.VRC_FP32, mode)
        assert e.value.status == status
    send3, recv3 = buffers(3)
    with pytest.raises(vrc.VrcError) as e:
        vrc.plan(vrc.COLL_ALLREDUCE_BUCKETED, send3, recv3, 100, 10, vrc.VRC_FP32, vrc.VRC_HD)
    assert e.value.status == vrc.VRC_ERR_INVALID_ARG


@pytest.mark.parametrize("n,count,want", [
    (12, 1000, "tree"),                        # saves 11 - 8 = 3 launches
    (12, 3 * (128 << 10) // 2, "tree"),        # exactly 3 x 128 KiB of fp16 per rank
    (12, 3 * (128 << 10) // 2 + 1, "ring"),
    (10, (128 << 10) // 2, "tree"),            # saves one launch: up to 128 KiB
    (10, (128 << 10) // 2 + 1, "ring"),
    (15, 6 * (128 << 10) // 2, "tree"),
    (9, 100, "ring"), (7, 100, "ring"), (6, 100, "ring"), (3, 100, "ring"),  # no launch saved
    (8, 100, "hd"), (16, 5000, "hd"),          # powers of two: halving-doubling
])
def test_select_all_gather_follows_the_tree_rule(n, count, want):
    """VRC_SELECT for the all-gather: the binomial tree at rank counts that
    are not powers of two while it saves L = (N-1) - 2 ceil(log2 N) launches
    and each rank's input holds at most L x 128 KiB; the reduce collectives
    never take the tree."""
    send, recv = wide_buffers(n)
    mode = {"tree": vrc.VRC_TREE, "ring": vrc.VRC_RING, "hd": vrc.VRC_HD}[want]
    got = vrc.plan(vrc.COLL_ALL_GATHER, send, recv, count, 1, vrc.VRC_FP16, vrc.VRC_SELECT)
    assert got == vrc.plan(vrc.COLL_ALL_GATHER, send, recv, count, 1, vrc.VRC_FP16, mode)
    if want == "tree":
        for coll in (vrc.COLL_ALLREDUCE, vrc.COLL_REDUCE_SCATTER):
            assert vrc.plan(coll, send, recv, count, 1, vrc.VRC_FP16, vrc.VRC_SELECT) == \
                vrc.plan(coll, send, recv, count, 1, vrc.VRC_FP16, vrc.VRC_RING)


def test_plan_validates_like_the_call():
    send, recv = buffers(3)
    with pytest.raises(vrc.VrcError):
        vrc.plan(vrc.COLL_ALLREDUCE, send, recv, 100, 1, vrc.VRC_FP32, vrc.VRC_HD)  # not a power of two
    with pytest.raises(vrc.VrcError):
        vrc.plan(vrc.COLL_ALLREDUCE, send, [recv[0], recv[0], recv[2]], 100, 1, vrc.VRC_FP32, vrc.VRC_RING)
    assert vrc.lib().vrc_last_hip_error() == 0


@pytest.mark.parametrize("n,count,esize_dtype,want", [
    (8, 1000, vrc.VRC_FP32, "hd"),
    (8, (64 << 20) // 4, vrc.VRC_FP32, "hd"),          # exactly the limit: halving-doubling
    (8, (64 << 20) // 4 + 1, vrc.VRC_FP32, "ring"),    # one element over: ring
    (8, (64 << 20) // 2 + 1, vrc.VRC_BF16, "ring"),
    (6, 1000, vrc.VRC_FP32, "ring"),                   # not a power of two
    (16, 5, vrc.VRC_INT32, "hd"),
    (2, 10, vrc.VRC_FP16, "hd"),
])
def test_select_follows_the_documented_rule(n, count, esize_dtype, want):
    """VRC_SELECT: halving-doubling for power-of-two N and at most 64 MiB per
    rank, else the ring; the plan shows which algorithm ran."""
    send, recv = wide_buffers(n)
    ops, launches = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, esize_dtype, vrc.VRC_SELECT)
    ref_ops, ref_launches = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, esize_dtype,
                                     vrc.VRC_HD if want == "hd" else vrc.VRC_RING)
    assert (ops, launches) == (ref_ops, ref_launches)
    assert launches == (2 * (n.bit_length() - 1) if want == "hd" else 2 * (n - 1))


@pytest.mark.parametrize("coll", [vrc.COLL_REDUCE_SCATTER, vrc.COLL_ALL_GATHER])
@pytest.mark.parametrize("count,want", [(4096, "hd"), ((64 << 20) // 2 + 8, "ring")])
def test_select_for_the_halves(coll, count, want):
    n = 8
    send, recv = wide_buffers(n)
    got = vrc.plan(coll, send, recv, count, 1, vrc.VRC_FP16, vrc.VRC_SELECT)
    ref = vrc.plan(coll, send, recv, count, 1, vrc.VRC_FP16, vrc.VRC_HD if want == "hd" else vrc.VRC_RING)
    assert got == ref
