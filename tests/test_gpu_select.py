"""VRC_SELECT on the GPU: the plan names the algorithm the library picked
(halving-doubling or ring, by the rule in include/vrc.h), and the result
must be that algorithm's bits, checked against its oracle."""
import pytest
import torch

import oracle
import workloads
from tests.parity_util import assert_bitwise, equal_to_expected, host, oracle_every_element, ranks_identical

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CODES = {"int32": 0, "fp32": 1, "fp16": 2, "bf16": 3}


@pytest.fixture(scope="module")
def vrc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_all_reduce_virtual_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def picked(vrc, coll, xs, ys, count, outer, dtype):
    """'hd', 'ring' or 'tree', from the launch plan of the same call."""
    send = [x.data_ptr() for x in xs]
    recv = [y.data_ptr() for y in ys]
    got = vrc.plan(coll, send, recv, count, outer, CODES[dtype], vrc.VRC_SELECT)
    for name, code in (("hd", vrc.VRC_HD), ("ring", vrc.VRC_RING), ("tree", vrc.VRC_TREE)):
        try:
            if vrc.plan(coll, send, recv, count, outer, CODES[dtype], code) == got:
                return name
        except vrc.VrcError:  # halving-doubling refuses rank counts that are not powers of two, the
            pass              # reduce collectives the tree
    raise AssertionError("VRC_SELECT planned none of halving-doubling, the ring and the tree")


def expected_algorithm(n, nbytes):
    return "hd" if n & (n - 1) == 0 and nbytes <= (64 << 20) else "ring"


@pytest.mark.parametrize("n,count,dtype", [(8, 100003, "fp32"), (6, 100003, "fp32"), (16, 4099, "bf16"),
                                           (3, 7, "int32"), (1, 1000, "fp16"), (4, 65536 * 3 + 1, "fp16")])
def test_select_small_allreduce(vrc, orc, n, count, dtype):
    print(f"select allreduce n={n} count={count} {dtype}", flush=True)
    xs = workloads.random_ranks(n, count, dtype, seed=40 + n, device=DEV)
    ys = [torch.empty_like(x) for x in xs]
    alg = picked(vrc, vrc.COLL_ALLREDUCE, xs, ys, count, 1, dtype)
    assert alg == expected_algorithm(n, count * xs[0].element_size()) or n == 1
    vrc.vrc_allreduce(xs, recv=ys, mode="select")
    torch.cuda.synchronize()
    hx = host(xs)
    want = orc.hd_allreduce(hx, dtype) if alg == "hd" else orc.ring_allreduce(hx, dtype)
    for r, y in enumerate(host(ys)):
        assert_bitwise(y, want[r], f"select n={n} {dtype} ({alg}) rank {r}")


@pytest.mark.parametrize("extra,alg", [(0, "hd"), (1, "ring")])
def test_select_at_the_limit(vrc, orc, extra, alg):
    """8 ranks of exactly 64 MiB run halving-doubling; one element more runs the ring."""
    count = (64 << 20) // 4 + extra
    print(f"select allreduce at the limit: count={count} ({alg})", flush=True)
    xs = workloads.random_ranks(8, count, "fp32", seed=77, device=DEV)
    ys = [torch.empty_like(x) for x in xs]
    assert picked(vrc, vrc.COLL_ALLREDUCE, xs, ys, count, 1, "fp32") == alg
    vrc.vrc_allreduce(xs, recv=ys, mode="select")
    torch.cuda.synchronize()
    ranks_identical(ys, f"select {alg}")
    at = orc.hd_allreduce_at if alg == "hd" else orc.ring_allreduce_at
    want = torch.from_numpy(oracle_every_element(at, host(xs), "fp32", count)).to(DEV)
    equal_to_expected(ys, want, f"select at the limit ({alg})")


def test_select_large_workload_runs_the_ring(vrc, orc):
    w = workloads.WORKLOADS["allreduce_fp16_n8_128mib"]
    print(f"select {w.name}", flush=True)
    xs = workloads.make_inputs(w, DEV)
    ys = [torch.empty_like(x) for x in xs]
    assert picked(vrc, vrc.COLL_ALLREDUCE, xs, ys, w.count, 1, "fp16") == "ring"
    vrc.vrc_allreduce(xs, recv=ys, mode="select")
    torch.cuda.synchronize()
    want = torch.from_numpy(oracle_every_element(orc.ring_allreduce_at, host(xs), "fp16", w.count)).to(DEV)
    equal_to_expected(ys, want, f"select {w.name}")


@pytest.mark.parametrize("n", [8, 6])
def test_select_halves(vrc, orc, n):
    print(f"select reduce-scatter / all-gather n={n}", flush=True)
    shape = (4, n * 96)
    xs = workloads.random_ranks(n, shape, "fp16", seed=90 + n, device=DEV)
    rs = vrc.vrc_reduce_scatter(xs, dim=-1, mode="select")
    ag = vrc.vrc_all_gather(rs, dim=-1, mode="select")
    torch.cuda.synchronize()
    hx = host(xs)
    alg = expected_algorithm(n, xs[0].numel() * 2)
    assert picked(vrc, vrc.COLL_REDUCE_SCATTER, xs, rs, xs[0].numel(), 4, "fp16") == alg
    want = (orc.hd_reduce_scatter if alg == "hd" else orc.ring_reduce_scatter)(hx, "fp16", outer=4)
    gathered = orc.ring_all_gather(want, "fp16", outer=4)
    for c in range(n):
        assert_bitwise(workloads.to_numpy(rs[c]), want[c], f"select rs n={n} ({alg}) chunk {c}")
        assert_bitwise(workloads.to_numpy(ag[c]), gathered[c], f"select ag n={n} rank {c}")


@pytest.mark.parametrize("n,count,alg", [(12, 1000, "tree"), (14, 300000, "tree"), (12, 300000, "ring"),
                                         (10, 70000, "ring")])
def test_select_all_gather_tree(vrc, orc, n, count, alg):
    """The all-gather at rank counts that are not powers of two takes the
    binomial tree while it saves launches and the input is small (at most
    128 KiB per launch saved); its bits are the tree oracle's."""
    print(f"select all-gather n={n} count={count} ({alg})", flush=True)
    xs = workloads.random_ranks(n, count, "fp16", seed=95 + n, device=DEV)
    ys = [torch.empty(n * count, dtype=xs[0].dtype, device=DEV) for _ in range(n)]
    assert picked(vrc, vrc.COLL_ALL_GATHER, xs, ys, count, 1, "fp16") == alg
    vrc.vrc_all_gather(xs, recv=ys, mode="select")
    torch.cuda.synchronize()
    want = (orc.tree_all_gather if alg == "tree" else orc.ring_all_gather)(host(xs), "fp16")
    for r in range(n):
        assert_bitwise(workloads.to_numpy(ys[r]), want[r], f"select all-gather n={n} ({alg}) rank {r}")
