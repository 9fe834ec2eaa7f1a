"""The collectives can be captured into a HIP graph: the library allocates
nothing, never synchronises and enqueues kernels only (no memsets).  Each
test captures one call, then replays the graph several times; between
replays the inputs are overwritten eagerly, and every replay is checked
against the oracle for the inputs it saw."""
import pytest
import torch

import oracle
import workloads
from tests.parity_util import assert_bitwise, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = ("ring", "fused", "ring_chained", "ring_order", "hd", "hd_order")


@pytest.fixture(scope="module")
def vrc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_all_reduce_virtual_amd as m
    return m


def oracle_allreduce(orc, hx, dtype, mode):
    if mode in ("ring", "ring_chained", "ring_order"):
        return orc.ring_allreduce(hx, dtype)
    if mode in ("hd", "hd_order"):
        return orc.hd_allreduce(hx, dtype)
    return orc.fused_allreduce(hx, dtype)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype,count", [("int32", 4099), ("bf16", 300007)])
def test_captured_allreduce_replays(vrc, mode, dtype, count):
    print(f"graph allreduce {mode} {dtype} {count}", flush=True)
    orc = oracle.get()
    n = 8
    xs = workloads.random_ranks(n, count, dtype, seed=500, device=DEV)
    ys = [torch.empty_like(x) for x in xs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up outside the capture
        vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = workloads.random_ranks(n, count, dtype, seed=600 + rep, device=DEV)
        for x, f in zip(xs, fresh):
            x.copy_(f)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle_allreduce(orc, host(fresh), dtype, mode)
        for r in range(n):
            assert_bitwise(workloads.to_numpy(ys[r]), want[r], f"replay {rep} {mode} {dtype} rank {r}")


@pytest.mark.parametrize("mode", ["ring", "fused", "ring_chained", "hd"])
def test_captured_reduce_scatter_and_all_gather(vrc, mode):
    print(f"graph rs/ag {mode}", flush=True)
    orc = oracle.get()
    n = 8
    xs = workloads.random_ranks(n, (8, 4096), "fp16", seed=501, device=DEV)
    rs = vrc.vrc_reduce_scatter(xs, dim=-1, mode=mode)
    ag = vrc.vrc_all_gather(rs, dim=-1, mode=mode)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vrc.vrc_reduce_scatter(xs, recv=rs, dim=-1, mode=mode)
        vrc.vrc_all_gather(rs, recv=ag, dim=-1, mode=mode)
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = workloads.random_ranks(n, (8, 4096), "fp16", seed=700 + rep, device=DEV)
        for x, f in zip(xs, fresh):
            x.copy_(f)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        hx = host(fresh)
        if mode in ("ring", "ring_chained"):
            want = orc.ring_reduce_scatter(hx, "fp16", outer=8)
        elif mode == "hd":
            want = orc.hd_reduce_scatter(hx, "fp16", outer=8)
        else:
            want = orc.fused_reduce_scatter(hx, "fp16", outer=8)
        gathered = orc.ring_all_gather(want, "fp16", outer=8)
        for c in range(n):
            assert_bitwise(workloads.to_numpy(rs[c]), want[c], f"replay {rep} rs {mode} chunk {c}")
            assert_bitwise(workloads.to_numpy(ag[c]), gathered[c], f"replay {rep} ag {mode} rank {c}")


@pytest.mark.parametrize("n", [5, 8])
def test_captured_tree_all_gather(vrc, n):
    """The binomial-tree all-gather (2 ceil(log2 N) launches) captured once
    and replayed on fresh inputs."""
    print(f"graph tree all-gather n={n}", flush=True)
    orc = oracle.get()
    xs = workloads.random_ranks(n, (3, 4097), "bf16", seed=520 + n, device=DEV)
    ag = vrc.vrc_all_gather(xs, dim=-1, mode="tree")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vrc.vrc_all_gather(xs, recv=ag, dim=-1, mode="tree")
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = workloads.random_ranks(n, (3, 4097), "bf16", seed=720 + rep, device=DEV)
        for x, f in zip(xs, fresh):
            x.copy_(f)
        for y in ag:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = orc.tree_all_gather(host(fresh), "bf16", outer=3)
        for r in range(n):
            assert_bitwise(workloads.to_numpy(ag[r]), want[r], f"replay {rep} tree rank {r}")


@pytest.mark.parametrize("mode", ["fused", "hd_order", "ring_order"])
def test_captured_realigned_allreduce(vrc, mode):
    """Outputs on eight different offsets modulo 128 bytes, above 64 MiB
    moved: the realigned kernel (vrc_plan says so) captured and replayed,
    with the eager program's own work between replays."""
    print(f"graph realigned allreduce {mode}", flush=True)
    orc = oracle.get()
    n, count = 8, 2 * (1 << 20) + 77  # bf16: 64 MiB + moved
    xs = workloads.random_ranks(n, count, "bf16", seed=502, device=DEV, sigma=1e-2)
    ys = []
    for r in range(n):
        off = (11 * r + 3) % 64  # elements: 2-byte shifts across the whole line
        buf = torch.zeros(count + 64, dtype=torch.bfloat16, device=DEV)
        ys.append(buf[off:off + count])
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, [x.data_ptr() for x in xs], [y.data_ptr() for y in ys], count, 1,
                      vrc.VRC_BF16, vrc.MODES[mode])
    assert ops[0]["kind"].endswith("_realigned")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = workloads.random_ranks(n, count, "bf16", seed=800 + rep, device=DEV, sigma=1e-2)
        for x, f in zip(xs, fresh):
            x.copy_(f)
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle_allreduce(orc, host(fresh), "bf16", mode)
        for r in range(n):
            assert_bitwise(workloads.to_numpy(ys[r]), want[r], f"replay {rep} realigned {mode} rank {r}")
