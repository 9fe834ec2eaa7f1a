"""The collectives are stream-ordered: running them on their own stream,
concurrently with compute on another (the pages' compute/communication
overlap), must not change a single bit of the result."""
import pytest
import torch

import oracle
import workloads
from tests.parity_util import assert_bitwise, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def vrc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_all_reduce_virtual_amd as m
    return m


@pytest.mark.parametrize("mode", ["fused", "ring", "ring_chained", "ring_order", "hd", "hd_order"])
def test_allreduce_concurrent_with_matmul(vrc, mode):
    print(f"overlap {mode}", flush=True)
    orc = oracle.get()
    xs = workloads.make_inputs(workloads.WORKLOADS["allreduce_fp32_n8_16mib"], DEV)
    g = torch.Generator(device=DEV).manual_seed(3)
    a = torch.randn(4096, 4096, generator=g, device=DEV)
    b = torch.randn(4096, 4096, generator=g, device=DEV)
    c_ref = torch.matmul(a, b)
    torch.cuda.synchronize()
    s_comp, s_comm = torch.cuda.Stream(), torch.cuda.Stream()
    start = torch.cuda.Event()
    start.record()
    s_comp.wait_event(start)
    s_comm.wait_event(start)
    with torch.cuda.stream(s_comp):
        cs = [torch.matmul(a, b) for _ in range(4)]
    ys = vrc.vrc_allreduce(xs, mode=mode, stream=s_comm)
    s_comp.synchronize()
    s_comm.synchronize()
    hx = host(xs)
    if mode in ("ring", "ring_chained", "ring_order"):
        want = orc.ring_allreduce(hx, "fp32")
    elif mode in ("hd", "hd_order"):
        want = orc.hd_allreduce(hx, "fp32")
    else:
        want = orc.fused_allreduce(hx, "fp32")
    for r in range(8):
        assert_bitwise(workloads.to_numpy(ys[r]), want[r], f"{mode} under overlap rank {r}")
    for c in cs:
        assert torch.allclose(c, c_ref, rtol=1e-3, atol=1e-2)
