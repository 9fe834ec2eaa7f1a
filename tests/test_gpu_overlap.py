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


# ---------------------------------------------------------------------------
# bucketed all-reduce fed by a producer stream: bucket k of every rank is
# written on the compute stream, which records ready[k]; the communication
# stream waits on ready[k] before it all-reduces bucket k
# ---------------------------------------------------------------------------
def want_bucketed(orc, hx, dtype, mode, count, bucket):
    """The oracle's all-reduce of each bucket on its own (the ring folds a
    bucket's chunk c from rank c); the rank fold and the butterfly do not
    depend on the partition, so those are also checked against the whole."""
    import numpy as np
    parts = []
    for lo in range(0, count, bucket):
        sl = [x[lo:lo + bucket] for x in hx]
        if mode in ("ring", "ring_chained", "ring_order"):
            parts.append(orc.ring_allreduce(sl, dtype)[0])
        elif mode in ("hd", "hd_order"):
            parts.append(orc.hd_allreduce(sl, dtype)[0])
        else:
            parts.append(orc.fused_allreduce(sl, dtype)[0])
    out = np.concatenate(parts) if parts else np.zeros(0, hx[0].dtype)
    if mode in ("fused", "hd", "hd_order"):
        whole = (orc.fused_allreduce if mode == "fused" else orc.hd_allreduce)(hx, dtype)[0]
        assert np.array_equal(out.view(np.uint8), whole.view(np.uint8))
    return out


@pytest.mark.parametrize("mode", ["fused", "ring", "ring_order", "ring_chained", "hd", "hd_order", "select"])
@pytest.mark.parametrize("count,bucket", [(3 * (1 << 20) + 17, 1 << 20), (2_000_003, 777_777), (4099, 5000)])
def test_bucketed_allreduce_behind_a_producer(vrc, mode, count, bucket):
    """The producer writes each bucket of every rank (a copy from the seeded
    inputs, behind a matmul so the stream is busy) and records the bucket's
    event; the all-reduce runs on another stream, bucket by bucket, each
    bucket after its event.  Every element against the oracle's per-bucket
    all-reduce."""
    print(f"bucketed {mode} count={count} bucket={bucket}", flush=True)
    orc = oracle.get()
    n = 8
    src = workloads.random_ranks(n, count, "bf16", seed=610, device=DEV, sigma=1e-2)
    grads = [torch.zeros_like(x) for x in src]
    outs = [torch.full_like(x, 7) for x in src]
    a = torch.randn(2048, 2048, device=DEV)
    torch.cuda.synchronize()
    s_comp, s_comm = torch.cuda.Stream(), torch.cuda.Stream()
    nb = vrc.bucket_count(count, bucket)
    ready = [torch.cuda.Event() for _ in range(nb)]
    with torch.cuda.stream(s_comp):
        for k in range(nb):
            torch.matmul(a, a)  # keeps the producer busy ahead of each bucket
            for g, x in zip(grads, src):
                g[k * bucket:(k + 1) * bucket].copy_(x[k * bucket:(k + 1) * bucket])
            ready[k].record(s_comp)
    vrc.vrc_allreduce_bucketed(grads, recv=outs, bucket=bucket, mode=mode, ready=ready, stream=s_comm)
    s_comm.synchronize()
    s_comp.synchronize()
    want = want_bucketed(orc, host(src), "bf16", mode if mode != "select" else
                         ("hd" if bucket * 2 <= vrc.SELECT_HD_MAX_BYTES else "ring"), count, bucket)
    for r in range(n):
        assert_bitwise(workloads.to_numpy(outs[r]), want, f"bucketed {mode} rank {r}")


def test_bucketed_allreduce_errors(vrc):
    xs = workloads.random_ranks(4, 1000, "fp32", seed=611, device=DEV)
    ev = torch.cuda.Event()
    ev.record()
    for kwargs, status in ((dict(bucket=0), None), (dict(bucket=100, mode="tree"), vrc.VRC_ERR_UNSUPPORTED)):
        with pytest.raises((vrc.VrcError, ValueError)) as e:
            vrc.vrc_allreduce_bucketed(xs, **kwargs)
        if status is not None:
            assert e.value.status == status
    with pytest.raises(ValueError):  # one event per bucket
        vrc.vrc_allreduce_bucketed(xs, bucket=100, ready=[ev])
    rc = vrc.raw_allreduce_bucketed([x.data_ptr() for x in xs], [x.data_ptr() for x in xs], 1000, vrc.VRC_FP32,
                                    vrc.VRC_FUSED, 100, [ev.cuda_event] * 9)
    assert rc == vrc.VRC_ERR_INVALID_ARG  # ten buckets, nine events
