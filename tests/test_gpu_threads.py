"""Several host threads call the library at once, each on its own stream
with its own buffers: every result must match the oracle bit for bit."""
import threading

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


def test_concurrent_callers_on_their_own_streams(vrc):
    print(f"threads: 4 callers x {len(vrc.REDUCE_MODES)} modes", flush=True)
    orc = oracle.get()
    n, count = 8, 200003
    modes = list(vrc.REDUCE_MODES)
    inputs = [workloads.random_ranks(n, count, "bf16", seed=900 + t, device=DEV) for t in range(4)]
    outs = [{m: [torch.empty_like(x) for x in inputs[t]] for m in modes} for t in range(4)]
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(4)

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                for _ in range(5):
                    for m in modes:
                        vrc.vrc_allreduce(inputs[t], recv=outs[t][m], mode=m)
            s.synchronize()
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors
    for t in range(4):
        hx = host(inputs[t])
        want = {"ring": orc.ring_allreduce(hx, "bf16"), "fused": orc.fused_allreduce(hx, "bf16"),
                "hd": orc.hd_allreduce(hx, "bf16")}
        want["ring_chained"] = want["ring_order"] = want["ring"]
        want["hd_order"] = want["hd"]
        want["select"] = want["hd"]  # 8 ranks (a power of two) of about 400 KB: halving-doubling
        for m in modes:
            for r in range(n):
                assert_bitwise(workloads.to_numpy(outs[t][m][r]), want[m][r], f"thread {t} {m} rank {r}")
