"""Plans built from several threads at once: vrc_plan keeps its recording
state per thread, so concurrent calls (ctypes drops the GIL around them)
must each get exactly the plan a lone call gets."""
import threading

import ring_all_reduce_virtual_amd as vrc

SEND_BASE, RECV_BASE, STRIDE = 0x10000000, 0x40000000, 1 << 24


def plan_for(k):
    n = (2, 4, 8, 16)[k % 4]
    mode = (vrc.VRC_RING, vrc.VRC_HD)[k % 2]
    send = [SEND_BASE + r * STRIDE for r in range(n)]
    recv = [RECV_BASE + r * STRIDE for r in range(n)]
    return vrc.plan(vrc.COLL_ALLREDUCE, send, recv, 1000 + 37 * k, 1, vrc.VRC_FP16, mode)


def test_concurrent_plans_are_isolated():
    cases = list(range(16))
    want = {k: plan_for(k) for k in cases}
    got, errors = {}, []
    start = threading.Barrier(len(cases))

    def worker(k):
        try:
            start.wait()
            for _ in range(50):
                p = plan_for(k)
                if p != want[k]:
                    errors.append((k, "differs"))
                    return
            got[k] = p
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors
    assert got == want
