"""bench.py's host-side pieces, on the CPU: the refusal of more than one
GPU, the algorithmic byte counts, the selector rule it mirrors, and the
counter record it reads for roofline.traffic."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("mode,n,size,want", [
    ("fused", 8, 100, 1600), ("ring_order", 8, 100, 1600), ("hd_order", 4, 10, 80),
    ("ring", 8, 100, 3500), ("ring_chained", 8, 100, 3500), ("hd", 8, 100, 3500),
    ("select", 8, 100, 3500), ("select", 6, 100, 2500),
])
def test_algorithmic_bytes(mode, n, size, want):
    """2*N*S for the single-pass modes, 5(N-1)*S for the step algorithms."""
    assert bench.alg_bytes(mode, n, size) == want


def test_selector_rule_matches_the_header():
    header = open(os.path.join(ROOT, "include", "vrc.h")).read()
    assert "#define VRC_SELECT_HD_MAX_BYTES (64ull << 20)" in header
    assert bench.selected("select", 8, 64 << 20) == "hd"
    assert bench.selected("select", 8, (64 << 20) + 1) == "ring"
    assert bench.selected("select", 6, 1024) == "ring"
    assert bench.selected("fused", 6, 1024) == "fused"


def test_suite_bytes_per_collective():
    w = workloads.WORKLOADS["reduce_scatter_fp16_n8_act"]
    s = w.count * w.esize
    assert bench.suite_bytes(w, "ring") == 3 * 7 * s
    assert bench.suite_bytes(w, "fused") == 9 * s
    assert bench.suite_bytes(w, "hd") == 9 * s  # runs as one butterfly launch
    g = workloads.WORKLOADS["all_gather_fp16_n8_heads"]
    sg = g.count * g.esize
    assert bench.suite_bytes(g, "ring") == 2 * 64 * sg
    assert bench.suite_bytes(g, "fused") == 8 * sg + 64 * sg
    assert bench.suite_bytes(g, "ring_chained") == 15 * 8 * sg


def test_recorded_traffic():
    """roofline.traffic comes from the committed counter summary, only while
    it was taken on the kernel sources in the tree; its bytes are within
    0.2 % of the headline's algorithmic 2*N*S (the phased kernel's meetings
    add about 0.1 %: device-scope polls and atomics of its meeting count)."""
    assert bench.recorded_traffic(workloads.HEADLINE, "select") is None
    t = bench.recorded_traffic(workloads.HEADLINE, "fused")
    if t is None:
        pytest.skip("the committed counters were taken on other kernel sources; re-take them on the GPU")
    assert abs(t / 8589934592 - 1) < 2e-3


def test_recorded_mixed_stream():
    """The mixed-stream counters come from the committed summary on the same
    kernel sources; the figures the headline line carries are present and
    plausible (fractions within [0, 1], latencies positive)."""
    m = bench.recorded_mixed_stream()
    if m is None:
        pytest.skip("the committed counters were taken on other kernel sources; re-take them on the GPU")
    for k in ("fused_read_latency_cycles", "fused_l2_busy", "fused_write_credit_stall",
              "fused_too_many_write_requests_stall", "fused_reads_in_flight_per_channel"):
        assert k in m
    assert m["fused_read_latency_cycles"] > 0 and 0 <= m["fused_l2_busy"] <= 1
    assert 0 <= m["fused_write_credit_stall"] <= 1 and 0 <= m["fused_too_many_write_requests_stall"] <= 1


def test_host_info_fields():
    info = bench.host_info()
    assert info["nproc"] >= 1 and info["affinity"] >= 1
    json.dumps(info)


def test_profile_rows_name_real_workloads_and_modes():
    """Every counter row names a workload (or one of its sweep sizes) and a
    mode the library has; every workload is covered in fused and ring form."""
    import ring_all_reduce_virtual_amd as vrc
    import workloads
    seen = set()
    for name, mode in bench.PROFILE_ROWS:
        base, _, count = name.partition("@")
        w = workloads.WORKLOADS[base]
        assert not count or int(count) in w.sweep
        assert mode in vrc.MODES
        seen.add((base, mode))
    for base in workloads.WORKLOADS:
        assert (base, "fused") in seen and (base, "ring") in seen


def test_profile_offset_rows_are_headline_all_reduces():
    """The mixed-offset counter rows run the headline workload, with every
    operand on its own offset, in every all-reduce mode that has its own
    kernel family (the realigned ones among them)."""
    import ring_all_reduce_virtual_amd as vrc
    modes = set()
    for name, mode in bench.PROFILE_OFFSET_ROWS:
        assert name == workloads.HEADLINE + bench.OFFSET_SUFFIX
        assert mode in vrc.REDUCE_MODES
        modes.add(mode)
    assert {"fused", "hd_order", "ring_order", "ring_chained", "ring"} <= modes
