"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU."""
import ctypes as C
import os
import re

import pytest

import ring_all_reduce_virtual_amd as vrc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vrc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vrc_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("vrc_allreduce", "vrc_reduce_scatter", "vrc_all_gather", "vrc_chunk_range",
                 "vrc_status_string", "vrc_last_hip_error", "vrc_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(vrc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_version_and_status_strings():
    header = open(os.path.join(ROOT, "include", "vrc.h")).read()
    declared = int(re.search(r"#define VRC_VERSION (\d+)", header).group(1))
    assert vrc.version() == declared == vrc.ABI_VERSION == 106
    for st in range(5):
        assert vrc.lib().vrc_status_string(st).decode().startswith("VRC_")
    assert b"unknown" in vrc.lib().vrc_status_string(99)
    assert vrc.lib().vrc_last_hip_error() == 0


@pytest.mark.parametrize("count,n", [(4099, 4), (0, 3), (7, 8), (16, 16), (1 << 28, 8), (10, 1)])
def test_chunk_range_follows_the_remainder_rule(count, n):
    # equal chunks of count // n, the last one takes the remainder
    base = count // n
    for c in range(n):
        off, ln = vrc.chunk_range(count, n, c)
        assert off == c * base
        assert ln == (count - (n - 1) * base if c == n - 1 else base)


def test_chunk_range_rejects_bad_arguments():
    for count, n, c in ((10, 0, 0), (10, 4, 4), (10, 4, -1), (10, 17 * 0, 0)):
        with pytest.raises(vrc.VrcError):
            vrc.chunk_range(count, n, c)


FAKE = 0x10000000  # host-side stand-in addresses: these calls must fail before any GPU work


def addrs(base, n, stride):
    return [base + k * stride for k in range(n)]


def test_invalid_arguments_return_before_any_gpu_call():
    n, count = 4, 1024
    x = addrs(FAKE, n, 1 << 20)
    y = addrs(FAKE + (64 << 20), n, 1 << 20)
    L = vrc.lib()
    # null arrays
    assert L.vrc_allreduce(None, None, n, count, 1, 0, 0, None) == vrc.VRC_ERR_INVALID_ARG
    # nranks out of range
    assert vrc.raw_allreduce([], [], count, vrc.VRC_FP32, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_allreduce(addrs(FAKE, 17, 1 << 20), addrs(FAKE + (64 << 20), 17, 1 << 20), count,
                             vrc.VRC_FP32, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    # unknown dtype / op / mode
    assert vrc.raw_allreduce(x, y, count, 7, vrc.VRC_RING) == vrc.VRC_ERR_UNSUPPORTED
    assert vrc.raw_allreduce(x, y, count, vrc.VRC_FP32, 9) == vrc.VRC_ERR_UNSUPPORTED
    assert vrc.raw_allreduce(x, y, count, vrc.VRC_FP32, vrc.VRC_RING, op=3) == vrc.VRC_ERR_UNSUPPORTED
    assert vrc.raw_all_gather(x, y, count, 1, vrc.VRC_FP32, 9) == vrc.VRC_ERR_UNSUPPORTED
    # null device pointer with count > 0
    assert vrc.raw_allreduce([0] + x[1:], y, count, vrc.VRC_FP32, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_allreduce(x, y[:3] + [0], count, vrc.VRC_FP32, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    # shapes: count not divisible by outer, row not divisible by nranks
    assert vrc.raw_reduce_scatter(x, y, 1000, 3, vrc.VRC_FP16, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_reduce_scatter(x, y, 1002, 2, vrc.VRC_FP16, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_reduce_scatter(x, y, 1000, 0, vrc.VRC_FP16, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_all_gather(x, y, 1000, 3, vrc.VRC_FP16, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_all_gather(x, y, 1000, 0, vrc.VRC_FP16, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    # counts whose byte sizes could wrap 64 bits (2^62 int32 all-gathered over 4 ranks is 2^66 bytes)
    huge = 1 << 62
    assert vrc.raw_allreduce(x, y, huge, vrc.VRC_FP32, vrc.VRC_FUSED) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_all_gather(x, y, huge, 1, vrc.VRC_INT32, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_reduce_scatter(x, y, huge, 1, vrc.VRC_FP32, vrc.VRC_RING) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.lib().vrc_last_hip_error() == 0


def test_count_zero_is_a_no_op_even_with_null_pointers():
    for mode in (vrc.VRC_RING, vrc.VRC_FUSED):
        assert vrc.raw_allreduce([0, 0, 0], [0, 0, 0], 0, vrc.VRC_BF16, mode) == vrc.VRC_OK
        assert vrc.raw_reduce_scatter([0, 0], [0, 0], 0, 1, vrc.VRC_FP16, mode) == vrc.VRC_OK
        assert vrc.raw_all_gather([0, 0], [0, 0], 0, 1, vrc.VRC_INT32, mode) == vrc.VRC_OK


def test_alias_detection():
    n, count, E = 4, 1024, 4
    x = addrs(FAKE, n, 1 << 20)
    y = addrs(FAKE + (64 << 20), n, 1 << 20)
    A = vrc.VRC_ERR_ALIAS
    # two outputs overlap
    y2 = list(y)
    y2[1] = y[0] + 8
    assert vrc.raw_allreduce(x, y2, count, vrc.VRC_FP32, vrc.VRC_RING) == A
    # output overlaps another rank's input
    y3 = list(y)
    y3[2] = x[1]
    assert vrc.raw_allreduce(x, y3, count, vrc.VRC_FP32, vrc.VRC_FUSED) == A
    # partial overlap with its own input (not exactly in place)
    y4 = list(y)
    y4[0] = x[0] + E
    assert vrc.raw_allreduce(x, y4, count, vrc.VRC_FP32, vrc.VRC_RING) == A
    # reduce-scatter / all-gather may not run in place
    assert vrc.raw_reduce_scatter(x, x, count, 1, vrc.VRC_FP32, vrc.VRC_RING) == A
    assert vrc.raw_all_gather(x, x, count, 1, vrc.VRC_FP32, vrc.VRC_FUSED) == A
    # all-gather outputs are n times larger: adjacent 1 MiB strides overlap
    ag_y = addrs(FAKE + (64 << 20), n, count * E)  # each output needs n*count*E bytes
    assert vrc.raw_all_gather(x, ag_y, count, 1, vrc.VRC_FP32, vrc.VRC_RING) == A


def test_halving_doubling_needs_a_power_of_two():
    x = addrs(FAKE, 3, 1 << 20)
    y = addrs(FAKE + (64 << 20), 3, 1 << 20)
    for mode in (vrc.VRC_HD, vrc.VRC_HD_ORDER):
        assert vrc.raw_allreduce(x, y, 1000, vrc.VRC_FP32, mode) == vrc.VRC_ERR_INVALID_ARG
        assert vrc.raw_reduce_scatter(x, y, 1000, 1, vrc.VRC_FP32, mode) == vrc.VRC_ERR_INVALID_ARG
        assert vrc.raw_all_gather(x, y, 1000, 1, vrc.VRC_FP32, mode) == vrc.VRC_ERR_INVALID_ARG
    assert vrc.raw_allreduce(x, y, 1000, vrc.VRC_FP32, 7) == vrc.VRC_ERR_UNSUPPORTED
