"""The library's launch shapes, checked on the CPU through vrc_plan (which
reports each launch's geometry for a 256-CU device and launches nothing).

These are the host-side rules behind the measured performance: one-wave
workgroups and a loads-in-flight budget for the fused all-reduce from 64 MiB
moved, one-wave workgroups for the single-launch ring all-reduce, 16
workgroups per CU for the fused all-gather, and the ring step shapes by size
and operation count.  The environment overrides are checked in a child
process, since the library reads them once."""
import ctypes as C
import os
import shutil
import subprocess
import sys

import pytest

import ring_all_reduce_virtual_amd as vrc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CUS = 256
ESZ = {vrc.VRC_INT32: 4, vrc.VRC_FP32: 4, vrc.VRC_FP16: 2, vrc.VRC_BF16: 2}


def wide(n):
    """Stand-in rank addresses 4 GiB apart (256-byte aligned)."""
    return [(1 << 40) + r * (1 << 32) for r in range(n)], [(1 << 42) + r * (1 << 32) for r in range(n)]


def gather_out(n, count, esz):
    """All-gather outputs hold n * count elements each: space them further apart."""
    return [(1 << 44) + r * ((n * count * esz + (1 << 32)) // (1 << 32) * (1 << 32)) for r in range(n)]


def launches(ops):
    """One geometry per launch: (kind, grid_x, grid_y, block, vectors), in launch order."""
    out = {}
    for op in ops:
        g = (op["kind"], op["grid_x"], op["grid_y"], op["block"], op["vectors"])
        assert out.setdefault(op["launch"], g) == g, "operations of one launch disagree on its geometry"
    return [out[k] for k in sorted(out)]


def plan_ar(n, count, dtype, mode):
    send, recv = wide(n)
    ops, nl = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, dtype, mode)
    got = launches(ops)
    assert len(got) == nl
    return got


def budget_blocks_per_cu(n, vectors):
    """Largest power of two <= 8 with workgroups x ranks x vectors <= 32."""
    b = 8
    while b > 1 and b * n * vectors > 32:
        b //= 2
    return b


def test_op_desc_layout_matches_the_header():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    src = os.path.join(ROOT, "tests", "_sizeof_op_desc.c")
    exe = os.path.join(ROOT, "tests", "_sizeof_op_desc")
    try:
        with open(src, "w") as fh:
            fh.write('#include <stdio.h>\n#include <stddef.h>\n#include "vrc.h"\n'
                     'int main(void) { printf("%zu %zu %zu\\n", sizeof(vrc_op_desc), '
                     'offsetof(vrc_op_desc, grid_x), offsetof(vrc_op_desc, vectors)); return 0; }\n')
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", exe, src], check=True)
        size, off_grid, off_vec = map(int, subprocess.run([exe], check=True, capture_output=True,
                                                          text=True).stdout.split())
    finally:
        for p in (src, exe):
            if os.path.exists(p):
                os.remove(p)
    assert C.sizeof(vrc.OpDesc) == size
    assert vrc.OpDesc.grid_x.offset == off_grid and vrc.OpDesc.vectors.offset == off_vec


FUSED_SHAPES = {2: (2, 8), 3: (2, 4), 4: (1, 8), 5: (2, 2), 6: (2, 2), 7: (2, 2), 8: (4, 1)}  # n: (per CU, U)


@pytest.mark.parametrize("n", list(range(2, 17)))
def test_fused_allreduce_one_wave_shapes(n):
    """2 GiB moved (above 64 MiB, under three phases of the phased kernel):
    one-wave workgroups taking U consecutive tiles, by rank count: U 8 at 2
    per CU (2 ranks), U 4 at 2 (3), U 8 at 1 (4), U 2 at 2 (5-7), U 1 at 4
    (8) and at 2 (9-16)."""
    count = (1 << 30) // n // 2 // 64 * 64
    bpc, vectors = FUSED_SHAPES.get(n, (2, 1))
    assert vectors * n <= 32
    got = plan_ar(n, count, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert got == [("fused_allreduce", CUS * bpc, 1, 64, vectors)]
    if n & (n - 1) == 0 and n > 2:  # halving-doubling in one launch: the same kernel with the butterfly fold
        assert plan_ar(n, count, vrc.VRC_BF16, vrc.VRC_HD_ORDER) == [("butterfly_allreduce", CUS * bpc, 1, 64,
                                                                      vectors)]


def off_grid_shape(n):
    """U consecutive tiles per wave (the largest U <= 8 with U x N <= 32, at
    least 2) at 64 / (U x N) workgroups per CU, rounded down to a power of two."""
    u = 8
    while u > 2 and u * n > 32:
        u //= 2
    bpc = max(1, 64 // (u * n))
    return 1 << (bpc.bit_length() - 1), u


@pytest.mark.parametrize("n", list(range(2, 17)))
def test_fused_allreduce_outputs_off_one_grid(n):
    """Outputs on different offsets modulo 128 bytes, none in place: the
    realigned kernel, which stores every output on its own 128-byte grid."""
    count = (4 << 30) // n // 2 // 64 * 64
    send, recv = wide(n)
    recv = [a + 2 * r for r, a in enumerate(recv)]
    bpc, u = off_grid_shape(n)
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert launches(ops) == [("fused_allreduce_realigned", CUS * bpc, 1, 64, u)]
    if n in (4, 8, 16):  # at 2 ranks the butterfly is the rank fold
        ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_BF16, vrc.VRC_HD_ORDER)
        assert launches(ops) == [("butterfly_allreduce_realigned", CUS * bpc, 1, 64, u)]


@pytest.mark.parametrize("n", list(range(2, 17)))
def test_ring_order_outputs_off_one_grid(n):
    """The ring-order all-reduce takes its realigned variant on the same
    terms (outputs on different 128-byte offsets, none in place, at least
    64 MiB moved), at the fused kernel's realigned shape; in place, or below
    64 MiB moved, the tile kernel."""
    count = (4 << 30) // n // 2 // 64 * 64
    send, recv = wide(n)
    mixed = [a + 2 * r for r, a in enumerate(recv)]
    bpc, u = off_grid_shape(n)
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, mixed, count, 1, vrc.VRC_BF16, vrc.VRC_RING_ORDER)
    assert launches(ops) == [("ring_order_allreduce_realigned", CUS * bpc, 1, 64, u)]
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, mixed, mixed, count, 1, vrc.VRC_BF16, vrc.VRC_RING_ORDER)
    assert launches(ops)[0][0] == "ring_order_allreduce"
    small = (32 << 20) // (2 * n * 2)
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, mixed, small, 1, vrc.VRC_BF16, vrc.VRC_RING_ORDER)
    assert launches(ops)[0][0] == "ring_order_allreduce"
    # the memory-faithful chain keeps its kernel
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, mixed, count, 1, vrc.VRC_BF16, vrc.VRC_RING_CHAINED)
    assert launches(ops)[0][0] == "chain_allreduce"


@pytest.mark.parametrize("n", [2, 5, 8, 16])
def test_in_place_outputs_off_one_grid_keep_the_tile_kernel(n):
    """In place, the realigned stores would run ahead of the reads of the
    next group: the tile kernel (consecutive tiles, unaligned stores) runs."""
    count = (4 << 30) // n // 2 // 64 * 64
    bufs = [(1 << 40) + r * (1 << 32) + 2 * r for r in range(n)]
    u = 8
    while u > 1 and u * n > 32:
        u //= 2
    bpc = 64 // (u * n)
    bpc = 1 << (bpc.bit_length() - 1)
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, bufs, bufs, count, 1, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert launches(ops) == [("fused_allreduce", CUS * bpc, 1, 64, u)]
    # one output in place is enough
    send, recv = wide(n)
    recv = [a + 2 * r for r, a in enumerate(recv)]
    recv[n - 1] = send[n - 1]
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert launches(ops)[0][0] == "fused_allreduce"


@pytest.mark.parametrize("dtype", [vrc.VRC_BF16, vrc.VRC_FP16, vrc.VRC_FP32, vrc.VRC_INT32])
def test_realigned_only_where_outputs_differ_modulo_128(dtype):
    """Outputs 128 bytes apart modulo 256 share the 128-byte grid (no
    realignment); one output 64 bytes off is enough to realign; at 8
    ranks x 2 MiB (below 64 MiB moved) the launch-bound 256-lane kernel
    runs whatever the offsets."""
    n, esz = 8, ESZ[dtype]
    count = (512 << 20) // esz
    send, recv = wide(n)
    shared = [a + 128 * (r % 2) for r, a in enumerate(recv)]
    assert launches(vrc.plan(vrc.COLL_ALLREDUCE, send, shared, count, 1, dtype, vrc.VRC_FUSED)[0])[0][0] == \
        "fused_allreduce_phased"  # one grid: no realignment (and large enough to run in phases)
    one_off = list(recv)
    one_off[3] += 64
    assert launches(vrc.plan(vrc.COLL_ALLREDUCE, send, one_off, count, 1, dtype, vrc.VRC_FUSED)[0])[0][0] == \
        "fused_allreduce_realigned"
    small = (2 << 20) // esz
    got = launches(vrc.plan(vrc.COLL_ALLREDUCE, send, one_off, small, 1, dtype, vrc.VRC_FUSED)[0])
    assert got[0][0] == "fused_allreduce" and got[0][3] == 256


def test_headline_shape():
    """8 ranks x 512 MiB bf16: the phased kernel, one 256-lane workgroup per
    CU, 96 sums per lane per phase (5 phases)."""
    assert plan_ar(8, 268435456, vrc.VRC_BF16, vrc.VRC_FUSED) == [("fused_allreduce_phased", 256, 1, 256, 96)]


def phased_k(n, dtype=vrc.VRC_BF16, butterfly=False):
    """Sums per lane per phase: 64 in registers up to 8 ranks, 32 above (16-bit
    butterfly: 32 and 16), plus 32 in LDS."""
    narrow = butterfly and ESZ[dtype] == 2
    regs = (32 if n <= 8 else 16) if narrow else (64 if n <= 8 else 32)
    return regs + 32


@pytest.mark.parametrize("n", list(range(2, 17)))
def test_phased_from_six_ranks_and_three_phases(n):
    """8 GiB moved, every output on one 128-byte grid: the phased kernel from
    6 ranks (there a phase reads 576 MiB or more), the one-wave kernel below."""
    count = (4 << 30) // n // 2 // 64 * 64
    got = plan_ar(n, count, vrc.VRC_BF16, vrc.VRC_FUSED)
    if n >= 6:
        assert got == [("fused_allreduce_phased", CUS, 1, 256, phased_k(n))]
    else:
        assert got[0][0] == "fused_allreduce" and got[0][3] == 64
    if n in (8, 16):
        for dtype in (vrc.VRC_BF16, vrc.VRC_FP32):
            assert plan_ar(n, count * 2 // ESZ[dtype], dtype, vrc.VRC_HD_ORDER) == [
                ("butterfly_allreduce_phased", CUS, 1, 256, phased_k(n, dtype, butterfly=True))]


def phased_skew(n, dtype=vrc.VRC_BF16, butterfly=False):
    """LDS sums fewer per lane in the odd workgroups: 16 at 8 ranks (96 sums
    per lane), 8 elsewhere."""
    narrow = butterfly and ESZ[dtype] == 2
    return 16 if n == 8 and not narrow else 8


def phased_vectors(n, skew):
    """16-byte vectors per rank in one phase: every lane's first K - skew
    slots, then the even workgroups' last `skew` slots."""
    return CUS * 256 * (phased_k(n) - skew) + CUS * 128 * skew


@pytest.mark.parametrize("n", [6, 8, 16])
def test_phased_needs_three_whole_phases(n):
    """Exactly three phases' vectors per rank take the phased kernel; one
    vector less keeps the one-wave kernel."""
    at = 3 * phased_vectors(n, phased_skew(n)) * 8  # bf16 elements
    assert plan_ar(n, at, vrc.VRC_BF16, vrc.VRC_FUSED)[0][0] == "fused_allreduce_phased"
    assert plan_ar(n, at - 8, vrc.VRC_BF16, vrc.VRC_FUSED)[0][0] == "fused_allreduce"


def test_phase_skew_off_restores_whole_slots():
    """VRC_PHASE_SKEW=0 (read once per process, so a child process checks it):
    every workgroup holds all K sums, so three phases need three times
    256 x 256 x K vectors per rank."""
    code = (
        "import sys, ring_all_reduce_virtual_amd as v\n"
        "n=int(sys.argv[1]); at=int(sys.argv[2])\n"
        "s=[(1<<40)+r*(1<<33) for r in range(n)]; d=[(1<<42)+r*(1<<33) for r in range(n)]\n"
        "a,_=v.plan(v.COLL_ALLREDUCE,s,d,at,1,v.VRC_BF16,v.VRC_FUSED)\n"
        "b,_=v.plan(v.COLL_ALLREDUCE,s,d,at-8,1,v.VRC_BF16,v.VRC_FUSED)\n"
        "print(a[0]['kind'],b[0]['kind'])\n")
    env = dict(os.environ, VRC_PHASE_SKEW="0", PYTHONPATH=ROOT)
    for n in (6, 8):
        at = 3 * phased_vectors(n, 0) * 8
        out = subprocess.run([sys.executable, "-c", code, str(n), str(at)], env=env, check=True,
                             capture_output=True, text=True, cwd=ROOT).stdout.split()
        assert out == ["fused_allreduce_phased", "fused_allreduce"], (n, out)


def test_phased_in_place_and_with_a_ragged_tail():
    """In place (every output its input, one grid) and with a count that
    leaves a partial phase, a partial vector and an unaligned head, the
    phased kernel still runs: its lanes write only what they read."""
    n = 8
    count = 268435456 + 12345
    bufs = [(1 << 40) + r * (1 << 32) + 6 for r in range(n)]
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, bufs, bufs, count, 1, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert launches(ops) == [("fused_allreduce_phased", CUS, 1, 256, 96)]


def test_fused_allreduce_launch_bound_shape_below_64_mib():
    """Exactly 64 MiB moved takes the one-wave shape; one vector less keeps
    256-lane workgroups, 8 per CU, two vectors per rank."""
    n, esz = 8, 2
    at = (64 << 20) // (2 * n * esz)
    assert plan_ar(n, at, vrc.VRC_BF16, vrc.VRC_FUSED) == [("fused_allreduce", 1024, 1, 64, 1)]
    below = at - 8
    nv = below * esz // 16
    assert plan_ar(n, below, vrc.VRC_BF16, vrc.VRC_FUSED) == [
        ("fused_allreduce", min((nv + 255) // 256, CUS * 8), 1, 256, 2)]
    small = plan_ar(n, 524288, vrc.VRC_FP16, vrc.VRC_FUSED)  # 8 x 1 MiB fp16
    assert small == [("fused_allreduce", 524288 * 2 // 16 // 256, 1, 256, 2)]


@pytest.mark.parametrize("n,per_cu_order", [(2, 8), (3, 4), (8, 4), (16, 4)])
def test_single_launch_ring_one_wave(n, per_cu_order):
    """2 GiB moved (under three phases of the phased ring-order kernel): ring
    order on one-wave workgroups, 4 per CU (8 at 2 ranks); the
    memory-faithful chain: 16 per CU."""
    count = (1 << 30) // n // 2 // 64 * 64
    assert plan_ar(n, count, vrc.VRC_BF16, vrc.VRC_RING_ORDER) == [
        ("ring_order_allreduce", CUS * per_cu_order, 1, 64, 1)]
    assert plan_ar(n, count, vrc.VRC_BF16, vrc.VRC_RING_CHAINED) == [("chain_allreduce", CUS * 16, 1, 64, 1)]


RING_ORDER_REGS = {  # sums per lane in registers of the phased ring-order kernel, by element type
    vrc.VRC_BF16: lambda n: 32 if n <= 7 else 24 if n <= 9 else 16 if n <= 14 else 0,
    vrc.VRC_FP16: lambda n: 40 if n <= 8 else 32 if n <= 11 else 24 if n <= 15 else 16,
    vrc.VRC_FP32: lambda n: 40,
    vrc.VRC_INT32: lambda n: 40,
}


@pytest.mark.parametrize("dtype", [vrc.VRC_BF16, vrc.VRC_FP16, vrc.VRC_FP32, vrc.VRC_INT32])
@pytest.mark.parametrize("n", list(range(2, 17)))
def test_ring_order_phased_from_six_ranks(n, dtype):
    """8 GiB moved, one output grid: the phased ring-order kernel from 6
    ranks (one 256-lane workgroup per CU, the table's register sums plus 40 in
    LDS per lane), the one-wave kernel below."""
    count = (4 << 30) // n // ESZ[dtype] // 64 * 64
    got = plan_ar(n, count, dtype, vrc.VRC_RING_ORDER)
    if n >= 6:
        assert got == [("ring_order_allreduce_phased", CUS, 1, 256, RING_ORDER_REGS[dtype](n) + 40)]
    else:
        assert got[0][0] == "ring_order_allreduce"


@pytest.mark.parametrize("n", [6, 8, 16])
def test_ring_order_phased_needs_three_whole_phases(n):
    """Phases count tiles (a chunk's last tile may be partial): exactly three
    phases' tiles take the phased kernel, one tile fewer does not.  A phase
    holds K tiles per wave, less 8 in the odd workgroups."""
    k, skew = RING_ORDER_REGS[vrc.VRC_BF16](n) + 40, 8
    tiles = 3 * (CUS * 4 * (k - skew) + CUS * 2 * skew)
    per_chunk = -(-tiles // n)  # whole tiles of 512 bf16 elements in every chunk
    count = per_chunk * n * 512
    assert plan_ar(n, count, vrc.VRC_BF16, vrc.VRC_RING_ORDER)[0][0] == "ring_order_allreduce_phased"
    fewer = (tiles - 1) // n * n * 512  # whole tiles below three phases
    assert plan_ar(n, fewer, vrc.VRC_BF16, vrc.VRC_RING_ORDER)[0][0] == "ring_order_allreduce"


def test_single_launch_ring_small_grid_covers_every_chunk():
    """4 x 4,099 int32: the grid is sized to the tiles (one per wave) and
    never below one wave per chunk for the scalar pass."""
    got = plan_ar(4, 4099, vrc.VRC_INT32, vrc.VRC_RING_ORDER)
    (kind, gx, gy, block, vectors), = got
    assert (kind, gy, block, vectors) == ("ring_order_allreduce", 1, 64, 1)
    tiles = sum((ln * 4 // 16 + 63) // 64 for ln in (1024, 1024, 1024, 1027))
    assert gx == max(tiles, 4)


@pytest.mark.parametrize("n,count,per_cu", [
    (8, 5 * 4096 * 128, 32),   # the heads: 320 MiB written, one store in flight per wave, 32 per CU
    (16, 5 << 19, 32),         # 16 x 5 MiB: 1.25 GiB written
    (8, 16 << 20, 32),         # 8 x 32 MiB: exactly 2 GiB written
    (8, (16 << 20) + 8, 16),   # just above 2 GiB written: stores back to back, 16 per CU
    (8, 64 << 20, 16),         # 8 x 128 MiB
])
def test_fused_all_gather_grid(n, count, per_cu):
    """fp16 all-gathers: 256-lane workgroups over the n source rows, 32 per
    CU up to 2 GiB written and 16 above."""
    esz = 2
    send, _ = wide(n)
    recv = gather_out(n, count, esz)
    ops, nl = vrc.plan(vrc.COLL_ALL_GATHER, send, recv, count, 1, vrc.VRC_FP16, vrc.VRC_FUSED)
    nv = count * esz // 16
    assert nl == 1
    assert launches(ops) == [("fused_all_gather", min((nv + 255) // 256, CUS * per_cu // n), n, 256, 1)]


@pytest.mark.parametrize("n,count,dtype,add_shape,copy_shape", [
    # 8 operations of >= 128 MiB: two vectors, 8 per CU
    (8, 268435456, vrc.VRC_BF16, (8, 256, 2), (8, 256, 2)),
    # <= 7 operations of >= 48 MiB: adds one-wave, 8 per CU; copies 256 lanes, 4 per CU; one vector
    (4, 536870912, vrc.VRC_BF16, (8, 64, 1), (4, 256, 1)),
    (7, 153391689, vrc.VRC_FP32, (8, 64, 1), (4, 256, 1)),
    (2, 268435459, vrc.VRC_BF16, (8, 64, 1), (4, 256, 1)),
    # >= 12 operations: two vectors, 16 per CU
    (16, 134217728, vrc.VRC_BF16, (16, 256, 2), (16, 256, 2)),
])
def test_ring_step_shapes(n, count, dtype, add_shape, copy_shape):
    got = plan_ar(n, count, dtype, vrc.VRC_RING)
    assert len(got) == 2 * (n - 1)
    for kind, gx, gy, block, vec in got:
        assert kind in ("add", "copy")
        per_cu, want_block, want_vec = add_shape if kind == "add" else copy_shape
        assert (gx, gy, block, vec) == (CUS * per_cu // n, n, want_block, want_vec), kind


def test_ring_reduce_scatter_adds_on_other_offsets_run_one_wave():
    """5 x 819 MiB bf16 reduce-scatter: chunk offsets of 171,756,748 bytes put
    chunks 1-3 of the inputs on other offsets than the outputs.  Those
    operations still move 16-byte vectors (unaligned loads), so their adds take
    the same one-wave shape as a count whose chunks are whole vectors."""
    n = 5
    send, recv = wide(n)
    for count in (5 * 85878374, 5 * 85878368):
        ops, _ = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, count, 1, vrc.VRC_BF16, vrc.VRC_RING)
        got = launches(ops)
        assert len(got) == n - 1
        for kind, gx, gy, b, vec in got:
            assert (kind, gx, gy, b, vec) == ("add", CUS * 8 // n, n, 64, 1)


def test_halving_doubling_steps_take_the_step_shapes():
    """4 x 1 GiB bf16: the halving adds (4 operations of >= 48 MiB) run
    one-wave workgroups, the doubling copies 256 lanes."""
    got = plan_ar(4, 536870912, vrc.VRC_BF16, vrc.VRC_HD)
    assert [k for k, *_ in got] == ["add", "add", "copy", "copy"]
    for kind, gx, gy, block, vec in got:
        assert (gy, block, vec) == ((4, 64, 1) if kind == "add" else (4, 256, 1))


def test_ring_steps_launch_bound_below_64_mib():
    """4 x 4,099 int32: every step is launch-bound, one vector per lane."""
    for kind, gx, gy, block, vec in plan_ar(4, 4099, vrc.VRC_INT32, vrc.VRC_RING):
        assert (gy, block, vec) == (4, 256, 1)
        assert 1 <= gx <= CUS * 8 // 4


def test_environment_overrides_reach_the_plan():
    """VRC_PHASED=0 keeps large fused all-reduces on the grid-stride kernels,
    whose shape VRC_FUSED_BLOCK / VRC_FUSED_BLOCKS_PER_CU / VRC_UNROLL set;
    VRC_CHAIN_BLOCK / VRC_CHAIN_BLOCKS_PER_CU and VRC_STEP_BLOCK replace the
    policy (read once per process, so a child process checks them)."""
    code = (
        "import ring_all_reduce_virtual_amd as v\n"
        "s=[(1<<40)+r*(1<<32) for r in range(8)]; d=[(1<<42)+r*(1<<32) for r in range(8)]\n"
        "f,_=v.plan(v.COLL_ALLREDUCE,s,d,268435456,1,v.VRC_BF16,v.VRC_FUSED)\n"
        "c,_=v.plan(v.COLL_ALLREDUCE,s,d,268435456,1,v.VRC_BF16,v.VRC_RING_CHAINED)\n"
        "r,_=v.plan(v.COLL_ALLREDUCE,s[:4],d[:4],536870912,1,v.VRC_BF16,v.VRC_RING)\n"
        "print(f[0]['grid_x'],f[0]['block'],f[0]['vectors'],c[0]['grid_x'],c[0]['block'],r[0]['block'])\n")
    env = dict(os.environ, VRC_FUSED_BLOCK="256", VRC_FUSED_BLOCKS_PER_CU="1", VRC_UNROLL="2",
               VRC_CHAIN_BLOCK="256", VRC_CHAIN_BLOCKS_PER_CU="4", VRC_STEP_BLOCK="256", VRC_PHASED="0",
               PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, check=True, capture_output=True, text=True,
                         cwd=ROOT).stdout.split()
    assert list(map(int, out)) == [256, 256, 2, 1024, 256, 256]


@pytest.mark.parametrize("n", [2, 3, 4, 8, 9, 16])
def test_fused_reduce_scatter_flat_shape(n):
    """Flat chunks from 64 MiB moved: one-wave workgroups over all chunks,
    8 per CU up to 4 ranks and 4 above (the butterfly fold of the
    halving-doubling reduce-scatter, which takes the same shape, turns
    ALU-bound with fewer)."""
    count = (4 << 30) // n // 2 // n // 64 * 64 * n  # whole 16-byte vectors in every chunk
    send, recv = wide(n)
    bpc = 8 if n <= 4 else 4
    ops, nl = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, count, 1, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert nl == 1 and launches(ops) == [("fused_reduce_scatter", CUS * bpc, 1, 64, 1)]
    ops, _ = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, count, 1, vrc.VRC_BF16, vrc.VRC_RING_ORDER)
    assert launches(ops) == [("ring_order_reduce_scatter", CUS * bpc, 1, 64, 1)]
    ops, _ = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, count, 1, vrc.VRC_BF16, vrc.VRC_RING_CHAINED)
    assert launches(ops) == [("chain_reduce_scatter", CUS * 16, 1, 64, 1)]
    if n & (n - 1) == 0:
        # at 2 ranks the butterfly is one add rounded once: the rank-fold kernel runs
        kind = "fused_reduce_scatter" if n == 2 else "butterfly_reduce_scatter"
        for mode in (vrc.VRC_HD_ORDER, vrc.VRC_HD):
            ops, _ = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, count, 1, vrc.VRC_BF16, mode)
            assert launches(ops) == [(kind, CUS * bpc, 1, 64, 1)]


def test_ragged_flat_reduce_scatter_takes_the_flat_walk():
    """Chunk bytes that are not a multiple of 16 put the inputs' chunks on
    other offsets than the outputs; the chunks still vectorize, so the flat
    one-wave walk serves them like whole-vector chunks."""
    n = 8
    send, recv = wide(n)
    ragged = 268435456 + n * 3 + 5
    for mode, kind, per_cu in ((vrc.VRC_FUSED, "fused_reduce_scatter", 4),
                               (vrc.VRC_RING_ORDER, "ring_order_reduce_scatter", 4),
                               (vrc.VRC_RING_CHAINED, "chain_reduce_scatter", 16),
                               (vrc.VRC_HD_ORDER, "butterfly_reduce_scatter", 4)):
        ops, _ = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, ragged, 1, vrc.VRC_BF16, mode)
        assert launches(ops) == [(kind, CUS * per_cu, 1, 64, 1)]


def test_split_dimension_and_small_reduce_scatters_keep_the_chunk_grid():
    """Split dimensions and calls below 64 MiB moved keep one grid row per
    chunk with 256-lane workgroups."""
    n = 8
    send, recv = wide(n)
    ops, _ = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, 268435456, 8, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert launches(ops)[0][2:4] == (n, 256)
    ops, _ = vrc.plan(vrc.COLL_REDUCE_SCATTER, send, recv, 1 << 20, 1, vrc.VRC_BF16, vrc.VRC_FUSED)
    assert launches(ops)[0][2:4] == (n, 256)


@pytest.mark.parametrize("mode", sorted(vrc.REDUCE_MODES))
def test_mixed_offsets_keep_the_full_grid(mode):
    """8 x 512 MiB bf16 all-reduce with rank r's input and output 2r bytes
    past a 256-byte boundary: every mode plans the launches of the aligned
    call, each with at least one workgroup per CU (a region off its
    destination's grid still runs 16-byte vectors)."""
    n, count = 8, 268435456
    send, recv = wide(n)
    mixed_send = [a + 2 * r for r, a in enumerate(send)]
    mixed_recv = [a + 2 * r for r, a in enumerate(recv)]
    aligned, nl = vrc.plan(vrc.COLL_ALLREDUCE, send, recv, count, 1, vrc.VRC_BF16, vrc.MODES[mode])
    mixed, nl2 = vrc.plan(vrc.COLL_ALLREDUCE, mixed_send, mixed_recv, count, 1, vrc.VRC_BF16, vrc.MODES[mode])
    assert nl2 == nl
    if mode in ("fused", "hd_order", "ring_order"):
        # the realigned variants (tests above); the aligned fused and butterfly calls run in phases
        assert [k[0] for k in launches(mixed)] == [k[0].replace("_phased", "") + "_realigned"
                                                   for k in launches(aligned)]
    else:
        assert launches(mixed) == launches(aligned)
    for kind, gx, gy, block, vec in launches(mixed):
        assert gx * gy * block >= CUS * 64, kind


def phase_layout(g, kr, kl, skew, lanes_per_wg=256):
    """Vector index (within a phase) of every (workgroup, lane, slot) that the
    phased kernels' skewed layout assigns: slot k of lane j at k * L + j for
    the first K - skew slots, then the even workgroups' last `skew` slots,
    L / 2 lanes wide; the odd workgroups hold `skew` fewer LDS slots."""
    import numpy as np
    k = kr + kl
    L = g * lanes_per_wg
    b = np.arange(g)[:, None]
    t = np.arange(lanes_per_wg)[None, :]
    w, l = t // 64, t % 64
    lane = (w * g + b) * 64 + l                    # [g, lanes]
    lane_even = (w * (g // 2) + b // 2) * 64 + l
    shared = k - skew
    out = []
    for s in range(k):
        # every workgroup holds slot s below K - skew; above it only the even ones
        take = np.ones((g, 1), bool) if s < shared else (b % 2 == 0)
        v = s * L + lane if s < shared else shared * L + (s - shared) * (L // 2) + lane_even
        out.append(np.broadcast_to(v, (g, lanes_per_wg))[np.broadcast_to(take, (g, lanes_per_wg))])
    return np.concatenate(out), shared * L + skew * (L // 2)


@pytest.mark.parametrize("g", [8, 32, 256])
@pytest.mark.parametrize("kr,kl,skew", [(64, 32, 16), (32, 32, 8), (16, 32, 8), (24, 40, 8), (0, 40, 8),
                                        (64, 32, 0)])
def test_skewed_phase_layout_covers_every_vector_once(g, kr, kl, skew):
    """For grids of whole XCD rounds, the skewed layout hands every vector of
    a phase to exactly one (workgroup, lane, slot), and a phase holds
    (K - skew) * L + skew * L / 2 vectors."""
    import numpy as np
    v, per_phase = phase_layout(g, kr, kl, skew)
    assert v.size == per_phase
    assert np.array_equal(np.sort(v), np.arange(per_phase))
