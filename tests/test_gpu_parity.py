"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases span several 4 KiB lane tiles and a ragged tail and are compared
element by element with the oracle's full simulation.  The named workloads
run at full size in the launch configuration the benchmark times.  At 128 MiB
and 512 MiB per rank the oracle's full simulation would take minutes, so every
element of every rank is compared with the oracle's per-element forms (the
ring, halving-doubling and rank-fold closed forms, pinned against the
simulation on the CPU), computed on host threads; the fp64 tolerance gate
runs on every element as well.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import (assert_bitwise, equal_to_expected, host, oracle_every_element, ranks_identical,
                               tolerance_gate_torch)

pytestmark = pytest.mark.gpu

DTYPES = ("int32", "fp32", "fp16", "bf16")
MODES = ("ring", "fused", "ring_chained", "ring_order", "hd", "hd_order")
RING_FAMILY = ("ring", "ring_chained", "ring_order")  # all return the per-step ring's bits
HD_FAMILY = ("hd", "hd_order")  # halving-doubling: power-of-two rank counts only
AG_MODES = MODES + ("tree",)  # the binomial tree is an all-gather mode only


def pow2(n):
    return n & (n - 1) == 0


def want_ar(orc, hx, dtype, mode):
    if mode in RING_FAMILY:
        return orc.ring_allreduce(hx, dtype)
    if mode in HD_FAMILY:
        return orc.hd_allreduce(hx, dtype)
    return orc.fused_allreduce(hx, dtype)


def want_rs(orc, hx, dtype, mode, outer=1):
    if mode in RING_FAMILY:
        return orc.ring_reduce_scatter(hx, dtype, outer=outer)
    if mode in HD_FAMILY:
        return orc.hd_reduce_scatter(hx, dtype, outer=outer)
    return orc.fused_reduce_scatter(hx, dtype, outer=outer)


def rejects_non_pow2(vrc, fn, mode, n):
    """HD modes need a power-of-two rank count; anything else is an argument error."""
    if mode in HD_FAMILY and not pow2(n):
        with pytest.raises(vrc.VrcError) as e:
            fn()
        assert e.value.status == vrc.VRC_ERR_INVALID_ARG
        return True
    return False


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def vrc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_all_reduce_virtual_amd as m  # fails loudly if libvrc.so is missing
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


DEV = "cuda:0"


# ---------------------------------------------------------------------------
# all-reduce, small and ragged, every dtype and mode, full oracle comparison
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,count", [(2, 1), (2, 4099), (3, 5), (3, 100003), (4, 4099), (5, 3),
                                     (8, 7), (8, 65536 * 3 + 13), (16, 1), (16, 100003)])
def test_allreduce_small(vrc, orc, mode, dtype, n, count):
    say(f"allreduce {mode} {dtype} n={n} count={count}")
    xs = workloads.random_ranks(n, count, dtype, seed=100 + n * 7 + count % 97, device=DEV)
    if rejects_non_pow2(vrc, lambda: vrc.vrc_allreduce(xs, mode=mode), mode, n):
        return
    ys = vrc.vrc_allreduce(xs, mode=mode)
    torch.cuda.synchronize()
    hx = host(xs)
    want = want_ar(orc, hx, dtype, mode)
    for r, y in enumerate(host(ys)):
        assert_bitwise(y, want[r], f"{mode} {dtype} n={n} count={count} rank {r}")


# ---------------------------------------------------------------------------
# reduce-scatter and all-gather, flat and along a dimension
# ---------------------------------------------------------------------------
RS_CASES = [  # (n, shape, dim)
    (2, (9,), 0), (4, (4099,), 0), (8, (7,), 0), (3, (100003,), 0), (16, (65536 * 2 + 5,), 0),
    (8, (8, 4096), -1), (4, (3, 40), 1), (2, (5, 6, 14), 2), (8, (2, 3, 16, 8), 2), (16, (4, 16 * 33), -1),
    (4, (7, 12), -1),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,shape,dim", RS_CASES)
def test_reduce_scatter_small(vrc, orc, mode, dtype, n, shape, dim):
    say(f"reduce_scatter {mode} {dtype} n={n} shape={shape} dim={dim}")
    xs = workloads.random_ranks(n, shape, dtype, seed=200 + n + len(shape), device=DEV)
    if rejects_non_pow2(vrc, lambda: vrc.vrc_reduce_scatter(xs, dim=dim, mode=mode), mode, n):
        return
    ys = vrc.vrc_reduce_scatter(xs, dim=dim, mode=mode)
    torch.cuda.synchronize()
    outer = int(np.prod(shape[:dim % len(shape)])) if len(shape) > 1 else 1
    hx = host(xs)
    want = want_rs(orc, hx, dtype, mode, outer)
    for c, y in enumerate(host(ys)):
        assert_bitwise(y, want[c], f"rs {mode} {dtype} n={n} shape={shape} chunk {c}")


AG_CASES = [  # (n, shape, dim)
    (2, (9,), 0), (4, (4099,), 0), (8, (1,), 0), (3, (100003,), 0), (16, (4096 + 3,), 0),
    (8, (1, 5, 64, 128), 1), (4, (3, 7), 1), (2, (5, 6, 14), 2), (8, (2, 3, 16, 8), 2), (3, (4, 33), -1),
]


def want_ag(orc, hx, dtype, mode, outer=1):
    """The all-gather of the mode's own step-literal oracle (every algorithm
    gives the concatenation; each is checked against its own simulation)."""
    if mode in HD_FAMILY:
        return orc.hd_all_gather(hx, dtype, outer=outer)
    if mode == "tree":
        return orc.tree_all_gather(hx, dtype, outer=outer)
    return orc.ring_all_gather(hx, dtype, outer=outer)


@pytest.mark.parametrize("mode", AG_MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,shape,dim", AG_CASES)
def test_all_gather_small(vrc, orc, mode, dtype, n, shape, dim):
    say(f"all_gather {mode} {dtype} n={n} shape={shape} dim={dim}")
    xs = workloads.random_ranks(n, shape, dtype, seed=300 + n + len(shape), device=DEV)
    if rejects_non_pow2(vrc, lambda: vrc.vrc_all_gather(xs, dim=dim, mode=mode), mode, n):
        return
    ys = vrc.vrc_all_gather(xs, dim=dim, mode=mode)
    torch.cuda.synchronize()
    outer = int(np.prod(shape[:dim % len(shape)])) if len(shape) > 1 else 1
    want = want_ag(orc, host(xs), dtype, mode, outer)
    ref = torch.cat(xs, dim=dim)
    for r, y in enumerate(ys):
        assert tuple(y.shape) == tuple(ref.shape)
        assert_bitwise(workloads.to_numpy(y), want[r], f"ag {mode} {dtype} n={n} shape={shape} rank {r}")


# ---------------------------------------------------------------------------
# the named workloads at full size
# ---------------------------------------------------------------------------
def test_workload_allreduce_int32_n4_4099(vrc, orc):
    w = workloads.WORKLOADS["allreduce_int32_n4_4099"]
    xs = workloads.make_inputs(w, DEV)
    hx = host(xs)
    naive = np.sum([x.astype(np.int64) for x in hx], axis=0).astype(np.int32)
    for mode in MODES:
        say(f"{w.name} {mode}")
        ys = vrc.vrc_allreduce(xs, mode=mode)
        torch.cuda.synchronize()
        want = want_ar(orc, hx, "int32", mode)
        for r, y in enumerate(host(ys)):
            assert_bitwise(y, want[r], f"{w.name} {mode} rank {r}")
            assert_bitwise(y, naive, f"{w.name} {mode} rank {r} vs naive sum")


def test_workload_allreduce_fp32_n8_16mib(vrc, orc):
    w = workloads.WORKLOADS["allreduce_fp32_n8_16mib"]
    xs = workloads.make_inputs(w, DEV)
    hx = host(xs)
    want_ring = orc.ring_allreduce(hx, "fp32")
    for mode in MODES:
        say(f"{w.name} {mode}")
        ys = vrc.vrc_allreduce(xs, mode=mode)
        torch.cuda.synchronize()
        ranks_identical(ys, f"{w.name} {mode}")
        if mode in RING_FAMILY:
            want = want_ring
        else:
            want = want_ar(orc, hx, "fp32", mode)
            tolerance_gate_torch(ys, xs, w.rtol, f"{w.name} {mode}")
        for r, y in enumerate(host(ys)):
            assert_bitwise(y, want[r], f"{w.name} {mode} rank {r}")


@pytest.mark.parametrize("count", [524288, 8388608])
def test_workload_allreduce_fp16_sweep(vrc, orc, count):
    w = workloads.WORKLOADS["allreduce_fp16_n8_128mib"].with_count(count)
    xs = workloads.make_inputs(w, DEV)
    hx = host(xs)
    want_ring = orc.ring_allreduce(hx, "fp16")
    for mode in MODES:
        say(f"{w.name} {mode}")
        ys = vrc.vrc_allreduce(xs, mode=mode)
        torch.cuda.synchronize()
        tolerance_gate_torch(ys, xs, w.rtol, f"{w.name} {mode}")
        want = want_ring if mode in RING_FAMILY else want_ar(orc, hx, "fp16", mode)
        for r, y in enumerate(host(ys)):
            assert_bitwise(y, want[r], f"{w.name} {mode} rank {r}")


def gamma(k: int, dtype: str) -> float:
    """gamma_k = k u / (1 - k u), u the storage unit roundoff (2^-24 fp32,
    2^-11 fp16, 2^-8 bf16): the bound of a sum whose every partial is
    rounded to the storage type along a depth-k tree."""
    u = {"fp32": 2.0**-24, "fp16": 2.0**-11, "bf16": 2.0**-8}[dtype]
    return k * u / (1 - k * u)


def ring_bound(n: int, dtype: str) -> float:
    """The ring's sequential sum: depth n-1."""
    return gamma(n - 1, dtype)


def gate_rtol(w, mode: str) -> float:
    """The workload's tolerance for its gated modes.  bf16 in the ring or
    halving-doubling family is not a gated mode of any workload: 7 (ring) or
    3 (halving-doubling) roundings to an 8-bit significand can exceed 1e-2,
    so it is held to its own derived bound instead."""
    if w.dtype == "bf16" and mode in RING_FAMILY:
        return ring_bound(w.n, "bf16")
    if w.dtype == "bf16" and mode in HD_FAMILY:
        return gamma(w.n.bit_length() - 1, "bf16")
    return w.rtol


def _full_allreduce(vrc, orc, w, modes):
    """Every mode on the full workload: every element of every rank bit for
    bit against the oracle's per-element form of the mode's algorithm (one
    expected array per algorithm family), plus the tolerance gate."""
    xs = workloads.make_inputs(w, DEV)
    hx = host(xs)
    families = {}
    for mode in modes:
        fam = "ring" if mode in RING_FAMILY else "hd" if mode in HD_FAMILY else "fused"
        families.setdefault(fam, []).append(mode)
    for fam, fam_modes in families.items():
        at = {"ring": orc.ring_allreduce_at, "hd": orc.hd_allreduce_at, "fused": orc.fused_allreduce_at}[fam]
        say(f"{w.name}: oracle {fam} form on all {w.count} elements")
        want = torch.from_numpy(oracle_every_element(at, hx, w.dtype, w.count)).to(DEV)
        for mode in fam_modes:
            say(f"{w.name} {mode}: every element of every rank")
            ys = vrc.vrc_allreduce(xs, mode=mode)
            torch.cuda.synchronize()
            equal_to_expected(ys, want, f"{w.name} {mode}")
            tolerance_gate_torch(ys, xs, gate_rtol(w, mode), f"{w.name} {mode}")
            del ys
            torch.cuda.empty_cache()
        del want


def test_workload_allreduce_fp16_n8_128mib(vrc, orc):
    w = workloads.WORKLOADS["allreduce_fp16_n8_128mib"]
    _full_allreduce(vrc, orc, w, MODES)


@pytest.mark.parametrize("family", ["fused", "ring", "hd"])
def test_workload_allreduce_bf16_n8_512mib(vrc, orc, family):
    # fused is the headline mode; the ring and halving-doubling families run too (not gated by the workload)
    w = workloads.WORKLOADS["allreduce_bf16_n8_512mib"]
    modes = {"fused": ("fused",), "ring": RING_FAMILY, "hd": HD_FAMILY}[family]
    _full_allreduce(vrc, orc, w, modes)


def test_workload_all_gather_fp16_n8_heads(vrc, orc):
    w = workloads.WORKLOADS["all_gather_fp16_n8_heads"]
    xs = workloads.make_inputs(w, DEV)
    want = orc.ring_all_gather(host(xs), "fp16", outer=1)
    assert all(np.array_equal(a, b) for a, b in zip(want, orc.hd_all_gather(host(xs), "fp16", outer=1)))
    assert all(np.array_equal(a, b) for a, b in zip(want, orc.tree_all_gather(host(xs), "fp16", outer=1)))
    for mode in AG_MODES:
        say(f"{w.name} {mode}")
        ys = vrc.vrc_all_gather(xs, dim=w.dim, mode=mode)
        torch.cuda.synchronize()
        assert tuple(ys[0].shape) == (1, 40, 4096, 128)
        ranks_identical(ys, f"{w.name} {mode}")
        for r, y in enumerate(ys):
            assert_bitwise(workloads.to_numpy(y), want[r], f"{w.name} {mode} rank {r}")


def test_workload_reduce_scatter_fp16_n8_act(vrc, orc):
    w = workloads.WORKLOADS["reduce_scatter_fp16_n8_act"]
    xs = workloads.make_inputs(w, DEV)
    hx = host(xs)
    for mode in MODES:
        say(f"{w.name} {mode}")
        ys = vrc.vrc_reduce_scatter(xs, dim=w.dim, mode=mode)
        torch.cuda.synchronize()
        assert tuple(ys[0].shape) == (8, 512)
        want = want_rs(orc, hx, "fp16", mode, outer=8)
        for c, y in enumerate(host(ys)):
            assert_bitwise(y, want[c], f"{w.name} {mode} chunk {c}")
        # tolerance gate against the fp64 sum of each column block
        for c in range(w.n):
            blocks = [x[:, c * 512:(c + 1) * 512].contiguous() for x in xs]
            tolerance_gate_torch([ys[c]], blocks, w.rtol, f"{w.name} {mode} chunk {c}")


# ---------------------------------------------------------------------------
# every step launch shape (vectors per lane, workgroups per CU), ragged sizes
# ---------------------------------------------------------------------------
SHAPE_CASES = [  # (n, count, dtype, modes): the shape each case's large steps take
    (3, 50_331_653, "fp16", ("ring",)),               # <= 7 operations of >= 48 MiB: one vector; adds one-wave
    (7, 8_388_613, "fp32", ("ring",)),                # <= 7 small operations: two vectors, 16 per CU
    (9, 104_857_601, "fp32", ("ring",)),              # 8-11 operations of >= 128 MiB: two vectors, 8 per CU
    (16, 16_777_219, "fp16", ("ring", "hd")),         # >= 12 operations: two vectors, 16 per CU
    (2, 268_435_459, "bf16", ("ring", "hd")),         # 2 operations of 768 MiB: one vector; adds one-wave
    (5, 41_943_047, "fp32", ("ring",)),               # 5 adds of 96 MiB, one-wave; ragged last chunk
]


@pytest.mark.parametrize("n,count,dtype,modes", SHAPE_CASES)
def test_step_launch_shapes(vrc, orc, n, count, dtype, modes):
    say(f"step shapes n={n} count={count} {dtype} {modes}")
    xs = workloads.random_ranks(n, count, dtype, seed=500 + n, device=DEV)
    hx = host(xs)
    for mode in modes:
        ys = vrc.vrc_allreduce(xs, mode=mode)
        torch.cuda.synchronize()
        at = orc.ring_allreduce_at if mode in RING_FAMILY else orc.hd_allreduce_at
        want = torch.from_numpy(oracle_every_element(at, hx, dtype, count)).to(DEV)
        equal_to_expected(ys, want, f"{mode} {dtype} n={n} count={count}")
        del ys, want
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# fused all-reduce launch shapes: from 64 MiB moved the workgroup count and
# the vectors each lane keeps in flight depend on the rank count; every rank
# count 2..16 at a ragged size above that limit, on misaligned views too
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", list(range(2, 17)))
def test_fused_launch_shapes(vrc, orc, n):
    dtype = ("fp32", "bf16", "fp16", "int32")[n % 4]
    esz = 2 if dtype in ("fp16", "bf16") else 4
    count = (64 << 20) // (2 * n * esz) + 4099  # just above 64 MiB moved, not a whole number of vectors
    say(f"fused shapes n={n} count={count} {dtype}")
    base = workloads.random_ranks(n, count + 1, dtype, seed=700 + n, device=DEV, sigma=1e-2)
    modes = ("fused", "hd_order") if pow2(n) else ("fused",)
    # offset 1: every buffer starts one element past a 16-byte boundary; "mixed": rank r's output r
    # elements into its own buffer, so the outputs do not share one vector grid (its own launch shape)
    for offset in (0, 1, "mixed"):
        xs = [b[1:1 + count] if offset == "mixed" else b[offset:offset + count] for b in base]
        hx = host(xs)
        for mode in modes:
            if offset == "mixed":
                ys = [torch.empty(count + 16, dtype=xs[0].dtype, device=DEV)[r % 16:r % 16 + count] for r in range(n)]
                vrc.vrc_allreduce(xs, recv=ys, mode=mode)
            else:
                ys = vrc.vrc_allreduce(xs, mode=mode)
            torch.cuda.synchronize()
            ranks_identical(ys, f"{mode} n={n} offset={offset}")
            want = want_ar(orc, hx, dtype, mode)
            for r in (0, n - 1):
                assert_bitwise(workloads.to_numpy(ys[r]), want[r], f"{mode} {dtype} n={n} offset={offset} rank {r}")
            del ys


# ---------------------------------------------------------------------------
# fused and single-launch ring reduce-scatter over flat chunks from 64 MiB moved:
# one-wave tiles over all chunks, whatever the offsets of inputs and outputs
# ---------------------------------------------------------------------------
RS_FLAT_LAYOUTS = {
    "aligned": (0, 0),         # inputs and outputs on 16-byte boundaries: vector body, ragged tail
    "both_offset": (1, 1),     # inputs and outputs one element past a boundary: scalar heads
    "inputs_offset": (1, 0),   # inputs off the outputs' grid: unaligned vector loads
}


@pytest.mark.parametrize("layout", list(RS_FLAT_LAYOUTS))
@pytest.mark.parametrize("n", [2, 3, 4, 5, 7, 8, 11, 16])
def test_fused_reduce_scatter_flat_shapes(vrc, orc, n, layout):
    dtype = ("fp32", "bf16", "fp16", "int32")[n % 4]
    esz = 2 if dtype in ("fp16", "bf16") else 4
    vec = 16 // esz
    base = ((64 << 20) // ((n + 1) * n * esz) // vec + 1) * vec  # chunk bytes a multiple of 16
    count = n * base + n - 1  # the last chunk takes the remainder and ends in a scalar tail
    in_off, out_off = RS_FLAT_LAYOUTS[layout]
    say(f"fused rs flat n={n} count={count} {dtype} {layout}")
    src = workloads.random_ranks(n, count + 1, dtype, seed=900 + n, device=DEV, sigma=1e-2)
    xs = [t[in_off:in_off + count] for t in src]
    lens = [base] * (n - 1) + [count - (n - 1) * base]
    hx = host(xs)
    modes = ("fused", "ring_order", "ring_chained", "hd_order", "hd") if pow2(n) else ("fused", "ring_order",
                                                                                       "ring_chained")
    for mode in modes:
        outs = [torch.empty(ln + 1, dtype=xs[0].dtype, device=DEV) for ln in lens]
        ys = [o[out_off:out_off + ln] for o, ln in zip(outs, lens)]
        vrc.vrc_reduce_scatter(xs, recv=ys, mode=mode)
        torch.cuda.synchronize()
        want = want_rs(orc, hx, dtype, mode)
        for c, y in enumerate(host(ys)):
            assert_bitwise(y, want[c], f"rs {mode} {dtype} n={n} {layout} chunk {c}")
        del outs, ys
