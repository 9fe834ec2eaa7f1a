"""Edge cases of the HIP path through the C ABI: in place, misaligned views,
degenerate rank counts and sizes, determinism, composition, streams and the
error paths with real device buffers."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import assert_bitwise, equal_to_expected, host, oracle_every_element

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DTYPES = ("int32", "fp32", "fp16", "bf16")
MODES = ("ring", "fused", "ring_chained", "ring_order", "hd", "hd_order")
RING_FAMILY = ("ring", "ring_chained", "ring_order")
HD_FAMILY = ("hd", "hd_order")


def runs(mode, n):
    """Halving-doubling needs a power-of-two rank count."""
    return mode not in HD_FAMILY or n & (n - 1) == 0


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def vrc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_all_reduce_virtual_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def oracle_ar(orc, hx, dtype, mode):
    if mode in RING_FAMILY:
        return orc.ring_allreduce(hx, dtype)
    if mode in HD_FAMILY:
        return orc.hd_allreduce(hx, dtype)
    return orc.fused_allreduce(hx, dtype)


def oracle_rs(orc, hx, dtype, mode, outer=1):
    if mode in RING_FAMILY:
        return orc.ring_reduce_scatter(hx, dtype, outer=outer)
    if mode in HD_FAMILY:
        return orc.hd_reduce_scatter(hx, dtype, outer=outer)
    return orc.fused_reduce_scatter(hx, dtype, outer=outer)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
def test_in_place_equals_out_of_place(vrc, orc, mode, dtype):
    say(f"in place {mode} {dtype}")
    n, count = 8, 50001
    xs = workloads.random_ranks(n, count, dtype, seed=400, device=DEV)
    want = oracle_ar(orc, host(xs), dtype, mode)
    ys = vrc.vrc_allreduce(xs, recv=xs, mode=mode)  # recv is send
    torch.cuda.synchronize()
    for r in range(n):
        assert_bitwise(workloads.to_numpy(ys[r]), want[r], f"in place {mode} {dtype} rank {r}")


@pytest.mark.parametrize("mode", MODES)
def test_some_ranks_in_place(vrc, orc, mode):
    say(f"mixed in place {mode}")
    n, count = (5 if runs(mode, 5) else 4), 40000
    xs = workloads.random_ranks(n, count, "fp32", seed=401, device=DEV)
    want = oracle_ar(orc, host(xs), "fp32", mode)
    recv = [xs[r] if r % 2 == 0 else torch.empty_like(xs[r]) for r in range(n)]
    vrc.vrc_allreduce(xs, recv=recv, mode=mode)
    torch.cuda.synchronize()
    for r in range(n):
        assert_bitwise(workloads.to_numpy(recv[r]), want[r], f"mixed {mode} rank {r}")


def _views(xs, offsets, count):
    """Contiguous views of `count` elements starting `offsets[r]` elements
    into a fresh buffer (so data pointers are misaligned by design)."""
    out = []
    for x, off in zip(xs, offsets):
        buf = torch.empty(count + 16, dtype=x.dtype, device=x.device)
        v = buf[off:off + count]
        v.copy_(x)
        out.append(v)
    return out


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("offsets", ["same", "mixed"])
def test_misaligned_views(vrc, orc, mode, dtype, offsets):
    say(f"misaligned {offsets} {mode} {dtype}")
    n, count = 4, 30011
    xs = workloads.random_ranks(n, count, dtype, seed=402, device=DEV)
    offs_in = [1] * n if offsets == "same" else [0, 1, 3, 5]
    offs_out = [1] * n if offsets == "same" else [2, 0, 1, 7]
    vx = _views(xs, offs_in, count)
    vy = _views([torch.zeros_like(x) for x in xs], offs_out, count)
    vrc.vrc_allreduce(vx, recv=vy, mode=mode)
    want = oracle_ar(orc, host(xs), dtype, mode)
    torch.cuda.synchronize()
    for r in range(n):
        assert_bitwise(workloads.to_numpy(vy[r]), want[r], f"misaligned {mode} {dtype} rank {r}")
    # reduce-scatter and all-gather through misaligned views too
    rs = vrc.vrc_reduce_scatter(vx, mode=mode)
    want_rs = oracle_rs(orc, host(xs), dtype, mode)
    ag = vrc.vrc_all_gather(vx, mode=mode)
    want_ag = orc.ring_all_gather(host(xs), dtype)
    torch.cuda.synchronize()
    for c in range(n):
        assert_bitwise(workloads.to_numpy(rs[c]), want_rs[c], f"misaligned rs {mode} {dtype} chunk {c}")
        assert_bitwise(workloads.to_numpy(ag[c]), want_ag[c], f"misaligned ag {mode} {dtype} rank {c}")


@pytest.mark.parametrize("mode", MODES)
def test_large_allreduce_on_mixed_offsets(vrc, orc, mode):
    """8 ranks x (6 Mi + 5) bf16, about 96 MiB moved (the launch shapes of
    large calls): rank r's input starts r elements and its output (3r mod 8)
    elements into a fresh buffer, so no two operands share an offset.  Every
    element of every rank against the oracle's per-element form."""
    n, count = 8, 6 * (1 << 20) + 5
    say(f"large mixed offsets {mode}: n={n} count={count}")
    xs = workloads.random_ranks(n, count, "bf16", seed=4101, device=DEV, sigma=1e-2)
    vx = _views(xs, list(range(n)), count)
    vy = _views([torch.zeros_like(x) for x in xs], [3 * r % 8 for r in range(n)], count)
    vrc.vrc_allreduce(vx, recv=vy, mode=mode)
    torch.cuda.synchronize()
    at = {"ring": orc.ring_allreduce_at, "hd": orc.hd_allreduce_at, "fused": orc.fused_allreduce_at}[
        "ring" if mode in RING_FAMILY else "hd" if mode in HD_FAMILY else "fused"]
    want = torch.from_numpy(oracle_every_element(at, host(xs), "bf16", count)).to(DEV)
    equal_to_expected(vy, want, f"large mixed offsets {mode}")


@pytest.mark.parametrize("n,dtype,mode,count", [
    (2, "fp32", "fused", 4 * (1 << 20) + 37),
    (3, "fp16", "fused", 6 * (1 << 20) + 11),
    (4, "fp16", "hd_order", 4 * (1 << 20) + 1),
    (5, "int32", "fused", 2 * (1 << 20) + 3),
    (8, "bf16", "hd_order", 2 * (1 << 20) + 77),
    (8, "bf16", "fused", 2 * (1 << 20) + 4096 + 13),
    (13, "fp32", "fused", (1 << 20) + 5),
    (16, "bf16", "fused", (1 << 20) + 9),
    (16, "fp32", "hd_order", (1 << 19) + 1),
    (3, "int32", "ring_order", 3 * (1 << 20) + 7),
    (5, "fp16", "ring_order", 4 * (1 << 20) + 5),
    (8, "bf16", "ring_order", 2 * (1 << 20) + 77),
    (16, "fp32", "ring_order", (1 << 19) + 1)])
def test_realigned_fused_allreduce(vrc, orc, n, dtype, mode, count):
    """Outputs on n different offsets modulo 128 bytes (every byte shift the
    realigned stores funnel, 2-byte ones included; the ring order per chunk,
    with the chunk's own rank rotation), inputs on their own
    offsets, a count that leaves a partial group and a scalar tail, at least
    64 MiB moved so the realigned kernel runs (vrc_plan says which).  Every
    element of every output against the oracle."""
    esz = {"fp32": 4, "int32": 4, "fp16": 2, "bf16": 2}[dtype]
    per_line = 128 // esz
    in_off = [r % 3 for r in range(n)]
    out_off = [(19 * r + 5) % per_line for r in range(n)]
    say(f"realigned fused all-reduce {mode}: n={n} {dtype} count={count} out offsets {out_off}")
    xs = workloads.random_ranks(n, count, dtype, seed=4301 + n, device=DEV, sigma=1e-2)

    def views(src, offsets):
        out = []
        for x, off in zip(src, offsets):
            buf = torch.zeros(count + per_line, dtype=x.dtype, device=DEV)
            v = buf[off:off + count]
            v.copy_(x)
            out.append(v)
        return out

    vx = views(xs, in_off)
    vy = views([torch.zeros_like(x) for x in xs], out_off)
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, [v.data_ptr() for v in vx], [v.data_ptr() for v in vy], count, 1,
                      {"int32": vrc.VRC_INT32, "fp32": vrc.VRC_FP32, "fp16": vrc.VRC_FP16, "bf16": vrc.VRC_BF16}[dtype],
                      vrc.MODES[mode])
    want_kind = {"hd_order": "butterfly", "ring_order": "ring_order", "fused": "fused"}[mode] + "_allreduce_realigned"
    assert [o["kind"] for o in ops] == [want_kind]
    vrc.vrc_allreduce(vx, recv=vy, mode=mode)
    torch.cuda.synchronize()
    at = {"hd_order": orc.hd_allreduce_at, "ring_order": orc.ring_allreduce_at,
          "fused": orc.fused_allreduce_at}[mode]
    want = torch.from_numpy(oracle_every_element(at, host(xs), dtype, count)).to(DEV)
    equal_to_expected(vy, want, f"realigned {mode} n={n} {dtype}")


@pytest.mark.parametrize("mode,n", [("ring", 5), ("fused", 5), ("ring_chained", 5), ("ring_order", 5),
                                    ("hd", 8), ("hd_order", 8)])
def test_large_ragged_flat_reduce_scatter(vrc, orc, mode, n):
    """A flat bf16 reduce-scatter whose chunk bytes are odd multiples of 2
    (count = n * base + 3, base odd): chunk c of every input sits on another
    16-byte offset than output c.  Above 64 MiB moved, so the flat kernels
    run; every element of every chunk against the oracle's simulation."""
    base = 3 * (1 << 21) + 3
    count = n * base + 3
    say(f"large ragged reduce-scatter {mode}: n={n} count={count}")
    xs = workloads.random_ranks(n, count, "bf16", seed=4201 + n, device=DEV, sigma=1e-2)
    ys = vrc.vrc_reduce_scatter(xs, mode=mode)
    torch.cuda.synchronize()
    want = oracle_rs(orc, host(xs), "bf16", mode)
    for c, y in enumerate(ys):
        assert_bitwise(workloads.to_numpy(y), want[c], f"large ragged rs {mode} chunk {c}")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 9, 16])
@pytest.mark.parametrize("count", [0, 1, 3, 4099])
def test_tree_all_gather_edges(vrc, orc, n, count):
    """The binomial-tree all-gather at any rank count (powers of two or not),
    empty and tiny inputs, inputs and outputs on different element offsets."""
    say(f"tree all-gather n={n} count={count}")
    xs = workloads.random_ranks(n, count, "fp16", seed=430 + n, device=DEV)
    vx = _views(xs, [r % 5 for r in range(n)], count)
    vy = _views([torch.zeros(n * count, dtype=xs[0].dtype, device=DEV) for _ in range(n)],
                [(2 * r + 1) % 7 for r in range(n)], n * count)
    vrc.vrc_all_gather(vx, recv=vy, mode="tree")
    torch.cuda.synchronize()
    want = orc.tree_all_gather(host(xs), "fp16") if count else [np.zeros(0, np.float16)] * n
    for r in range(n):
        assert_bitwise(workloads.to_numpy(vy[r]), want[r], f"tree n={n} count={count} rank {r}")


def test_tree_refuses_the_reduce_collectives(vrc):
    xs = workloads.random_ranks(4, 64, "fp32", seed=431, device=DEV)
    for call in (lambda: vrc.vrc_allreduce(xs, mode="tree"), lambda: vrc.vrc_reduce_scatter(xs, mode="tree")):
        with pytest.raises(vrc.VrcError) as e:
            call()
        assert e.value.status == vrc.VRC_ERR_UNSUPPORTED


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
def test_single_rank_is_identity(vrc, mode, dtype):
    say(f"n=1 {mode} {dtype}")
    (x,) = workloads.random_ranks(1, 1234, dtype, seed=403, device=DEV)
    (y,) = vrc.vrc_allreduce([x], mode=mode)
    (z,) = vrc.vrc_reduce_scatter([x], mode=mode)
    (g,) = vrc.vrc_all_gather([x], mode=mode)
    (p,) = vrc.vrc_allreduce([x], recv=[x], mode=mode)
    torch.cuda.synchronize()
    hx = workloads.to_numpy(x)
    for t, what in ((y, "ar"), (z, "rs"), (g, "ag"), (p, "ar in place")):
        assert_bitwise(workloads.to_numpy(t), hx, f"n=1 {what} {mode} {dtype}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,count", [(8, 3), (16, 15), (4, 1), (3, 0)])
def test_fewer_elements_than_ranks(vrc, orc, mode, n, count):
    say(f"count<n {mode} n={n} count={count}")
    xs = workloads.random_ranks(n, count, "fp32", seed=404, device=DEV)
    if not runs(mode, n):  # halving-doubling needs a power-of-two rank count
        for call in (lambda: vrc.vrc_allreduce(xs, mode=mode), lambda: vrc.vrc_reduce_scatter(xs, mode=mode)):
            with pytest.raises(vrc.VrcError) as e:
                call()
            assert e.value.status == vrc.VRC_ERR_INVALID_ARG
        return
    ys = vrc.vrc_allreduce(xs, mode=mode)
    rs = vrc.vrc_reduce_scatter(xs, mode=mode)
    torch.cuda.synchronize()
    hx = host(xs)
    want = oracle_ar(orc, hx, "fp32", mode)
    want_rs = oracle_rs(orc, hx, "fp32", mode)
    for r in range(n):
        assert_bitwise(workloads.to_numpy(ys[r]), want[r], f"count<n {mode} rank {r}")
        assert_bitwise(workloads.to_numpy(rs[r]), want_rs[r], f"count<n rs {mode} chunk {r}")


@pytest.mark.parametrize("mode", MODES)
def test_repeat_runs_are_bitwise_identical(vrc, mode):
    say(f"determinism {mode}")
    xs = workloads.make_inputs(workloads.WORKLOADS["allreduce_fp32_n8_16mib"], DEV)
    outs = []
    for _ in range(3):
        ys = vrc.vrc_allreduce(xs, mode=mode)
        torch.cuda.synchronize()
        outs.append(torch.stack(ys).view(torch.int32))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("mode", RING_FAMILY + HD_FAMILY)
@pytest.mark.parametrize("dtype", DTYPES)
def test_all_gather_of_reduce_scatter_is_allreduce(vrc, dtype, mode):
    say(f"composition {dtype} {mode}")
    n, count = 8, 8 * 12345  # equal chunks
    xs = workloads.random_ranks(n, count, dtype, seed=405, device=DEV)
    ar = vrc.vrc_allreduce(xs, mode=mode)
    rs = vrc.vrc_reduce_scatter(xs, mode=mode)
    ag = vrc.vrc_all_gather(rs, mode=mode)
    torch.cuda.synchronize()
    for r in range(n):
        assert_bitwise(workloads.to_numpy(ag[r]), workloads.to_numpy(ar[r]), f"AG(RS) vs AR {dtype} rank {r}")


def test_exact_small_integers_ring_equals_fused(vrc):
    say("exact small integers")
    n, count = 8, 77777
    g = torch.Generator(device=DEV).manual_seed(406)
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        xs = [torch.randint(-15, 16, (count,), generator=g, device=DEV).to(dt) for _ in range(n)]
        a = vrc.vrc_allreduce(xs, mode="ring")
        b = vrc.vrc_allreduce(xs, mode="fused")
        s = torch.stack([x.double() for x in xs]).sum(0)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(a[r].double(), s) and torch.equal(b[r].double(), s)


def test_int32_wraps(vrc):
    say("int32 wrap")
    xs = [torch.full((1000,), 2**31 - 1, dtype=torch.int32, device=DEV) for _ in range(4)]
    for mode in MODES:
        ys = vrc.vrc_allreduce(xs, mode=mode)
        torch.cuda.synchronize()
        assert torch.all(ys[0] == -4)  # 4 * (2^31 - 1) = 2^33 - 4, which wraps to -4


def test_fp16_overflow_goes_to_inf(vrc, orc):
    say("fp16 overflow")
    xs = [torch.full((100,), 60000.0, dtype=torch.float16, device=DEV) for _ in range(2)]
    for mode in MODES:
        ys = vrc.vrc_allreduce(xs, mode=mode)
        torch.cuda.synchronize()
        assert torch.all(torch.isinf(ys[1])) and torch.all(ys[1] > 0)


def test_subnormals_are_kept(vrc, orc):
    say("subnormals")
    n = 4
    tiny32 = torch.tensor([1e-45, -3e-44, 1.2e-38, 5.9e-39] * 64, dtype=torch.float32, device=DEV)
    tiny16 = torch.tensor([6e-8, -1.2e-7, 3e-5, 6.1e-5] * 64, dtype=torch.float16, device=DEV)
    for x0, dtype in ((tiny32, "fp32"), (tiny16, "fp16"), (tiny32.to(torch.bfloat16), "bf16")):
        xs = [x0 * (r + 1) for r in range(n)]
        for mode in MODES:
            ys = vrc.vrc_allreduce(xs, mode=mode)
            torch.cuda.synchronize()
            want = oracle_ar(orc, host(xs), dtype, mode)
            assert_bitwise(workloads.to_numpy(ys[0]), want[0], f"subnormal {mode} {dtype}")
            assert torch.any(ys[0] != 0)


def test_side_stream(vrc, orc):
    say("side stream")
    xs = workloads.random_ranks(8, 300000, "bf16", seed=407, device=DEV)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = {m: vrc.vrc_allreduce(xs, mode=m) for m in MODES}
    s.synchronize()
    hx = host(xs)
    for m, ys in outs.items():
        assert_bitwise(workloads.to_numpy(ys[3]), oracle_ar(orc, hx, "bf16", m)[3], f"side stream {m}")


def test_binding_enqueues_on_the_current_stream(vrc):
    """The binding's stream lookup returns the handle of torch's current
    stream, on the default stream and inside a side-stream context, and an
    explicit stream wins."""
    say("binding stream lookup")
    dev = torch.cuda.current_device()
    assert vrc._stream(None, dev) == torch.cuda.current_stream().cuda_stream
    assert vrc._stream(None, torch.device(DEV)) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert vrc._stream(None, dev) == s.cuda_stream != torch.cuda.default_stream().cuda_stream
    assert vrc._stream(s, dev) == s.cuda_stream


def test_in_place_list_through_the_binding(vrc, orc):
    """recv given as the very list of inputs: the sums land in the inputs."""
    say("in place, same list")
    xs = workloads.random_ranks(8, 12345, "fp32", seed=409, device=DEV)
    hx = host(xs)
    ys = vrc.vrc_allreduce(xs, recv=xs, mode="fused")
    torch.cuda.synchronize()
    assert ys is xs
    assert_bitwise(workloads.to_numpy(xs[5]), oracle_ar(orc, hx, "fp32", "fused")[5], "in place, same list")


def test_errors_through_the_binding(vrc):
    say("errors")
    xs = workloads.random_ranks(4, 1000, "fp32", seed=408, device=DEV)
    with pytest.raises(vrc.VrcError) as e:
        vrc.vrc_allreduce(xs, recv=[xs[1], xs[0], xs[2], xs[3]])  # outputs are other ranks' inputs
    assert e.value.status == vrc.VRC_ERR_ALIAS
    with pytest.raises(vrc.VrcError) as e:
        vrc.vrc_reduce_scatter(xs, recv=[x[:250] for x in xs])
    assert e.value.status == vrc.VRC_ERR_ALIAS
    with pytest.raises(ValueError):
        vrc.vrc_reduce_scatter([x.view(8, 125) for x in xs], dim=1)  # 125 not divisible by 4
    with pytest.raises(TypeError):
        vrc.vrc_allreduce([x.double() for x in xs])
    with pytest.raises(vrc.VrcError) as e:
        vrc.vrc_allreduce(xs[:3], mode="hd")  # halving-doubling needs a power of two
    assert e.value.status == vrc.VRC_ERR_INVALID_ARG
    empty = [torch.empty(0, device=DEV) for _ in range(4)]
    for mode in MODES:
        vrc.vrc_allreduce(empty, mode=mode)
        vrc.vrc_all_gather(empty, mode=mode)
    torch.cuda.synchronize()
    assert vrc.lib().vrc_last_hip_error() == 0


@pytest.mark.parametrize("mode", MODES)
def test_more_than_2_to_31_elements_per_rank(vrc, orc, mode):
    """64-bit indexing: 2^31 + 7 bf16 elements per rank (4 GiB), 2 ranks,
    checked on sampled elements (chunk boundary, ends, beyond 2^31)."""
    say(f"2^31+7 elements {mode}")
    count = (1 << 31) + 7
    g = torch.Generator(device=DEV).manual_seed(409)
    xs = [torch.randint(-8, 9, (count,), generator=g, device=DEV, dtype=torch.int8).to(torch.bfloat16)
          for _ in range(2)]
    ys = vrc.vrc_allreduce(xs, mode=mode)
    torch.cuda.synchronize()
    rng = np.random.default_rng(409)
    idx = np.unique(np.concatenate([
        rng.integers(0, count, 200000), np.arange(0, 64), np.arange(count - 64, count),
        np.arange((1 << 31) - 64, (1 << 31) + 7), np.arange(count // 2 - 64, count // 2 + 64)])).astype(np.int64)
    tidx = torch.from_numpy(idx).to(DEV)
    sx = [workloads.to_numpy(x[tidx]) for x in xs]
    # small integers: every order gives the exact sum
    want = (sx[0].astype(np.uint32) << 16).view(np.float32) + (sx[1].astype(np.uint32) << 16).view(np.float32)
    for r in range(2):
        got = (workloads.to_numpy(ys[r][tidx]).astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(got, want), f"{mode} rank {r}"
    del xs, ys
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["fused", "hd_order", "ring_order"])
def test_realigned_past_2_to_31_elements_per_rank(vrc, orc, mode):
    """64-bit indexing in the realigned kernels: 2^31 + 7 bf16 elements per
    rank, 2 ranks, outputs 74 bytes apart modulo 128 (vrc_plan confirms the
    realigned launch); sampled elements, ends and the 2^31 boundary."""
    say(f"realigned 2^31+7 elements {mode}")
    count = (1 << 31) + 7
    xs = small_int_bf16(count, 2, 410)
    bufs = [torch.empty(count + 64, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    ys = [bufs[0][:count], bufs[1][37:37 + count]]
    ops, _ = vrc.plan(vrc.COLL_ALLREDUCE, [x.data_ptr() for x in xs], [y.data_ptr() for y in ys], count, 1,
                      vrc.VRC_BF16, vrc.MODES[mode])
    assert ops[0]["kind"].endswith("_realigned"), ops[0]["kind"]
    vrc.vrc_allreduce(xs, recv=ys, mode=mode)
    torch.cuda.synchronize()
    rng = np.random.default_rng(410)
    idx = np.unique(np.concatenate([
        rng.integers(0, count, 200000), np.arange(0, 256), np.arange(count - 256, count),
        np.arange((1 << 31) - 256, (1 << 31) + 7), np.arange(count // 2 - 256, count // 2 + 256)])).astype(np.int64)
    want = as_f32(xs[0], idx) + as_f32(xs[1], idx)  # small integers: every order gives the exact sum
    for r in range(2):
        assert np.array_equal(as_f32(ys[r], idx), want), f"{mode} rank {r}"
    del xs, ys, bufs
    torch.cuda.empty_cache()


def small_int_bf16(count, n, seed):
    """n bf16 tensors of small integers: any summation order gives the exact sum."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    return [torch.randint(-8, 9, (count,), generator=g, device=DEV, dtype=torch.int8).to(torch.bfloat16)
            for _ in range(n)]


def as_f32(t, idx):
    """bf16 values of t at indices idx, widened to float32 on the host."""
    return (workloads.to_numpy(t[torch.from_numpy(idx).to(t.device)]).astype(np.uint32) << 16).view(np.float32)


def sample_idx(length, seed):
    """Random indices of [0, length) plus both ends and the 2^31 and 2^32 boundaries."""
    rng = np.random.default_rng(seed)
    parts = [rng.integers(0, length, 200000), np.arange(0, 64), np.arange(length - 64, length)]
    for b in (1 << 31, 1 << 32):
        if b < length:
            parts.append(np.arange(b - 64, min(b + 64, length)))
    return np.unique(np.concatenate(parts)).astype(np.int64)


@pytest.mark.parametrize("mode", MODES)
def test_reduce_scatter_chunks_past_2_to_31_elements(vrc, orc, mode):
    """64-bit indexing in the reduce-scatter: 2 ranks of 2^32 + 17 bf16 elements
    (8 GiB each), so both chunks hold more than 2^31 elements and chunk 1
    starts 4 GiB into every input; chunk 1 has a one-element tail.  Checked
    on sampled elements."""
    say(f"reduce-scatter 2^32+17 elements {mode}")
    count = (1 << 32) + 17
    xs = small_int_bf16(count, 2, 411)
    ys = vrc.vrc_reduce_scatter(xs, mode=mode)
    torch.cuda.synchronize()
    for c in range(2):
        base = count // 2  # chunk c starts at c*base; the last chunk takes the remainder
        off, length = c * base, (base if c == 0 else count - base)
        assert ys[c].numel() == length
        idx = sample_idx(length, 411 + c)
        want = as_f32(xs[0], idx + off) + as_f32(xs[1], idx + off)
        assert np.array_equal(as_f32(ys[c], idx), want), f"{mode} chunk {c}"
    del xs, ys
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", MODES + ("tree",))
def test_all_gather_output_past_2_to_32_elements(vrc, orc, mode):
    """64-bit indexing in the all-gather: 2 ranks of 2^31 + 8 bf16 elements,
    so every output holds 2^32 + 16 elements (8 GiB) and slab 1 starts past
    2^31 elements.  Checked on sampled elements of both outputs."""
    say(f"all-gather 2^31+8 elements {mode}")
    count = (1 << 31) + 8
    xs = small_int_bf16(count, 2, 413)
    ys = vrc.vrc_all_gather(xs, mode=mode)
    torch.cuda.synchronize()
    idx = sample_idx(2 * count, 413)
    src = np.where(idx < count, 0, 1)
    want = np.where(src == 0, as_f32(xs[0], np.minimum(idx, count - 1)),
                    as_f32(xs[1], np.maximum(idx - count, 0)))
    for r in range(2):
        assert np.array_equal(as_f32(ys[r], idx), want), f"{mode} rank {r}"
    del xs, ys
    torch.cuda.empty_cache()
