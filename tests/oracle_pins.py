"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
AssertionError (or an oracle error) when the oracle disagrees with:

* the message schedule and end states of the 4-card walkthrough on
  hwcomputing.csdn.net/6a0dc11a10ee7a33f273f7fd.html ("Ring 通信为什么常见"),
  written out by hand in ``tests/golden``;
* its per-card traffic formula 2(N-1)*S/N;
* closed forms that hold whatever the summation order: integer sums,
  exactly representable float sums, concatenation for the all-gather;
* library arithmetic (numpy float16/float32, torch bfloat16) through the
  independent relay simulation in ``brute_ring``;
* the IEEE 754 format definitions (exhaustive fp16/bf16 decode checks);
* the standard error bound of recursive summation (Higham, Accuracy and
  Stability of Numerical Algorithms, 2nd ed., eq. 4.4);
* for halving-doubling and the binomial-tree all-gather, hand-derived
  schedules of their textbook forms (Thakur, Rabenseifner and Gropp 2005).

The same functions run against deliberately broken builds of the oracle in
``test_oracle_mutants.py``, to show that each plausible mistake is caught.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle as orc_mod
from tests import brute_ring as brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DTYPES = ("int32", "fp32", "fp16", "bf16")
NPT = {"int32": np.int32, "fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}


# ---------------------------------------------------------------------------
# input helpers (numpy, seeded)
# ---------------------------------------------------------------------------
def _rand(rng, dtype, count, scale=1.0):
    if dtype == "int32":
        return rng.integers(-1000, 1001, size=count, dtype=np.int32)
    f = (rng.standard_normal(count) * scale).astype(np.float32)
    if dtype == "fp32":
        return f
    if dtype == "fp16":
        return f.astype(np.float16)
    return brute.narrow(f, "bf16")


def _ranks(rng, dtype, n, count, scale=1.0):
    return [_rand(rng, dtype, count, scale) for _ in range(n)]


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8)


def _same_bits(a, b, what):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.array_equal(_bits(a), _bits(b)), f"{what}: bits differ"


def _to_f64(a, dtype):
    if dtype == "bf16":
        return brute.widen(a, "bf16").astype(np.float64)
    return a.astype(np.float64)


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ---------------------------------------------------------------------------
# schedule and end states (the pages' walkthrough)
# ---------------------------------------------------------------------------
def pin_schedule_golden_n4(orc):
    """Every message of the N=4 all-reduce matches the hand-derived schedule."""
    want = []
    for row in _read_rows("ring_n4_schedule.txt"):
        ph, s, src, dst, c = row.split()
        want.append((0 if ph == "rs" else 1, int(s), int(src), int(dst), int(c)))
    xs = [np.arange(12, dtype=np.int32) for _ in range(4)]
    _, tr = orc.ring_allreduce(xs, "int32", trace=True)
    got = [m[:5] for m in tr.messages]
    assert sorted(got) == sorted(want), f"schedule differs:\n{got}\nvs\n{want}"


def pin_schedule_first_step(orc):
    """In the first step rank r hands block r to rank r+1, for every N."""
    for n in range(2, 9):
        xs = [np.zeros(3 * n + 1, dtype=np.int32) for _ in range(n)]
        _, tr = orc.ring_allreduce(xs, "int32", trace=True)
        first = sorted(m[2:5] for m in tr.messages if m[0] == 0 and m[1] == 0)
        assert first == [(r, (r + 1) % n, r) for r in range(n)], f"n={n}: {first}"
        assert len(tr.messages) == 2 * n * (n - 1), f"n={n}: {len(tr.messages)} messages"


def pin_contributors_golden_n4(orc):
    """Contributor masks after each reduce-scatter step match the hand table."""
    table = {}
    for row in _read_rows("ring_n4_contributors.txt"):
        s, r, *masks = (int(v) for v in row.split())
        table[(s, r)] = masks
    n, count = 4, 8  # two elements per block
    xs = [np.full(count, 1 << r, dtype=np.int32) for r in range(n)]
    for s in range(-1, n - 1):
        ys = orc.ring_allreduce(xs, "int32", rs_steps=s + 1, ag_steps=0)
        for r in range(n):
            got = [int(ys[r][2 * c]) for c in range(n)]
            got2 = [int(ys[r][2 * c + 1]) for c in range(n)]
            assert got == table[(s, r)] and got2 == got, f"after step {s} rank {r}: {got}"


def pin_rs_end_state_every_n(orc):
    """After N-1 reduce-scatter steps each rank owns exactly one complete block,
    and each block is complete at exactly one rank (every contribution once)."""
    for n in range(2, 9):
        xs = [np.full(n, 1 << r, dtype=np.int32) for r in range(n)]
        ys = orc.ring_allreduce(xs, "int32", rs_steps=n - 1, ag_steps=0)
        full = (1 << n) - 1
        owners = {}
        for r in range(n):
            complete = [c for c in range(n) if int(ys[r][c]) == full]
            assert len(complete) == 1, f"n={n} rank {r} complete blocks {complete}"
            owners.setdefault(complete[0], []).append(r)
            for c in range(n):  # partial masks never double count: values are sub-masks
                v = int(ys[r][c])
                assert v & ~full == 0
        assert sorted(owners) == list(range(n)) and all(len(v) == 1 for v in owners.values())


def pin_traffic_formula(orc):
    """Per-rank traffic is 2(N-1)/N of the buffer when N divides the count,
    and 2(N-1)*count elements in total for any count."""
    for n in range(1, 9):
        for count in (0, 1, n, 4 * n, 4 * n + 3, 1000):
            xs = [np.zeros(count, dtype=np.float32) for _ in range(n)]
            _, tr = orc.ring_allreduce(xs, "fp32", trace=True)
            assert sum(tr.sent_elems) == 2 * (n - 1) * count, (n, count)
            assert sum(tr.recv_elems) == 2 * (n - 1) * count, (n, count)
            if count % n == 0:
                assert all(s == 2 * (n - 1) * count // n for s in tr.sent_elems), (n, count)


# ---------------------------------------------------------------------------
# order-free closed forms
# ---------------------------------------------------------------------------
def pin_integer_equals_naive_sum(orc):
    """int32 ring and fused all-reduce equal the exact sum (mod 2^32) on every rank."""
    rng = np.random.default_rng(11)
    for n in range(1, 9):
        for count in (0, 1, n - 1, n, 2 * n + 1, 4099):
            xs = _ranks(rng, "int32", n, count)
            want = brute.narrow(np.sum([x.astype(np.int64) for x in xs], axis=0), "int32") \
                if count else np.zeros(0, np.int32)
            for ys in (orc.ring_allreduce(xs, "int32"), orc.fused_allreduce(xs, "int32")):
                for r in range(n):
                    _same_bits(ys[r], want, f"int32 n={n} count={count} rank {r}")
    # wrap-around: the sum overflows int32
    xs = [np.full(5, 2**31 - 1, dtype=np.int32) for _ in range(3)]
    want = np.full(5, np.int32(2**31 - 3))
    _same_bits(orc.ring_allreduce(xs, "int32")[0], want, "int32 wrap ring")
    _same_bits(orc.fused_allreduce(xs, "int32")[0], want, "int32 wrap fused")


def pin_exact_small_integer_floats(orc):
    """When every partial sum is exactly representable the order cannot
    matter: ring == fused == the integer sum, for all float types."""
    rng = np.random.default_rng(12)
    for dtype in ("fp32", "fp16", "bf16"):
        for n in (2, 3, 5, 8):
            count = 37
            ints = [rng.integers(-15, 16, size=count) for _ in range(n)]  # |partial| <= 120
            xs = [brute.narrow(i.astype(np.float32), dtype) for i in ints]
            want = np.sum(ints, axis=0).astype(np.float64)
            for ys in (orc.ring_allreduce(xs, dtype), orc.fused_allreduce(xs, dtype)):
                for r in range(n):
                    assert np.array_equal(_to_f64(ys[r], dtype), want), (dtype, n, r)


def pin_all_ranks_identical(orc):
    """Every rank ends with the same bits (ring, all dtypes, random data)."""
    rng = np.random.default_rng(13)
    for dtype in DTYPES:
        for n in (2, 3, 7, 8):
            xs = _ranks(rng, dtype, n, 101)
            ys = orc.ring_allreduce(xs, dtype)
            for r in range(1, n):
                _same_bits(ys[r], ys[0], f"{dtype} n={n} rank {r}")


def pin_all_gather_is_concat(orc):
    """All-gather output is the concatenation of the inputs along the row axis."""
    rng = np.random.default_rng(14)
    for dtype in DTYPES:
        for n, outer, row in ((1, 1, 5), (2, 1, 7), (3, 4, 5), (8, 2, 16), (4, 3, 1)):
            xs = _ranks(rng, dtype, n, outer * row)
            want = np.concatenate([x.reshape(outer, row) for x in xs], axis=1).reshape(-1)
            ys = orc.ring_all_gather(xs, dtype, outer=outer)
            for r in range(n):
                _same_bits(ys[r], want, f"{dtype} n={n} outer={outer} rank {r}")


def pin_composition(orc):
    """All-reduce = reduce-scatter followed by all-gather, bit for bit."""
    rng = np.random.default_rng(15)
    for dtype in ("int32", "fp32", "fp16", "bf16"):
        for n in (2, 3, 4, 8):
            count = 8 * n  # equal blocks so the gathered pieces have one size
            xs = _ranks(rng, dtype, n, count)
            ar = orc.ring_allreduce(xs, dtype)
            rs = orc.ring_reduce_scatter(xs, dtype)
            ag = orc.ring_all_gather(rs, dtype)
            for r in range(n):
                _same_bits(ag[r], ar[r], f"{dtype} n={n} rank {r}")


# ---------------------------------------------------------------------------
# brute force and library arithmetic
# ---------------------------------------------------------------------------
def pin_brute_force_small(orc):
    """N = 1..4 and count 0..3N+2: the oracle equals the independent relay
    simulation and the numpy/torch fold, bit for bit, for every dtype."""
    rng = np.random.default_rng(16)
    for dtype in DTYPES:
        for n in range(1, 5):
            for count in range(0, 3 * n + 3):
                xs = _ranks(rng, dtype, n, count)
                want = brute.ring_allreduce(xs, dtype)
                got = orc.ring_allreduce(xs, dtype)
                for r in range(n):
                    _same_bits(got[r], want[r], f"ring {dtype} n={n} count={count} rank {r}")
                fused = orc.fused_allreduce(xs, dtype)
                ref = brute.fused_fold(xs, dtype) if count else xs[0].copy()
                for r in range(n):
                    _same_bits(fused[r], ref, f"fused {dtype} n={n} count={count} rank {r}")
                rs = orc.ring_reduce_scatter(xs, dtype)
                want_rs = brute.ring_reduce_scatter(xs, dtype)
                for c in range(n):
                    _same_bits(rs[c], want_rs[c], f"rs {dtype} n={n} count={count} chunk {c}")
                frs = orc.fused_reduce_scatter(xs, dtype)
                want_frs = brute.fused_reduce_scatter(xs, dtype) if count else [
                    np.zeros(0, NPT[dtype])] * n
                for c in range(n):
                    _same_bits(frs[c], want_frs[c], f"frs {dtype} n={n} count={count} chunk {c}")


def pin_brute_force_columns(orc):
    """Reduce-scatter over column blocks of an [outer, row] view matches the
    relay simulation and the fold (dim-aware reduce-scatter)."""
    rng = np.random.default_rng(17)
    for dtype in DTYPES:
        for n, outer, w in ((2, 3, 2), (4, 2, 3), (3, 5, 1), (8, 2, 2)):
            count = outer * n * w
            xs = _ranks(rng, dtype, n, count)
            rs = orc.ring_reduce_scatter(xs, dtype, outer=outer)
            want = brute.ring_reduce_scatter(xs, dtype, outer=outer)
            frs = orc.fused_reduce_scatter(xs, dtype, outer=outer)
            want_f = brute.fused_reduce_scatter(xs, dtype, outer=outer)
            for c in range(n):
                _same_bits(rs[c], want[c], f"rs {dtype} n={n} outer={outer} chunk {c}")
                _same_bits(frs[c], want_f[c], f"frs {dtype} n={n} outer={outer} chunk {c}")


def pin_brute_force_wide(orc):
    """Larger N (5..8) with remainder blocks against the relay simulation."""
    rng = np.random.default_rng(18)
    for dtype in DTYPES:
        for n in (5, 6, 8):
            for count in (n - 1, 2 * n + 3, 64 + 5):
                xs = _ranks(rng, dtype, n, count)
                want = brute.ring_allreduce(xs, dtype)
                got = orc.ring_allreduce(xs, dtype)
                for r in range(n):
                    _same_bits(got[r], want[r], f"ring {dtype} n={n} count={count} rank {r}")


def pin_order_golden_n4(orc):
    """The hand-derived order-sensitive example (ring rounds per block in its
    travel order; fused accumulates in fp32 and rounds once)."""
    for row in _read_rows("ring_n4_order.txt"):
        head, ring_s, fused_s = (p.strip() for p in row.split("|"))
        dtype, *vs = head.split()
        v = [float(t) for t in vs]
        ring_want = np.array([float(t) for t in ring_s.split()], dtype=np.float64)
        fused_want = float(fused_s)
        count = ring_want.size
        xs = [brute.narrow(np.full(count, v[r], dtype=np.float32), dtype) for r in range(4)]
        for r in range(4):  # the inputs themselves must be exact
            assert np.all(_to_f64(xs[r], dtype) == v[r])
        ys = orc.ring_allreduce(xs, dtype)
        for r in range(4):
            assert np.array_equal(_to_f64(ys[r], dtype), ring_want), (dtype, r, ys[r])
        fs = orc.fused_allreduce(xs, dtype)
        for r in range(4):
            assert np.all(_to_f64(fs[r], dtype) == fused_want), (dtype, r, fs[r])


def pin_closed_forms_match_simulation(orc):
    """The per-element forms used for sampled checks at full size agree with
    the simulation and the fused fold at every index."""
    rng = np.random.default_rng(19)
    for dtype in DTYPES:
        for n, count in ((1, 5), (2, 9), (4, 4099), (8, 1000), (8, 5)):
            xs = _ranks(rng, dtype, n, count)
            idx = np.arange(count, dtype=np.uint64)
            _same_bits(orc.ring_allreduce_at(xs, dtype, idx), orc.ring_allreduce(xs, dtype)[0],
                       f"ring_at {dtype} n={n} count={count}")
            _same_bits(orc.fused_allreduce_at(xs, dtype, idx), orc.fused_allreduce(xs, dtype)[0],
                       f"fused_at {dtype} n={n} count={count}")


# ---------------------------------------------------------------------------
# codecs and element arithmetic against library routines
# ---------------------------------------------------------------------------
def pin_codec_fp16_exhaustive(orc):
    """Decoding all 2^16 fp16 patterns agrees with numpy; encode(decode(h))
    is the identity on every non-NaN pattern; NaNs stay NaN."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    back = orc.f32_to_f16_bits(got)
    assert np.array_equal(back[~nan], h[~nan])
    assert np.all(np.isnan(back.view(np.float16)[nan]))


def pin_codec_bf16_exhaustive(orc):
    """bfloat16 is the top half of a float32: decoding every pattern equals
    that float; encode(decode(b)) is the identity on non-NaN patterns."""
    b = np.arange(65536, dtype=np.uint32)
    got = orc.bf16_bits_to_f32(b.astype(np.uint16))
    ref = (b << 16).astype(np.uint32).view(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    back = orc.f32_to_bf16_bits(got)
    assert np.array_equal(back[~nan], b.astype(np.uint16)[~nan])


def _rounding_probe_floats(rng):
    """Random floats over the whole range, plus exact ties and near-ties for
    both fp16 and bf16 (mid-points between neighbouring values)."""
    parts = [rng.standard_normal(20000).astype(np.float32),
             (rng.standard_normal(20000) * 1e-5).astype(np.float32),   # fp16 subnormals
             (rng.standard_normal(20000) * 3e4).astype(np.float32),    # near fp16 overflow
             rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32).view(np.float32)]
    # fp16 mid-points: average of consecutive fp16 values is exact in float32
    h = np.arange(0, 0x7c00, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float32)
    hi = (h + 1).view(np.float16).astype(np.float32)
    mid = (lo + hi) / np.float32(2)
    parts += [mid, -mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))]
    # bf16 mid-points: low half 0x8000 is an exact tie
    b = rng.integers(0, 0x7f7f, size=20000, dtype=np.uint32)
    ties = ((b << 16) | 0x8000).astype(np.uint32).view(np.float32)
    parts += [ties, -ties, ((b << 16) | 0x7fff).astype(np.uint32).view(np.float32),
              ((b << 16) | 0x8001).astype(np.uint32).view(np.float32)]
    parts.append(np.array([65504, 65519.99, 65520, 65536, 1e-8, 5.96e-8, 2.98e-8, 0.0, -0.0,
                           3.4e38, np.inf, -np.inf], dtype=np.float32))
    return np.concatenate(parts).astype(np.float32)


def pin_codec_rounding_vs_libraries(orc):
    """Round-to-nearest-even narrowing agrees with numpy's float16 cast and
    torch's bfloat16 cast on random values, exact ties and overflow."""
    rng = np.random.default_rng(20)
    f = _rounding_probe_floats(rng)
    f = f[~np.isnan(f)]
    with np.errstate(over="ignore"):
        ref16 = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f32_to_f16_bits(f), ref16)
    ref_bf = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16_bits(f), ref_bf)


def pin_element_add_vs_libraries(orc):
    """One storage-format add equals numpy (int32, fp32, fp16) and torch (bf16)."""
    rng = np.random.default_rng(21)
    for dtype in DTYPES:
        a = _rand(rng, dtype, 50000, 1.0)
        b = _rand(rng, dtype, 50000, 1e-3)
        _same_bits(orc.add(a, b, dtype), brute.storage_add(a, b, dtype), f"add {dtype}")
        _same_bits(orc.add(a, a, dtype), brute.storage_add(a, a, dtype), f"add {dtype} self")


# ---------------------------------------------------------------------------
# error bound of the fused fold (Higham eq. 4.4 plus one final rounding)
# ---------------------------------------------------------------------------
def pin_fused_error_bound(orc):
    """|y - s| <= gamma_{N-1} * sum|x| + u_s * (|s| + gamma_{N-1} * sum|x|) + eta,
    with u = 2^-24 for the fp32 accumulator, u_s the storage unit roundoff
    (0 for fp32, 2^-11 fp16, 2^-8 bf16) and eta the storage subnormal spacing."""
    rng = np.random.default_rng(22)
    us = {"fp32": 0.0, "fp16": 2.0**-11, "bf16": 2.0**-8}
    eta = {"fp32": 0.0, "fp16": 2.0**-24, "bf16": 2.0**-133}
    for dtype in ("fp32", "fp16", "bf16"):
        n, count = 8, 200000
        xs = _ranks(rng, dtype, n, count, 1e-2)
        x64 = [_to_f64(x, dtype) for x in xs]
        s = np.sum(x64, axis=0)
        sabs = np.sum(np.abs(x64), axis=0)
        k = n - 1
        gamma = k * 2.0**-24 / (1 - k * 2.0**-24)
        y = _to_f64(orc.fused_allreduce(xs, dtype)[0], dtype)
        bound = gamma * sabs + us[dtype] * (np.abs(s) + gamma * sabs) + eta[dtype]
        assert np.all(np.abs(y - s) <= bound), dtype
        # the bound is tight enough to matter: accumulating in the storage
        # type would violate it somewhere for fp16/bf16
        if dtype != "fp32":
            acc = xs[0]
            for x in xs[1:]:
                acc = brute.storage_add(acc, x, dtype)
            err = np.abs(_to_f64(acc, dtype) - s)
            assert np.any(err > bound), dtype


# ---------------------------------------------------------------------------
# special cases and the simulated transport's failure detection
# ---------------------------------------------------------------------------
def pin_special_cases(orc):
    """N = 1 is the identity; count < N leaves empty blocks; count = 0 is a no-op."""
    rng = np.random.default_rng(23)
    for dtype in DTYPES:
        x = _rand(rng, dtype, 17)
        _same_bits(orc.ring_allreduce([x], dtype)[0], x, f"{dtype} n=1 ring")
        _same_bits(orc.fused_allreduce([x], dtype)[0], x, f"{dtype} n=1 fused")
        _same_bits(orc.ring_reduce_scatter([x], dtype)[0], x, f"{dtype} n=1 rs")
        _same_bits(orc.ring_all_gather([x], dtype)[0], x, f"{dtype} n=1 ag")
        xs = _ranks(rng, dtype, 6, 4)  # blocks of 0,0,0,0,0,4 elements
        lens = [orc.chunk_range(4, 6, c)[1] for c in range(6)]
        assert lens == [0, 0, 0, 0, 0, 4]
        rs = orc.ring_reduce_scatter(xs, dtype)
        assert [r.size for r in rs] == lens
        empty = [np.zeros(0, NPT[dtype]) for _ in range(3)]
        assert all(y.size == 0 for y in orc.ring_allreduce(empty, dtype))
    for count, n in ((4099, 4), (10, 3), (7, 8), (1 << 20, 8)):
        lens = [orc.chunk_range(count, n, c) for c in range(n)]
        base = count // n
        assert all(off == c * base for c, (off, _) in enumerate(lens))
        assert [ln for _, ln in lens] == [base] * (n - 1) + [count - (n - 1) * base]


def pin_fault_detection(orc):
    """A dropped, duplicated, misrouted or wrong-block message in either phase
    makes the simulation fail loudly instead of returning a wrong sum."""
    rng = np.random.default_rng(24)
    n = 4
    xs = _ranks(rng, "fp32", n, 4 * n + 1)
    for kind in (orc_mod.FAULT_DROP, orc_mod.FAULT_DUP, orc_mod.FAULT_MISROUTE,
                 orc_mod.FAULT_WRONG_CHUNK):
        for phase in (orc_mod.PHASE_RS, orc_mod.PHASE_AG):
            for step in (0, n - 2):
                f = orc_mod.Fault(kind, phase, step, rank=1)
                try:
                    orc.ring_allreduce(xs, "fp32", fault=f)
                except orc_mod.OracleError as e:
                    assert e.code in (orc_mod.E_EMPTY, orc_mod.E_TAG, orc_mod.E_LEFTOVER), e
                else:
                    raise AssertionError(f"fault {kind} phase {phase} step {step} not detected")
    for kind in (orc_mod.FAULT_DROP, orc_mod.FAULT_DUP, orc_mod.FAULT_MISROUTE,
                 orc_mod.FAULT_WRONG_CHUNK):
        f = orc_mod.Fault(kind, orc_mod.PHASE_AG, 1, rank=2)
        for call in (lambda: orc.ring_all_gather(xs, "fp32", fault=f),
                     lambda: orc.ring_reduce_scatter(xs, "fp32", fault=orc_mod.Fault(
                         kind, orc_mod.PHASE_RS, 1, rank=2))):
            try:
                call()
            except orc_mod.OracleError:
                pass
            else:
                raise AssertionError(f"fault {kind} not detected")




# ---------------------------------------------------------------------------
# halving-doubling (recursive halving reduce-scatter + recursive doubling
# all-gather), pinned the same way: hand-derived N = 4 fixtures, integer
# sums, the traffic formula, an independent recursive brute force, the
# pairwise-summation error bound and fault detection
# ---------------------------------------------------------------------------
def pin_hd_schedule_golden_n4(orc):
    want = []
    for row in _read_rows("hd_n4_schedule.txt"):
        ph, s, src, dst, lo, hi = row.split()
        want.append((orc_mod.PHASE_HD_RS if ph == "rs" else orc_mod.PHASE_HD_AG, int(s), int(src), int(dst),
                     int(lo), int(hi)))
    xs = [np.arange(12, dtype=np.int32) for _ in range(4)]
    _, tr = orc.hd_allreduce(xs, "int32", trace=True)
    got = [(m[0], m[1], m[2], m[3], m[4], m[6]) for m in tr.messages]
    assert sorted(got) == sorted(want), f"hd schedule differs:\n{got}\nvs\n{want}"


def pin_hd_contributors_golden_n4(orc):
    table = {}
    for row in _read_rows("hd_n4_contributors.txt"):
        s, r, *masks = (int(v) for v in row.split())
        table[(s, r)] = masks
    xs = [np.full(8, 1 << r, dtype=np.int32) for r in range(4)]
    for s in range(-1, 2):
        ys = orc.hd_allreduce(xs, "int32", rs_steps=s + 1, ag_steps=0)
        for r in range(4):
            got = [int(ys[r][2 * c]) for c in range(4)]
            assert got == table[(s, r)] and [int(ys[r][2 * c + 1]) for c in range(4)] == got, (s, r, got)


def pin_hd_order_golden_n4(orc):
    for row in _read_rows("hd_n4_order.txt"):
        head, out_s = (p.strip() for p in row.split("|"))
        dtype, *vs = head.split()
        v = [float(t) for t in vs]
        want = np.array([float(t) for t in out_s.split()], dtype=np.float64)
        xs = [brute.narrow(np.full(want.size, v[r], dtype=np.float32), dtype) for r in range(4)]
        for ys in (orc.hd_allreduce(xs, dtype),):
            for r in range(4):
                assert np.array_equal(_to_f64(ys[r], dtype), want), (dtype, r)


def pin_hd_integer_equals_naive_sum(orc):
    rng = np.random.default_rng(31)
    for n in (1, 2, 4, 8, 16):
        for count in (0, 1, n - 1, n, 3 * n + 5, 4099):
            xs = _ranks(rng, "int32", n, count)
            want = brute.narrow(np.sum([x.astype(np.int64) for x in xs], axis=0), "int32") if count else \
                np.zeros(0, np.int32)
            for r, y in enumerate(orc.hd_allreduce(xs, "int32")):
                _same_bits(y, want, f"hd int32 n={n} count={count} rank {r}")


def pin_hd_all_ranks_identical_and_traffic(orc):
    rng = np.random.default_rng(32)
    for dtype in DTYPES:
        for n in (2, 4, 8, 16):
            for count in (n, 8 * n, 8 * n + 3):
                xs = _ranks(rng, dtype, n, count)
                ys, tr = orc.hd_allreduce(xs, dtype, trace=True)
                for r in range(1, n):
                    _same_bits(ys[r], ys[0], f"hd {dtype} n={n} rank {r}")
                assert sum(tr.sent_elems) == 2 * (n - 1) * count, (n, count)
                if count % n == 0:
                    assert all(s == 2 * (n - 1) * count // n for s in tr.sent_elems), (n, count)
                k = n.bit_length() - 1
                assert len(tr.messages) == 2 * k * n


def pin_hd_brute_force(orc):
    rng = np.random.default_rng(33)
    for dtype in DTYPES:
        for n in (1, 2, 4, 8):
            for count in range(0, 3 * n + 3, max(1, n // 2)):
                xs = _ranks(rng, dtype, n, count)
                want = brute.hd_allreduce(xs, dtype)
                got = orc.hd_allreduce(xs, dtype)
                for r in range(n):
                    _same_bits(got[r], want[r], f"hd {dtype} n={n} count={count} rank {r}")
                rs = orc.hd_reduce_scatter(xs, dtype)
                want_rs = brute.hd_reduce_scatter(xs, dtype)
                for c in range(n):
                    _same_bits(rs[c], want_rs[c], f"hd rs {dtype} n={n} count={count} chunk {c}")
        for n, outer, w in ((2, 3, 2), (4, 2, 3), (8, 2, 2)):
            xs = _ranks(rng, dtype, n, outer * n * w)
            rs = orc.hd_reduce_scatter(xs, dtype, outer=outer)
            want = brute.hd_reduce_scatter(xs, dtype, outer=outer)
            for c in range(n):
                _same_bits(rs[c], want[c], f"hd rs {dtype} n={n} outer={outer} chunk {c}")


def pin_hd_all_gather_and_composition(orc):
    rng = np.random.default_rng(34)
    for dtype in DTYPES:
        for n, outer, row in ((1, 1, 5), (2, 1, 7), (4, 3, 5), (8, 2, 16), (16, 1, 3)):
            xs = _ranks(rng, dtype, n, outer * row)
            want = np.concatenate([x.reshape(outer, row) for x in xs], axis=1).reshape(-1)
            for r, y in enumerate(orc.hd_all_gather(xs, dtype, outer=outer)):
                _same_bits(y, want, f"hd ag {dtype} n={n} rank {r}")
        for n in (2, 4, 8):
            xs = _ranks(rng, dtype, n, 8 * n)
            ar = orc.hd_allreduce(xs, dtype)
            ag = orc.hd_all_gather(orc.hd_reduce_scatter(xs, dtype), dtype)
            for r in range(n):
                _same_bits(ag[r], ar[r], f"hd AG(RS) {dtype} n={n} rank {r}")


def pin_hd_closed_form_matches_simulation(orc):
    rng = np.random.default_rng(35)
    for dtype in DTYPES:
        for n, count in ((1, 5), (2, 9), (4, 4099), (8, 1000), (16, 77)):
            xs = _ranks(rng, dtype, n, count)
            idx = np.arange(count, dtype=np.uint64)
            _same_bits(orc.hd_allreduce_at(xs, dtype, idx), orc.hd_allreduce(xs, dtype)[0],
                       f"hd_at {dtype} n={n} count={count}")


def pin_hd_error_bound(orc):
    """Pairwise summation (Higham eq. 4.6) with each partial rounded to the
    storage type: |y - s| <= gamma_{log2 N}(u_s) * sum|x|, on same-sign data
    in [1, 2) where rounding errors pile up fastest, and on N(0, 0.01^2)."""
    rng = np.random.default_rng(36)
    for dtype, u in (("fp16", 2.0**-11), ("bf16", 2.0**-8)):
        n, count = 16, 100000
        for xs in ([brute.narrow((1 + rng.random(count)).astype(np.float32), dtype) for _ in range(n)],
                   _ranks(rng, dtype, n, count, 1e-2)):
            x64 = [_to_f64(x, dtype) for x in xs]
            s = np.sum(x64, axis=0)
            sabs = np.sum(np.abs(x64), axis=0)
            k = 4
            bound = k * u / (1 - k * u) * sabs + 2.0**-24
            y = _to_f64(orc.hd_allreduce(xs, dtype)[0], dtype)
            assert np.all(np.abs(y - s) <= bound), dtype


def pin_hd_rejects_non_power_of_two_and_detects_faults(orc):
    rng = np.random.default_rng(37)
    for n in (3, 5, 6, 12):
        xs = _ranks(rng, "fp32", n, 10)
        try:
            orc.hd_allreduce(xs, "fp32")
        except orc_mod.OracleError as e:
            assert e.code == orc_mod.E_ARG
        else:
            raise AssertionError(f"n={n} accepted")
    n = 8
    xs = _ranks(rng, "fp32", n, 4 * n + 1)
    for kind in (orc_mod.FAULT_DROP, orc_mod.FAULT_DUP, orc_mod.FAULT_MISROUTE, orc_mod.FAULT_WRONG_CHUNK):
        for phase in (orc_mod.PHASE_HD_RS, orc_mod.PHASE_HD_AG):
            for step in (0, 2):
                f = orc_mod.Fault(kind, phase, step, rank=5)
                try:
                    orc.hd_allreduce(xs, "fp32", fault=f)
                except orc_mod.OracleError as e:
                    assert e.code in (orc_mod.E_EMPTY, orc_mod.E_TAG, orc_mod.E_LEFTOVER), e
                else:
                    raise AssertionError(f"hd fault {kind} phase {phase} step {step} not detected")


# ---------------------------------------------------------------------------
# binomial-tree all-gather (gather to rank 0, then broadcast from it), pinned
# by hand-derived N = 4 and N = 5 schedules, concatenation (the all-gather's
# result is unique), message and step counts, the traffic each slab's path
# through the tree fixes, and fault detection
# ---------------------------------------------------------------------------
def _tree_golden(name):
    want = []
    for row in _read_rows(name):
        ph, s, src, dst, lo, hi = row.split()
        phase = orc_mod.PHASE_TREE_GATHER if ph == "gather" else orc_mod.PHASE_TREE_BCAST
        want.append((phase, int(s), int(src), int(dst), int(lo), int(hi)))
    return want


def pin_tree_schedule_golden(orc):
    for n, name in ((4, "tree_n4_schedule.txt"), (5, "tree_n5_schedule.txt")):
        xs = [np.arange(6, dtype=np.int32) + 100 * r for r in range(n)]
        _, tr = orc.tree_all_gather(xs, "int32", trace=True)
        got = [(m[0], m[1], m[2], m[3], m[4], m[6]) for m in tr.messages]
        assert sorted(got) == sorted(_tree_golden(name)), f"tree schedule n={n} differs:\n{got}"


def pin_tree_all_gather_is_concatenation(orc):
    rng = np.random.default_rng(41)
    for dtype in DTYPES:
        for n, outer, row in ((1, 1, 5), (2, 1, 7), (3, 2, 5), (4, 3, 5), (5, 1, 9), (6, 2, 4), (7, 1, 3),
                              (8, 2, 16), (12, 1, 3), (16, 1, 3)):
            xs = _ranks(rng, dtype, n, outer * row)
            want = np.concatenate([x.reshape(outer, row) for x in xs], axis=1).reshape(-1)
            for r, y in enumerate(orc.tree_all_gather(xs, dtype, outer=outer)):
                _same_bits(y, want, f"tree ag {dtype} n={n} outer={outer} rank {r}")


def pin_tree_traffic_and_steps(orc):
    """Every rank but 0 sends once in the gather and receives once in the
    broadcast; each phase takes ceil(log2 N) steps; slab j reaches rank 0 in
    one hop per set bit of j (a hop clears the lowest one), so the gather
    carries sum_j popcount(j) slabs, and the broadcast N slabs to each of the
    N - 1 other ranks."""
    for n in range(1, 17):
        outer, row = 2, 3
        xs = [np.arange(outer * row, dtype=np.int32) + 10 * r for r in range(n)]
        _, tr = orc.tree_all_gather(xs, "int32", outer=outer, trace=True)
        slab = outer * row
        gather = [m for m in tr.messages if m[0] == orc_mod.PHASE_TREE_GATHER]
        bcast = [m for m in tr.messages if m[0] == orc_mod.PHASE_TREE_BCAST]
        assert len(gather) == n - 1 and len(bcast) == n - 1, n
        assert sorted(m[2] for m in gather) == list(range(1, n)), n
        assert sorted(m[3] for m in bcast) == list(range(1, n)), n
        k = (n - 1).bit_length()
        assert {m[1] for m in gather} == set(range(k)) and {m[1] for m in bcast} == set(range(k)), n
        assert sum(m[5] for m in gather) == slab * sum(bin(j).count("1") for j in range(n)), n
        assert sum(m[5] for m in bcast) == slab * n * (n - 1), n
        assert tr.recv_elems[0] == slab * (n - 1), n


def pin_tree_detects_faults(orc):
    rng = np.random.default_rng(42)
    for n, cases in ((8, ((orc_mod.PHASE_TREE_GATHER, 0, 5), (orc_mod.PHASE_TREE_GATHER, 2, 4),
                          (orc_mod.PHASE_TREE_BCAST, 0, 0), (orc_mod.PHASE_TREE_BCAST, 2, 6))),
                     (5, ((orc_mod.PHASE_TREE_GATHER, 2, 4), (orc_mod.PHASE_TREE_BCAST, 2, 2)))):
        xs = _ranks(rng, "fp32", n, 6)
        for kind in (orc_mod.FAULT_DROP, orc_mod.FAULT_DUP, orc_mod.FAULT_MISROUTE, orc_mod.FAULT_WRONG_CHUNK):
            for phase, step, rank in cases:
                try:
                    orc.tree_all_gather(xs, "fp32", fault=orc_mod.Fault(kind, phase, step, rank=rank))
                except orc_mod.OracleError as e:
                    assert e.code in (orc_mod.E_EMPTY, orc_mod.E_TAG, orc_mod.E_LEFTOVER), e
                else:
                    raise AssertionError(f"tree fault {kind} phase {phase} step {step} rank {rank} not detected")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
