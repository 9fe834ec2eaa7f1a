"""CPU oracle for the virtual-rank ring collectives (ctypes over oracle.c).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and the library never calls it.

Arrays are numpy arrays, one per rank.  dtype names: ``int32`` (np.int32),
``fp32`` (np.float32), ``fp16`` (np.float16) and ``bf16`` (np.uint16 holding
the raw bfloat16 bit patterns, since numpy has no bfloat16).

What each function computes, and which passage of the pages it follows, is
stated next to the C function it wraps in ``oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DTYPES = {"int32": 0, "fp32": 1, "fp16": 2, "bf16": 3}
NP_DTYPES = {"int32": np.int32, "fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}

OK, E_ARG, E_NOMEM, E_EMPTY, E_TAG, E_LEFTOVER = range(6)
PHASE_RS, PHASE_AG, PHASE_HD_RS, PHASE_HD_AG, PHASE_TREE_GATHER, PHASE_TREE_BCAST = 0, 1, 2, 3, 4, 5
FAULT_NONE, FAULT_DROP, FAULT_DUP, FAULT_MISROUTE, FAULT_WRONG_CHUNK = range(5)

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", *CFLAGS, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class OracleError(RuntimeError):
    def __init__(self, fn: str, code: int):
        names = {E_ARG: "E_ARG", E_NOMEM: "E_NOMEM", E_EMPTY: "E_EMPTY", E_TAG: "E_TAG",
                 E_LEFTOVER: "E_LEFTOVER"}
        super().__init__(f"oracle {fn} failed: {names.get(code, code)}")
        self.code = code


class _MsgRec(C.Structure):
    _fields_ = [("phase", C.c_int), ("step", C.c_int), ("src", C.c_int), ("dst", C.c_int),
                ("chunk", C.c_int), ("elems", C.c_uint64), ("chunk_hi", C.c_int)]


class _Trace(C.Structure):
    _fields_ = [("log", C.POINTER(_MsgRec)), ("log_cap", C.c_uint64), ("log_len", C.c_uint64),
                ("sent_elems", C.POINTER(C.c_uint64)), ("recv_elems", C.POINTER(C.c_uint64))]


class _Fault(C.Structure):
    _fields_ = [("kind", C.c_int), ("phase", C.c_int), ("step", C.c_int), ("rank", C.c_int)]


@dataclass
class Trace:
    """What the simulated transport saw: one record per posted message."""
    messages: list = field(default_factory=list)  # (phase, step, src, dst, chunk, elems, chunk_hi)
    sent_elems: list = field(default_factory=list)
    recv_elems: list = field(default_factory=list)


@dataclass
class Fault:
    kind: int
    phase: int
    step: int
    rank: int


def _ptrs(arrs):
    arr_t = C.c_void_p * len(arrs)
    return arr_t(*[a.ctypes.data for a in arrs])


class Oracle:
    """Bound oracle library.  ``Oracle(path)`` loads a specific build."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
                build()
        self.path = path
        L = C.CDLL(path)
        self._L = L
        vp, u64, i = C.c_void_p, C.c_uint64, C.c_int
        L.orc_ring_allreduce_steps.argtypes = [i, i, u64, vp, vp, i, i, C.POINTER(_Trace),
                                               C.POINTER(_Fault)]
        L.orc_ring_reduce_scatter.argtypes = [i, i, u64, u64, vp, vp, C.POINTER(_Trace),
                                              C.POINTER(_Fault)]
        L.orc_ring_all_gather.argtypes = [i, i, u64, u64, vp, vp, C.POINTER(_Trace),
                                          C.POINTER(_Fault)]
        L.orc_hd_allreduce_steps.argtypes = [i, i, u64, vp, vp, i, i, C.POINTER(_Trace), C.POINTER(_Fault)]
        L.orc_hd_reduce_scatter.argtypes = [i, i, u64, u64, vp, vp, C.POINTER(_Trace), C.POINTER(_Fault)]
        L.orc_hd_all_gather.argtypes = [i, i, u64, u64, vp, vp, C.POINTER(_Trace), C.POINTER(_Fault)]
        L.orc_hd_allreduce_at.argtypes = [i, i, u64, vp, vp, u64, vp]
        L.orc_tree_all_gather.argtypes = [i, i, u64, u64, vp, vp, C.POINTER(_Trace), C.POINTER(_Fault)]
        L.orc_fused_allreduce.argtypes = [i, i, u64, vp, vp]
        L.orc_fused_reduce_scatter.argtypes = [i, i, u64, u64, vp, vp]
        L.orc_ring_allreduce_at.argtypes = [i, i, u64, vp, vp, u64, vp]
        L.orc_fused_allreduce_at.argtypes = [i, i, u64, vp, vp, u64, vp]
        for f in ("orc_f32_to_f16", "orc_f16_to_f32", "orc_f32_to_bf16", "orc_bf16_to_f32"):
            getattr(L, f).argtypes = [vp, vp, u64]
            getattr(L, f).restype = None
        L.orc_add.argtypes = [i, vp, vp, vp, u64]
        L.orc_chunk_range.argtypes = [u64, i, i, C.POINTER(u64), C.POINTER(u64)]

    # -- helpers --------------------------------------------------------------
    @staticmethod
    def _check_inputs(xs, dtype):
        if dtype not in DTYPES:
            raise ValueError(f"unknown dtype {dtype}")
        want = np.dtype(NP_DTYPES[dtype])
        out = []
        for x in xs:
            x = np.ascontiguousarray(x).reshape(-1)
            if x.dtype != want:
                raise TypeError(f"expected {want}, got {x.dtype}")
            out.append(x)
        if len({x.size for x in out}) > 1:
            raise ValueError("all ranks need the same element count")
        return out

    @staticmethod
    def _make_trace(n, log_cap):
        log = (_MsgRec * max(log_cap, 1))()
        sent = (C.c_uint64 * n)()
        recv = (C.c_uint64 * n)()
        tr = _Trace(C.cast(log, C.POINTER(_MsgRec)), log_cap, 0,
                    C.cast(sent, C.POINTER(C.c_uint64)), C.cast(recv, C.POINTER(C.c_uint64)))
        return tr, (log, sent, recv)

    @staticmethod
    def _read_trace(tr, keep, n):
        log, sent, recv = keep
        t = Trace()
        for k in range(min(tr.log_len, tr.log_cap)):
            r = log[k]
            t.messages.append((r.phase, r.step, r.src, r.dst, r.chunk, int(r.elems), r.chunk_hi))
        t.sent_elems = [int(sent[r]) for r in range(n)]
        t.recv_elems = [int(recv[r]) for r in range(n)]
        return t

    @staticmethod
    def _fault(f):
        if f is None:
            return None
        return C.byref(_Fault(f.kind, f.phase, f.step, f.rank))

    # -- literal ring simulations ---------------------------------------------
    def ring_allreduce(self, xs, dtype, rs_steps=-1, ag_steps=-1, trace=False, fault=None):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty_like(x) for x in xs]
        tr = keep = None
        if trace:
            tr, keep = self._make_trace(n, 2 * n * max(n - 1, 0) + 8)
        rc = self._L.orc_ring_allreduce_steps(DTYPES[dtype], n, count, _ptrs(xs), _ptrs(ys),
                                              rs_steps, ag_steps,
                                              C.byref(tr) if trace else None, self._fault(fault))
        if rc:
            raise OracleError("ring_allreduce", rc)
        return (ys, self._read_trace(tr, keep, n)) if trace else ys

    def ring_reduce_scatter(self, xs, dtype, outer=1, trace=False, fault=None):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty(self.rs_len(count, n, outer, c), dtype=xs[0].dtype) for c in range(n)]
        tr = keep = None
        if trace:
            tr, keep = self._make_trace(n, n * max(n - 1, 0) + 8)
        rc = self._L.orc_ring_reduce_scatter(DTYPES[dtype], n, count, outer, _ptrs(xs), _ptrs(ys),
                                             C.byref(tr) if trace else None, self._fault(fault))
        if rc:
            raise OracleError("ring_reduce_scatter", rc)
        return (ys, self._read_trace(tr, keep, n)) if trace else ys

    def ring_all_gather(self, xs, dtype, outer=1, trace=False, fault=None):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty(n * count, dtype=xs[0].dtype) for _ in range(n)]
        tr = keep = None
        if trace:
            tr, keep = self._make_trace(n, n * max(n - 1, 0) + 8)
        rc = self._L.orc_ring_all_gather(DTYPES[dtype], n, count, outer, _ptrs(xs), _ptrs(ys),
                                         C.byref(tr) if trace else None, self._fault(fault))
        if rc:
            raise OracleError("ring_all_gather", rc)
        return (ys, self._read_trace(tr, keep, n)) if trace else ys

    # -- halving-doubling ------------------------------------------------------
    def hd_allreduce(self, xs, dtype, rs_steps=-1, ag_steps=-1, trace=False, fault=None):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty_like(x) for x in xs]
        tr = keep = None
        if trace:
            tr, keep = self._make_trace(n, 2 * n * 8 + 8)
        rc = self._L.orc_hd_allreduce_steps(DTYPES[dtype], n, count, _ptrs(xs), _ptrs(ys), rs_steps, ag_steps,
                                            C.byref(tr) if trace else None, self._fault(fault))
        if rc:
            raise OracleError("hd_allreduce", rc)
        return (ys, self._read_trace(tr, keep, n)) if trace else ys

    def hd_reduce_scatter(self, xs, dtype, outer=1, trace=False, fault=None):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty(self.rs_len(count, n, outer, c), dtype=xs[0].dtype) for c in range(n)]
        tr = keep = None
        if trace:
            tr, keep = self._make_trace(n, n * 8 + 8)
        rc = self._L.orc_hd_reduce_scatter(DTYPES[dtype], n, count, outer, _ptrs(xs), _ptrs(ys),
                                           C.byref(tr) if trace else None, self._fault(fault))
        if rc:
            raise OracleError("hd_reduce_scatter", rc)
        return (ys, self._read_trace(tr, keep, n)) if trace else ys

    def hd_all_gather(self, xs, dtype, outer=1, trace=False, fault=None):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty(n * count, dtype=xs[0].dtype) for _ in range(n)]
        tr = keep = None
        if trace:
            tr, keep = self._make_trace(n, n * 8 + 8)
        rc = self._L.orc_hd_all_gather(DTYPES[dtype], n, count, outer, _ptrs(xs), _ptrs(ys),
                                       C.byref(tr) if trace else None, self._fault(fault))
        if rc:
            raise OracleError("hd_all_gather", rc)
        return (ys, self._read_trace(tr, keep, n)) if trace else ys

    # -- binomial tree ---------------------------------------------------------
    def tree_all_gather(self, xs, dtype, outer=1, trace=False, fault=None):
        """Binomial-tree all-gather: gather to rank 0, then broadcast from it
        (2 ceil(log2 N) steps, any N)."""
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty(n * count, dtype=xs[0].dtype) for _ in range(n)]
        tr = keep = None
        if trace:
            tr, keep = self._make_trace(n, 2 * n + 8)
        rc = self._L.orc_tree_all_gather(DTYPES[dtype], n, count, outer, _ptrs(xs), _ptrs(ys),
                                         C.byref(tr) if trace else None, self._fault(fault))
        if rc:
            raise OracleError("tree_all_gather", rc)
        return (ys, self._read_trace(tr, keep, n)) if trace else ys

    def hd_allreduce_at(self, xs, dtype, idx):
        xs = self._check_inputs(xs, dtype)
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty(idx.size, dtype=xs[0].dtype)
        rc = self._L.orc_hd_allreduce_at(DTYPES[dtype], len(xs), xs[0].size, _ptrs(xs), idx.ctypes.data,
                                         idx.size, out.ctypes.data)
        if rc:
            raise OracleError("hd_allreduce_at", rc)
        return out

    # -- fused (naive) reductions ---------------------------------------------
    def fused_allreduce(self, xs, dtype):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty_like(x) for x in xs]
        rc = self._L.orc_fused_allreduce(DTYPES[dtype], n, count, _ptrs(xs), _ptrs(ys))
        if rc:
            raise OracleError("fused_allreduce", rc)
        return ys

    def fused_reduce_scatter(self, xs, dtype, outer=1):
        xs = self._check_inputs(xs, dtype)
        n, count = len(xs), xs[0].size
        ys = [np.empty(self.rs_len(count, n, outer, c), dtype=xs[0].dtype) for c in range(n)]
        rc = self._L.orc_fused_reduce_scatter(DTYPES[dtype], n, count, outer, _ptrs(xs), _ptrs(ys))
        if rc:
            raise OracleError("fused_reduce_scatter", rc)
        return ys

    # -- per-element closed forms ---------------------------------------------
    def ring_allreduce_at(self, xs, dtype, idx):
        xs = self._check_inputs(xs, dtype)
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty(idx.size, dtype=xs[0].dtype)
        rc = self._L.orc_ring_allreduce_at(DTYPES[dtype], len(xs), xs[0].size, _ptrs(xs),
                                           idx.ctypes.data, idx.size, out.ctypes.data)
        if rc:
            raise OracleError("ring_allreduce_at", rc)
        return out

    def fused_allreduce_at(self, xs, dtype, idx):
        xs = self._check_inputs(xs, dtype)
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty(idx.size, dtype=xs[0].dtype)
        rc = self._L.orc_fused_allreduce_at(DTYPES[dtype], len(xs), xs[0].size, _ptrs(xs),
                                            idx.ctypes.data, idx.size, out.ctypes.data)
        if rc:
            raise OracleError("fused_allreduce_at", rc)
        return out

    # -- codecs, element add, partition ---------------------------------------
    def f32_to_f16_bits(self, f):
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.empty(f.size, dtype=np.uint16)
        self._L.orc_f32_to_f16(f.ctypes.data, out.ctypes.data, f.size)
        return out

    def f16_bits_to_f32(self, h):
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.size, dtype=np.float32)
        self._L.orc_f16_to_f32(h.ctypes.data, out.ctypes.data, h.size)
        return out

    def f32_to_bf16_bits(self, f):
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.empty(f.size, dtype=np.uint16)
        self._L.orc_f32_to_bf16(f.ctypes.data, out.ctypes.data, f.size)
        return out

    def bf16_bits_to_f32(self, b):
        b = np.ascontiguousarray(b, dtype=np.uint16)
        out = np.empty(b.size, dtype=np.float32)
        self._L.orc_bf16_to_f32(b.ctypes.data, out.ctypes.data, b.size)
        return out

    def add(self, a, b, dtype):
        a, b = self._check_inputs([a, b], dtype)
        out = np.empty_like(a)
        rc = self._L.orc_add(DTYPES[dtype], a.ctypes.data, b.ctypes.data, out.ctypes.data, a.size)
        if rc:
            raise OracleError("add", rc)
        return out

    def chunk_range(self, count, n, c):
        off, ln = C.c_uint64(), C.c_uint64()
        rc = self._L.orc_chunk_range(count, n, c, C.byref(off), C.byref(ln))
        if rc:
            raise OracleError("chunk_range", rc)
        return off.value, ln.value

    def rs_len(self, count, n, outer, c):
        """Elements of rank c's reduce-scatter output."""
        if outer == 1:
            return self.chunk_range(count, n, c)[1]
        return outer * ((count // outer) // n)


_DEFAULT: Oracle | None = None


def get() -> Oracle:
    """The oracle built from oracle.c in this directory (built on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
