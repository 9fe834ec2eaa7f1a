"""Virtual-rank ring collectives on one MI355X: Python binding of include/vrc.h.

N virtual ranks are N equally sized device buffers in one GPU's HBM.  The
functions named like the C entry points (``vrc_allreduce``,
``vrc_reduce_scatter``, ``vrc_all_gather``) take lists of torch tensors, one
per rank, check shapes and marshal pointers, sizes and the current HIP
stream into the C ABI of ``libvrc.so``; every step of the computation runs in
that library's HIP kernels.  PyTorch only allocates memory and supplies the
stream.  The library must have been built (``ring_all_reduce_virtual_amd.build``);
importing the package fails loudly otherwise.

Modes: ``"ring"`` is the step-faithful ring (one launch per reduce-scatter
and per all-gather step), ``"fused"`` the single-launch N-way kernel,
``"ring_chained"`` the ring's per-step reads and writes in one launch, and
``"ring_order"`` one launch with fused traffic but the ring's summation order
(the three ring modes return the same bits), ``"hd"`` halving-doubling with
one launch per step and ``"hd_order"`` halving-doubling in one launch (both
need a power-of-two rank count and return the same bits); ``"select"`` picks
``"hd"`` for power-of-two rank counts with at most 64 MiB per rank and
``"ring"`` otherwise, and returns the bits of the one it picks.  ``"tree"``
is the binomial-tree all-gather (gather to rank 0, broadcast from it; the
all-gather only).
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvrc.so")

VRC_INT32, VRC_FP32, VRC_FP16, VRC_BF16 = 0, 1, 2, 3
VRC_SUM = 0
VRC_RING, VRC_FUSED, VRC_RING_CHAINED, VRC_RING_ORDER, VRC_HD, VRC_HD_ORDER, VRC_SELECT, VRC_TREE = range(8)
SELECT_HD_MAX_BYTES = 64 << 20  # VRC_SELECT_HD_MAX_BYTES of include/vrc.h
VRC_OK, VRC_ERR_INVALID_ARG, VRC_ERR_UNSUPPORTED, VRC_ERR_ALIAS, VRC_ERR_HIP = range(5)
MAX_RANKS = 16

MODES = {"ring": VRC_RING, "fused": VRC_FUSED, "ring_chained": VRC_RING_CHAINED, "ring_order": VRC_RING_ORDER,
         "hd": VRC_HD, "hd_order": VRC_HD_ORDER, "select": VRC_SELECT, "tree": VRC_TREE}
GATHER_ONLY_MODES = ("tree",)  # the all-reduce and reduce-scatter return VRC_ERR_UNSUPPORTED for these
REDUCE_MODES = {k: v for k, v in MODES.items() if k not in GATHER_ONLY_MODES}
RING_MODES = ("ring", "ring_chained", "ring_order")  # same bits as the per-step ring
HD_MODES = ("hd", "hd_order")  # halving-doubling; nranks must be a power of two


class VrcError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.vrc_status_string(status).decode()
        if status == VRC_ERR_HIP:
            msg += f" (hipError {_lib.vrc_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


ABI_VERSION = 106  # VRC_VERSION of include/vrc.h that these mirrors follow


class OpDesc(C.Structure):
    """One operation of a launch plan (vrc_op_desc in include/vrc.h)."""
    _fields_ = [("launch", C.c_int), ("kind", C.c_int), ("a", C.c_void_p), ("b", C.c_void_p), ("d", C.c_void_p),
                ("rows", C.c_size_t), ("width", C.c_size_t), ("stride_a", C.c_size_t), ("stride_b", C.c_size_t),
                ("stride_d", C.c_size_t), ("grid_x", C.c_uint), ("grid_y", C.c_uint), ("block", C.c_uint),
                ("vectors", C.c_uint)]


COLL_ALLREDUCE, COLL_REDUCE_SCATTER, COLL_ALL_GATHER, COLL_ALLREDUCE_BUCKETED = 0, 1, 2, 3
OP_KINDS = {0: "add", 1: "copy", 2: "fused_allreduce", 3: "fused_reduce_scatter", 4: "fused_all_gather",
            5: "chain_allreduce", 6: "chain_reduce_scatter", 7: "chain_all_gather", 8: "ring_order_allreduce",
            9: "ring_order_reduce_scatter", 10: "butterfly_allreduce", 11: "butterfly_reduce_scatter",
            12: "fused_allreduce_realigned", 13: "butterfly_allreduce_realigned",
            14: "ring_order_allreduce_realigned", 15: "fused_allreduce_phased", 16: "butterfly_allreduce_phased",
            17: "ring_order_allreduce_phased"}


def _load():
    # PyTorch-ROCm ships its own HIP runtime.  Import it first so that
    # libvrc.so binds to that same runtime (the dynamic linker reuses an
    # already-loaded libamdhip64 with a matching soname); loading libvrc.so
    # first would bring up a second HIP runtime that cannot see the device
    # memory torch allocates.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python ring_all_reduce_virtual_amd/build.py, or __graft_entry__.build())")
    L = C.CDLL(LIB_PATH)
    vp, sz, i = C.c_void_p, C.c_size_t, C.c_int
    ptrs = C.POINTER(C.c_void_p)
    L.vrc_allreduce.argtypes = [ptrs, ptrs, i, sz, i, i, i, vp]
    L.vrc_allreduce.restype = i
    L.vrc_reduce_scatter.argtypes = [ptrs, ptrs, i, sz, sz, i, i, i, vp]
    L.vrc_reduce_scatter.restype = i
    L.vrc_all_gather.argtypes = [ptrs, ptrs, i, sz, sz, i, i, vp]
    L.vrc_all_gather.restype = i
    L.vrc_allreduce_bucketed.argtypes = [ptrs, ptrs, i, sz, i, i, i, sz, ptrs, i, vp]
    L.vrc_allreduce_bucketed.restype = i
    L.vrc_plan.argtypes = [i, ptrs, ptrs, i, sz, sz, i, i, C.POINTER(OpDesc), i, C.POINTER(i), C.POINTER(i)]
    L.vrc_plan.restype = i
    L.vrc_chunk_range.argtypes = [sz, i, i, C.POINTER(sz), C.POINTER(sz)]
    L.vrc_chunk_range.restype = i
    L.vrc_status_string.argtypes = [i]
    L.vrc_status_string.restype = C.c_char_p
    L.vrc_last_hip_error.argtypes = []
    L.vrc_last_hip_error.restype = i
    L.vrc_version.argtypes = []
    L.vrc_version.restype = i
    if L.vrc_version() != ABI_VERSION:
        # OpDesc mirrors vrc_op_desc of this version; another layout would
        # be read (or written by vrc_plan) with the wrong size.
        raise ImportError(f"{LIB_PATH} reports ABI version {L.vrc_version()}, this binding needs {ABI_VERSION}: "
                          "rebuild the library")
    return L


_lib = _load()


def lib() -> C.CDLL:
    """The loaded libvrc.so."""
    return _lib


def _ptr_array(addrs):
    arr = (C.c_void_p * max(len(addrs), 1))()
    for k, a in enumerate(addrs):
        arr[k] = a
    return arr


# ---------------------------------------------------------------------------
# Raw C ABI mirrors: integer device addresses in, status out.
# ---------------------------------------------------------------------------
def raw_allreduce(send, recv, count, dtype, mode, stream=0, op=VRC_SUM) -> int:
    return _lib.vrc_allreduce(_ptr_array(send), _ptr_array(recv), len(send), count, dtype, op, mode,
                              stream or None)


def raw_reduce_scatter(send, recv, count, outer, dtype, mode, stream=0, op=VRC_SUM) -> int:
    return _lib.vrc_reduce_scatter(_ptr_array(send), _ptr_array(recv), len(send), count, outer, dtype, op,
                                   mode, stream or None)


def raw_all_gather(send, recv, count, outer, dtype, mode, stream=0) -> int:
    return _lib.vrc_all_gather(_ptr_array(send), _ptr_array(recv), len(send), count, outer, dtype, mode,
                               stream or None)


def raw_allreduce_bucketed(send, recv, count, dtype, mode, bucket, ready=(), stream=0, op=VRC_SUM) -> int:
    """`ready`: raw hipEvent_t handles, one per bucket, or empty for none."""
    events = _ptr_array(list(ready)) if ready else None
    return _lib.vrc_allreduce_bucketed(_ptr_array(send), _ptr_array(recv), len(send), count, dtype, op, mode, bucket,
                                       events, len(ready), stream or None)


def plan(coll: int, send, recv, count: int, outer: int, dtype: int, mode: int):
    """The operations a call would enqueue (host only, nothing launched):
    a list of dicts with launch, kind, a, b, d, rows, width, strides and the
    launch geometry (grid_x, grid_y, block, vectors) for a 256-CU device."""
    cap = 4096
    n_ops, n_launches = C.c_int(), C.c_int()
    while True:
        ops = (OpDesc * cap)()
        st = _lib.vrc_plan(coll, _ptr_array(send), _ptr_array(recv), len(send), count, outer, dtype, mode, ops, cap,
                           C.byref(n_ops), C.byref(n_launches))
        # A plan longer than `cap` reports its full length: ask again with room for all of it.
        if st == VRC_ERR_INVALID_ARG and n_ops.value > cap:
            cap = n_ops.value
            continue
        break
    if st != VRC_OK:
        raise VrcError(st, "vrc_plan")
    out = []
    for k in range(n_ops.value):
        o = ops[k]
        out.append({"launch": o.launch, "kind": OP_KINDS[o.kind], "a": o.a or 0, "b": o.b or 0, "d": o.d or 0,
                    "rows": o.rows, "width": o.width, "stride_a": o.stride_a, "stride_b": o.stride_b,
                    "stride_d": o.stride_d, "grid_x": o.grid_x, "grid_y": o.grid_y, "block": o.block,
                    "vectors": o.vectors})
    return out, n_launches.value


def chunk_range(count: int, nranks: int, chunk: int) -> tuple[int, int]:
    off, ln = C.c_size_t(), C.c_size_t()
    st = _lib.vrc_chunk_range(count, nranks, chunk, C.byref(off), C.byref(ln))
    if st != VRC_OK:
        raise VrcError(st, "vrc_chunk_range")
    return off.value, ln.value


def version() -> int:
    return _lib.vrc_version()


# ---------------------------------------------------------------------------
# Tensor-level binding (marshalling only).
# ---------------------------------------------------------------------------
def _torch():
    import torch  # imported lazily so the raw ABI needs no torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.int32: VRC_INT32, torch.float32: VRC_FP32, torch.float16: VRC_FP16,
             torch.bfloat16: VRC_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_ranks(tensors, what) -> int:
    """Validate one tensor per rank; return their device index.  One pass,
    with rank 0's attributes read once and device indices compared as ints:
    this check is most of the host cost of a small call."""
    if not isinstance(tensors, (list, tuple)) or not tensors:
        raise ValueError(f"{what}: expected a non-empty list of tensors, one per rank")
    if len(tensors) > MAX_RANKS:
        raise ValueError(f"{what}: at most {MAX_RANKS} ranks")
    t0 = tensors[0]
    if not t0.is_cuda:
        raise ValueError(f"{what}: tensors must live on the GPU")
    dtype, shape, dev = t0.dtype, t0.shape, t0.get_device()
    for t in tensors:
        if t.dtype is not dtype or t.shape != shape or t.get_device() != dev:
            raise ValueError(f"{what}: all ranks need the same dtype, shape and device")
        if not t.is_contiguous():
            raise ValueError(f"{what}: tensors must be contiguous")
    return dev


def _mode(mode) -> int:
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}")
    return MODES[mode]


def _stream(stream, device) -> int:
    """The HIP stream to enqueue on: the given one, else the current stream
    of the tensors' device (`device`: a torch.device or its index), which
    must be the current device, since the library launches on the current
    device.  torch's raw current-stream query, where it has one, returns the
    same handle as torch.cuda.current_stream(...).cuda_stream at a fraction
    of the cost."""
    torch = _torch()
    idx = device if isinstance(device, int) else device.index
    cur = torch.cuda.current_device()
    if idx is not None and idx != cur:
        raise ValueError(f"tensors live on cuda:{idx} but the current device is cuda:{cur}; "
                         "call inside torch.cuda.device(...)")
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(cur)
    return torch.cuda.current_stream(cur).cuda_stream


def _same_device(send, recv, what):
    if recv[0].device != send[0].device:
        raise ValueError(f"{what}: outputs must be on the inputs' device {send[0].device}")


def _outer(shape, dim) -> tuple[int, int]:
    """(product of the sizes before `dim`, `dim` made non-negative)."""
    nd = len(shape)
    if nd == 0:
        raise ValueError("tensors need at least one dimension")
    d = dim % nd
    outer = 1
    for k in shape[:d]:
        outer *= k
    return outer, d


def vrc_allreduce(send, recv=None, mode: str = "fused", stream=None):
    """recv[r] = sum over ranks of send[r] (every rank gets the sum).

    ``recv=None`` allocates outputs; ``recv=send`` runs in place.
    """
    torch = _torch()
    dev = _check_ranks(send, "vrc_allreduce")
    if recv is None:
        recv = [torch.empty_like(t) for t in send]
    elif recv is not send:  # in place (the same list) needs no second check
        _check_ranks(recv, "vrc_allreduce")
        if len(recv) != len(send) or recv[0].shape != send[0].shape or recv[0].dtype != send[0].dtype:
            raise ValueError("vrc_allreduce: recv must match send")
        _same_device(send, recv, "vrc_allreduce")
    st = raw_allreduce([t.data_ptr() for t in send], [t.data_ptr() for t in recv], send[0].numel(),
                       _dtype_code(send[0]), _mode(mode), _stream(stream, dev))
    if st != VRC_OK:
        raise VrcError(st, "vrc_allreduce")
    return recv


def bucket_count(count: int, bucket: int) -> int:
    """Number of buckets vrc_allreduce_bucketed cuts `count` elements into."""
    return 0 if count == 0 else (count - 1) // bucket + 1


def vrc_allreduce_bucketed(send, recv=None, bucket: int = 1 << 20, mode: str = "fused", ready=None, stream=None):
    """The all-reduce of `send` bucket by bucket (`bucket` elements per rank
    each, the last one smaller): bucket k's launches wait on ``ready[k]`` (a
    recorded torch.cuda.Event, e.g. marking that the compute stream has
    written bucket k of every rank), so the all-reduce of early buckets
    overlaps the computation of later ones."""
    torch = _torch()
    _check_ranks(send, "vrc_allreduce_bucketed")
    if recv is None:
        recv = [torch.empty_like(t) for t in send]
    _check_ranks(recv, "vrc_allreduce_bucketed")
    if len(recv) != len(send) or recv[0].shape != send[0].shape or recv[0].dtype != send[0].dtype:
        raise ValueError("vrc_allreduce_bucketed: recv must match send")
    _same_device(send, recv, "vrc_allreduce_bucketed")
    if bucket < 1:
        raise ValueError("vrc_allreduce_bucketed: bucket must be at least one element")
    handles = []
    if ready is not None:
        if len(ready) != bucket_count(send[0].numel(), bucket):
            raise ValueError("vrc_allreduce_bucketed: one event per bucket")
        handles = [e.cuda_event for e in ready]
        if not all(handles):
            raise ValueError("vrc_allreduce_bucketed: every event must have been recorded")
    st = raw_allreduce_bucketed([t.data_ptr() for t in send], [t.data_ptr() for t in recv], send[0].numel(),
                                _dtype_code(send[0]), _mode(mode), bucket, handles, _stream(stream, send[0].device))
    if st != VRC_OK:
        raise VrcError(st, "vrc_allreduce_bucketed")
    return recv


def reduce_scatter_shape(shape, nranks: int, dim: int = 0):
    """Output shape of rank c for the reduce-scatter of `shape` along `dim`.

    The last dimension of a flat (outer == 1) split may be uneven: the last
    rank takes the remainder, so its shape is returned separately."""
    outer, d = _outer(shape, dim)
    if outer == 1:
        count = 1
        for k in shape:
            count *= k
        return [(chunk_range(count, nranks, c)[1],) for c in range(nranks)]
    if shape[d] % nranks != 0:
        raise ValueError(f"dimension {dim} ({shape[d]}) is not divisible by {nranks} ranks")
    out = list(shape)
    out[d] = shape[d] // nranks
    return [tuple(out)] * nranks


def vrc_reduce_scatter(send, recv=None, dim: int = 0, mode: str = "fused", stream=None):
    """recv[c] = sum over ranks of chunk c of send[r].

    The chunks split dimension `dim` when the sizes before it multiply to
    more than one (``outer > 1``); otherwise the flat buffer is split into
    equal chunks with the remainder on the last rank (recv is then 1-D)."""
    torch = _torch()
    _check_ranks(send, "vrc_reduce_scatter")
    n = len(send)
    outer, _ = _outer(send[0].shape, dim)
    shapes = reduce_scatter_shape(tuple(send[0].shape), n, dim)
    if recv is None:
        recv = [torch.empty(shapes[c], dtype=send[0].dtype, device=send[0].device) for c in range(n)]
    if len(recv) != n:
        raise ValueError("vrc_reduce_scatter: one output per rank")
    for c, t in enumerate(recv):
        if t.numel() != _prod(shapes[c]) or t.dtype != send[0].dtype or not t.is_contiguous():
            raise ValueError(f"vrc_reduce_scatter: output {c} must be contiguous {shapes[c]} {send[0].dtype}")
        if t.device != send[0].device:
            raise ValueError(f"vrc_reduce_scatter: outputs must be on the inputs' device {send[0].device}")
    st = raw_reduce_scatter([t.data_ptr() for t in send], [t.data_ptr() for t in recv], send[0].numel(),
                            outer, _dtype_code(send[0]), _mode(mode), _stream(stream, send[0].device))
    if st != VRC_OK:
        raise VrcError(st, "vrc_reduce_scatter")
    return recv


def vrc_all_gather(send, recv=None, dim: int = 0, mode: str = "fused", stream=None):
    """recv[r] = concatenation of all send tensors along `dim`, for every rank."""
    torch = _torch()
    _check_ranks(send, "vrc_all_gather")
    n = len(send)
    outer, d = _outer(send[0].shape, dim)
    out_shape = list(send[0].shape)
    out_shape[d] *= n
    if recv is None:
        recv = [torch.empty(out_shape, dtype=send[0].dtype, device=send[0].device) for _ in range(n)]
    if len(recv) != n:
        raise ValueError("vrc_all_gather: one output per rank")
    for t in recv:
        if list(t.shape) != out_shape or t.dtype != send[0].dtype or not t.is_contiguous():
            raise ValueError(f"vrc_all_gather: outputs must be contiguous {out_shape} {send[0].dtype}")
        if t.device != send[0].device:
            raise ValueError(f"vrc_all_gather: outputs must be on the inputs' device {send[0].device}")
    st = raw_all_gather([t.data_ptr() for t in send], [t.data_ptr() for t in recv], send[0].numel(), outer,
                        _dtype_code(send[0]), _mode(mode), _stream(stream, send[0].device))
    if st != VRC_OK:
        raise VrcError(st, "vrc_all_gather")
    return recv


def all_reduce(tensors, mode: str = "fused", out=None, stream=None):
    """all_reduce(list of per-rank tensors, mode, out=None): ``vrc_allreduce``
    under the name of the tensor-parallel interface (``tp.all_reduce``)."""
    return vrc_allreduce(tensors, recv=out, mode=mode, stream=stream)


def reduce_scatter(tensors, dim: int = 0, mode: str = "fused", out=None, stream=None):
    """reduce_scatter(list of per-rank tensors, dim, mode): ``vrc_reduce_scatter``."""
    return vrc_reduce_scatter(tensors, recv=out, dim=dim, mode=mode, stream=stream)


def all_gather(tensors, dim: int = 0, mode: str = "fused", out=None, stream=None):
    """all_gather(list of per-rank tensors, dim, mode): ``vrc_all_gather``
    under the name of the tensor-parallel interface (``tp.all_gather``)."""
    return vrc_all_gather(tensors, recv=out, dim=dim, mode=mode, stream=stream)


def _prod(shape) -> int:
    p = 1
    for k in shape:
        p *= k
    return p


__all__ = [
    "plan", "OpDesc", "OP_KINDS", "COLL_ALLREDUCE", "COLL_REDUCE_SCATTER", "COLL_ALL_GATHER",
    "COLL_ALLREDUCE_BUCKETED", "vrc_allreduce", "vrc_reduce_scatter", "vrc_all_gather", "vrc_allreduce_bucketed",
    "all_reduce", "reduce_scatter", "all_gather", "bucket_count", "raw_allreduce_bucketed",
    "reduce_scatter_shape", "chunk_range",
    "version", "raw_allreduce", "raw_reduce_scatter", "raw_all_gather", "lib", "VrcError",
    "VRC_INT32", "VRC_FP32", "VRC_FP16", "VRC_BF16", "VRC_SUM", "VRC_RING", "VRC_FUSED", "VRC_RING_CHAINED",
    "VRC_RING_ORDER", "VRC_HD", "VRC_HD_ORDER", "VRC_SELECT", "VRC_TREE", "MODES", "REDUCE_MODES",
    "GATHER_ONLY_MODES", "RING_MODES", "HD_MODES", "VRC_OK",
    "VRC_ERR_INVALID_ARG", "VRC_ERR_UNSUPPORTED", "VRC_ERR_ALIAS", "VRC_ERR_HIP", "MAX_RANKS",
]
