"""Pure-Python brute force for tiny ring collectives (a pin for the oracle).

It is written independently of ``oracle/oracle.c`` and in a different
formulation.  The oracle indexes chunks by formula ((r - s) mod N); this
module only follows the relay rule of the 4-card walkthrough on the page
hwcomputing.csdn.net/6a0dc11a10ee7a33f273f7fd.html, section "Ring 通信为什么常见":

* reduce-scatter: in the first step every rank hands the block with its own
  index to its successor; from then on a rank passes on the block it has just
  added into.  After N-1 steps each rank owns one complete block;
* all-gather: each rank first passes on the complete block it owns, then
  passes on whatever block it received last, for N-1 steps.

Element arithmetic comes from libraries, not from code of this project:
numpy's int32 (wrapping), float32 and float16 adds, and torch's CPU bfloat16
add.  Blocks follow the remainder rule of the custom all-gather listing on
ai6s.net/6a157e6510ee7a33f27553e9.html (equal blocks, the last one takes the
rest).
"""
from __future__ import annotations

import numpy as np
import torch


def _bf16_bits_to_torch(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy()).view(
        torch.bfloat16)


def _torch_bf16_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def storage_add(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """Element-wise a + b in the storage type, by library arithmetic."""
    if dtype == "int32":
        with np.errstate(over="ignore"):
            return (a.astype(np.int32) + b.astype(np.int32)).astype(np.int32)
    if dtype == "fp32":
        return (a.astype(np.float32) + b.astype(np.float32)).astype(np.float32)
    if dtype == "fp16":
        return (a.astype(np.float16) + b.astype(np.float16)).astype(np.float16)
    if dtype == "bf16":
        return _torch_bf16_to_bits(_bf16_bits_to_torch(a) + _bf16_bits_to_torch(b))
    raise ValueError(dtype)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored values to float32 (int32 to int64)."""
    if dtype == "int32":
        return x.astype(np.int64)
    if dtype == "bf16":
        return _bf16_bits_to_torch(x).float().numpy()
    return x.astype(np.float32)


def narrow(acc: np.ndarray, dtype: str) -> np.ndarray:
    """Round the float32 accumulator to the storage type (library RNE)."""
    if dtype == "int32":
        return ((acc + 2**31) % 2**32 - 2**31).astype(np.int32)
    if dtype == "fp32":
        return acc.astype(np.float32)
    if dtype == "fp16":
        return acc.astype(np.float32).astype(np.float16)
    if dtype == "bf16":
        return _torch_bf16_to_bits(torch.from_numpy(acc.astype(np.float32)).to(torch.bfloat16))
    raise ValueError(dtype)


def blocks(count: int, n: int) -> list[range]:
    base = count // n
    out = []
    for c in range(n):
        lo = c * base
        hi = count if c == n - 1 else lo + base
        out.append(range(lo, hi))
    return out


def column_blocks(count: int, n: int, outer: int) -> list[np.ndarray]:
    """Flat element indices of each column block of an [outer, count/outer] buffer."""
    row = count // outer
    w = row // n
    grid = np.arange(count).reshape(outer, row)
    return [grid[:, c * w:(c + 1) * w].reshape(-1) for c in range(n)]


def _block_index(blk) -> np.ndarray:
    return np.asarray(list(blk), dtype=np.int64) if isinstance(blk, range) else blk


def relay_reduce_scatter(xs: list[np.ndarray], dtype: str, blks) -> tuple[list[np.ndarray], list[int]]:
    """Run the reduce-scatter relay.  Returns the rank states and, for each
    rank, the block it owns completely at the end."""
    n = len(xs)
    state = [x.copy() for x in xs]
    passing = list(range(n))  # first step: rank r hands over block r
    for _ in range(n - 1):
        sent = [(r, passing[r], state[r][_block_index(blks[passing[r]])].copy()) for r in range(n)]
        nxt = [None] * n
        for src, blk, payload in sent:
            dst = (src + 1) % n
            ix = _block_index(blks[blk])
            state[dst][ix] = storage_add(state[dst][ix], payload, dtype)
            nxt[dst] = blk  # the receiver passes on what it just added into
        passing = nxt
    return state, passing


def relay_all_gather_blocks(state: list[np.ndarray], owned: list[int], blks) -> list[np.ndarray]:
    n = len(state)
    state = [s.copy() for s in state]
    passing = list(owned)
    for _ in range(n - 1):
        sent = [(r, passing[r], state[r][_block_index(blks[passing[r]])].copy()) for r in range(n)]
        nxt = [None] * n
        for src, blk, payload in sent:
            dst = (src + 1) % n
            state[dst][_block_index(blks[blk])] = payload
            nxt[dst] = blk
        passing = nxt
    return state


def ring_allreduce(xs: list[np.ndarray], dtype: str) -> list[np.ndarray]:
    n = len(xs)
    if n == 1:
        return [xs[0].copy()]
    blks = blocks(xs[0].size, n)
    state, owned = relay_reduce_scatter(xs, dtype, blks)
    return relay_all_gather_blocks(state, owned, blks)


def ring_reduce_scatter(xs: list[np.ndarray], dtype: str, outer: int = 1) -> list[np.ndarray]:
    """Rank c's output is the complete block c, taken from whichever rank owns it."""
    n = len(xs)
    count = xs[0].size
    blks = blocks(count, n) if outer == 1 else column_blocks(count, n, outer)
    if n == 1:
        return [xs[0][_block_index(blks[0])].copy()]
    state, owned = relay_reduce_scatter(xs, dtype, blks)
    out = [None] * n
    for r, blk in enumerate(owned):
        out[blk] = state[r][_block_index(blks[blk])].copy()
    return out


def all_gather(xs: list[np.ndarray], outer: int = 1) -> list[np.ndarray]:
    """Concatenation of every rank's [outer, row] input along the row axis."""
    cat = np.concatenate([x.reshape(outer, -1) for x in xs], axis=1).reshape(-1)
    return [cat.copy() for _ in xs]


def fused_fold(xs: list[np.ndarray], dtype: str) -> np.ndarray:
    """Left fold in rank order in float32 (int64 then wrap for int32), one rounding."""
    acc = widen(xs[0], dtype)
    for x in xs[1:]:
        acc = acc + widen(x, dtype)
        if dtype != "int32":
            acc = acc.astype(np.float32)
    return narrow(acc, dtype)


def fused_reduce_scatter(xs: list[np.ndarray], dtype: str, outer: int = 1) -> list[np.ndarray]:
    n = len(xs)
    count = xs[0].size
    blks = blocks(count, n) if outer == 1 else column_blocks(count, n, outer)
    full = fused_fold(xs, dtype)
    return [full[_block_index(blks[c])].copy() for c in range(n)]


# ---------------------------------------------------------------------------
# Halving-doubling, written recursively (divide and conquer over rank
# groups) rather than with the oracle's XOR partners: a group of 2m ranks
# sharing a block range splits it in two; the lower m ranks keep the lower
# half, the upper m ranks the upper half; lower rank k pairs with upper
# rank k and each adds the partner's copy of the half it keeps; then each
# half-group recurses on its half.  The all-gather undoes the recursion:
# each half-group first completes its half, then partners swap halves.
# ---------------------------------------------------------------------------
def _hd_rs(state, dtype, ranks, lo, hi, blks):
    if len(ranks) == 1:
        return
    m = len(ranks) // 2
    mid = (lo + hi) // 2
    lower, upper = ranks[:m], ranks[m:]
    lo_ix = np.concatenate([_block_index(blks[b]) for b in range(lo, mid)]) if mid > lo else np.zeros(0, np.int64)
    hi_ix = np.concatenate([_block_index(blks[b]) for b in range(mid, hi)]) if hi > mid else np.zeros(0, np.int64)
    sent = {}
    for a, b in zip(lower, upper):
        sent[(b, a)] = state[b][lo_ix].copy()  # upper sends the lower half to lower
        sent[(a, b)] = state[a][hi_ix].copy()  # lower sends the upper half to upper
    for a, b in zip(lower, upper):
        state[a][lo_ix] = storage_add(state[a][lo_ix], sent[(b, a)], dtype)
        state[b][hi_ix] = storage_add(state[b][hi_ix], sent[(a, b)], dtype)
    _hd_rs(state, dtype, lower, lo, mid, blks)
    _hd_rs(state, dtype, upper, mid, hi, blks)


def _hd_ag(state, ranks, lo, hi, blks):
    if len(ranks) == 1:
        return
    m = len(ranks) // 2
    mid = (lo + hi) // 2
    lower, upper = ranks[:m], ranks[m:]
    _hd_ag(state, lower, lo, mid, blks)
    _hd_ag(state, upper, mid, hi, blks)
    lo_ix = np.concatenate([_block_index(blks[b]) for b in range(lo, mid)]) if mid > lo else np.zeros(0, np.int64)
    hi_ix = np.concatenate([_block_index(blks[b]) for b in range(mid, hi)]) if hi > mid else np.zeros(0, np.int64)
    for a, b in zip(lower, upper):
        state[b][lo_ix] = state[a][lo_ix]
        state[a][hi_ix] = state[b][hi_ix]


def hd_allreduce(xs, dtype):
    n = len(xs)
    blks = blocks(xs[0].size, n)
    state = [x.copy() for x in xs]
    _hd_rs(state, dtype, list(range(n)), 0, n, blks)
    _hd_ag(state, list(range(n)), 0, n, blks)
    return state


def hd_reduce_scatter(xs, dtype, outer=1):
    n = len(xs)
    count = xs[0].size
    blks = blocks(count, n) if outer == 1 else column_blocks(count, n, outer)
    state = [x.copy() for x in xs]
    _hd_rs(state, dtype, list(range(n)), 0, n, blks)
    return [state[c][_block_index(blks[c])].copy() for c in range(n)]
