"""The memory-faithful single-launch ring must really issue the ring's reads.

The compiler may replace a load of a value the lane has just stored with the
stored register; results stay bit-exact, so no numerical test notices.  This
test compiles the chain kernels for gfx950 with the library's own flags and
counts the 16-byte global loads and stores in each: per vector the
all-reduce chain must read the N inputs, N-2 partials and N-1 relayed chunks
(3N-3) and store 2(N-1) times, the reduce-scatter chain 2(N-1) reads and N-1
stores, the all-gather relay N-1 reads and N stores.  No flat (address-space
generic) access may appear in any of them."""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
N = 8

SRC = f"""
#include "vrc_kernels.hpp"
template __global__ void vrc::k_fused_allreduce<vrc::BF16, {N}, 2, true, vrc::RankFold>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::F16, {N}, 2, true, vrc::RankFold>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::F32, {N}, 2, true, vrc::RankFold>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::I32, {N}, 2, true, vrc::RankFold>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::F32, {N}, 2, true, vrc::Butterfly>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::BF16, {N}, 1, true, vrc::RankFold, 64>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::F32, {N}, 1, true, vrc::Butterfly, 64>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::I32, 4, 2, true, vrc::RankFold, 64>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_allreduce<vrc::F16, 16, 1, true, vrc::RankFold, 64>(vrc::FusedArArgs);
template __global__ void vrc::k_fused_reduce_scatter<vrc::F32, {N}, true, vrc::RankFold>(vrc::FusedRsArgs);
template __global__ void vrc::k_fused_reduce_scatter_flat<vrc::BF16, {N}, true, vrc::RankFold, 64>(vrc::ChainArgs);
template __global__ void vrc::k_fused_reduce_scatter_flat<vrc::F32, {N}, true, vrc::Butterfly, 64>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_reduce_scatter_flat<vrc::BF16, {N}, false, true, 64>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_reduce_scatter_flat<vrc::F16, {N}, true, true, 64>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_allreduce<vrc::F32, {N}, false, true>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_allreduce<vrc::BF16, {N}, true, true>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_allreduce<vrc::BF16, {N}, false, true>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_allreduce<vrc::BF16, {N}, true, true, 64>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_allreduce<vrc::F32, {N}, false, true, 64>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_reduce_scatter<vrc::F16, {N}, true, true>(vrc::ChainArgs);
template __global__ void vrc::k_ring_chain_all_gather<vrc::F32, {N}, true>(vrc::FusedAgArgs);
template __global__ void vrc::k_ring_step<vrc::BF16, true, true, 8>(vrc::StepArgsK<8>);
template __global__ void vrc::k_ring_step<vrc::F32, true, false, 8>(vrc::StepArgsK<8>);
"""


def builder():
    spec = importlib.util.spec_from_file_location("_vrc_build", os.path.join(ROOT, "ring_all_reduce_virtual_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    b = builder()
    if not shutil.which(b.HIPCC) and not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("codegen")
    src, out = d / "chain.hip", d / "chain.s"
    src.write_text(SRC)
    flags = [f for f in b.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([b.HIPCC, *flags, "--cuda-device-only", "-S", "-I", b.INCLUDE, "-I", b.CSRC, "-o", str(out),
                    str(src)], check=True, capture_output=True)
    return out.read_text()


def body(asm_text, pattern):
    m = re.search(r"^(_ZN3vrc\w*" + pattern + r"\w*):[^\n]*\n(.*?)^\.Lfunc_end", asm_text, re.S | re.M)
    assert m, f"kernel {pattern} not found"
    return m.group(2)


def count(text, op):
    return len(re.findall(r"^\s*" + op + r"\b", text, re.M))


@pytest.mark.parametrize("pattern,loads,stores", [
    (r"k_ring_chain_allreduceINS_4BF16ELi8ELb1ELb1ELi256", 3 * N - 3, 2 * (N - 1)),
    (r"k_ring_chain_allreduceINS_4BF16ELi8ELb0ELb1ELi256", N, N),
    (r"k_ring_chain_allreduceINS_4BF16ELi8ELb1ELb1ELi64", 3 * N - 3, 2 * (N - 1)),
    (r"k_ring_chain_allreduceINS_3F32ELi8ELb0ELb1ELi64", N, N),
    (r"k_ring_chain_reduce_scatterINS_3F16ELi8ELb1", 2 * (N - 1), N - 1),
    (r"k_ring_chain_reduce_scatter_flatINS_3F16ELi8ELb1", 2 * (N - 1), N - 1),
    (r"k_ring_chain_all_gatherINS_3F32ELi8", N - 1, N),
])
def test_chain_kernels_issue_every_access(asm, pattern, loads, stores):
    text = body(asm, pattern)
    assert count(text, "global_load_dwordx4") == loads
    assert count(text, "global_store_dwordx4") == stores
    assert count(text, r"flat_(load|store)\w*") == 0


def longest_load_run(text):
    """Longest run of 16-byte global loads with no wait on the vector memory counter between them."""
    best = run = 0
    for line in text.splitlines():
        line = line.strip()
        if re.match(r"global_load_dwordx4\b", line):
            run += 1
            best = max(best, run)
        elif re.match(r"s_waitcnt\b.*vmcnt", line):
            run = 0
    return best


@pytest.mark.parametrize("pattern,loads", [
    (r"k_fused_allreduceINS_4BF16ELi8ELi2ELb1ENS_8RankFold", 2 * N),
    (r"k_fused_allreduceINS_3F16ELi8ELi2ELb1ENS_8RankFold", 2 * N),
    (r"k_fused_allreduceINS_3F32ELi8ELi2ELb1ENS_8RankFold", 2 * N),
    (r"k_fused_allreduceINS_3I32ELi8ELi2ELb1ENS_8RankFold", 2 * N),
    (r"k_fused_allreduceINS_3F32ELi8ELi2ELb1ENS_9Butterfly", 2 * N),
    (r"k_fused_allreduceINS_4BF16ELi8ELi1ELb1ENS_8RankFoldELi64", N),
    (r"k_fused_allreduceINS_3F32ELi8ELi1ELb1ENS_9ButterflyELi64", N),
    (r"k_fused_allreduceINS_3I32ELi4ELi2ELb1ENS_8RankFoldELi64", 8),
    (r"k_fused_allreduceINS_3F16ELi16ELi1ELb1ENS_8RankFoldELi64", 16),
    (r"k_fused_reduce_scatterINS_3F32ELi8ELb1ENS_8RankFold", N),
    (r"k_fused_reduce_scatter_flatINS_4BF16ELi8ELb1ENS_8RankFoldELi64", N),
    (r"k_fused_reduce_scatter_flatINS_3F32ELi8ELb1ENS_9ButterflyELi64", N),
    (r"k_ring_chain_reduce_scatter_flatINS_4BF16ELi8ELb0ELb1ELi64", N),
    (r"k_ring_chain_reduce_scatter_flatINS_3F16ELi8ELb1ELb1ELi64", N),
    (r"k_ring_chain_allreduceINS_3F32ELi8ELb0ELb1ELi256", N),
    (r"k_ring_chain_allreduceINS_4BF16ELi8ELb1ELb1ELi256", N),
    (r"k_ring_chain_allreduceINS_3F32ELi8ELb0ELb1ELi64", N),
    (r"k_ring_chain_allreduceINS_4BF16ELi8ELb1ELb1ELi64", N),
    (r"k_ring_chain_reduce_scatterINS_3F16ELi8ELb1", N),
    (r"k_ring_stepINS_4BF16ELb1ELb1ELi8", 2),
    (r"k_ring_stepINS_3F32ELb1ELb0ELi8", 2),
])
def test_single_pass_kernels_keep_all_loads_in_flight(asm, pattern, loads):
    """Every lane issues all of its loads (N per vector per rank it keeps in
    flight) before it waits for the first one.  A compiler that interleaves the fold with
    the loads leaves two in flight and runs the 8 x 512 MiB fused all-reduce
    at 3.8 TB/s instead of 5.4.  A ring step's chunk-add has both of its
    operands in flight together."""
    assert longest_load_run(body(asm, pattern)) >= loads