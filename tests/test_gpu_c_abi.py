"""The C ABI from plain C (tests/c/vrc_c_check.c): no Python binding, no
PyTorch, hipMalloc'd buffers and /opt/rocm's HIP runtime.  The binary is
built by __graft_entry__.build()."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "vrc_c_check")
CVT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "bf16_cvt_check")


def test_c_program_runs_every_mode():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build()"
    print("c abi check", flush=True)
    p = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.strip() == "ok"


def test_bf16_conversion_is_round_to_nearest_even_on_every_input():
    """The bf16 kernels round with the target's float -> bfloat16
    conversion; tests/c/bf16_cvt_check.hip compares it with the bit-level
    definition on all 2^32 binary32 inputs (NaNs, infinities, subnormals,
    ties)."""
    assert os.path.exists(CVT), f"{CVT} is missing: run __graft_entry__.build()"
    print("bf16 conversion check", flush=True)
    p = subprocess.run([CVT], capture_output=True, text=True, timeout=100)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.strip().endswith("mismatches 0 of 4294967296"), p.stdout
