"""The C ABI from plain C (tests/c/vrc_c_check.c): no Python binding, no
PyTorch, hipMalloc'd buffers and /opt/rocm's HIP runtime.  The binary is
built by __graft_entry__.build()."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "vrc_c_check")


def test_c_program_runs_every_mode():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build()"
    print("c abi check", flush=True)
    p = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.strip() == "ok"
