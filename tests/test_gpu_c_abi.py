"""The C ABI from a plain C program on the GPU: tests/c_abi/abi_check runs a
dispatch, reads the handle's layout and runs a combine, and checks each
result from its definition in C (no Python binding involved)."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "abi_check")


def test_plain_c_dispatch_and_combine():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with `python tests/c_abi/build.py` "
                    "(or __graft_entry__.build())")
    sys.__stderr__.write("\n[gpu-test] tests/c_abi/abi_check gpu\n")
    sys.__stderr__.flush()
    r = subprocess.run([EXE, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check gpu: ok" in r.stdout
