"""The oracle's C under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle is plain C with hand-written index arithmetic.  This test builds
it with both sanitizers and runs the quick pins in a child process, since the
interpreter itself is not instrumented and the ASan runtime must be loaded
first.  The quick pins reach every oracle function.  Any out-of-bounds
access, use of freed memory or undefined integer operation (overflow, bad
shift) ends the child with an error, and the pins must still pass."""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _gcc_runtime(name: str):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_under_asan_and_ubsan():
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "liboracle_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off",
                               "-fno-fast-math", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fPIC",
                               "-shared", "-o", so, SRC, "-lm"])
        code = "\n".join([
            "import ctypes, sys",
            f"sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]",
            "import oracle",
            f"oracle._lib = oracle._configure(ctypes.CDLL({so!r}))",
            "import test_oracle_mutants",
            "test_oracle_mutants.quick_pins()",
            "print('sanitized quick pins passed')",
        ])
        preload = asan + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
        env = dict(os.environ, LD_PRELOAD=preload,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=900)
    assert r.returncode == 0, (r.stdout[-2000:] + "\n" + r.stderr[-6000:])
    assert "sanitized quick pins passed" in r.stdout
