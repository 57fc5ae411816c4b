"""The library's host code under AddressSanitizer.

libep.so is built again into a temporary package with AddressSanitizer on the
host side only (``-Xarch_host -fsanitize=address``; the gfx950 device code
is unchanged).  The CPU ABI tests then run against it in a child process with
clang's ASan runtime preloaded, since the interpreter is not instrumented.
They cover argument validation, the handle utilities, tuning and status
text, the host paths that run without a GPU.  Any out-of-bounds access or
use after free in that code ends the child with an error."""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_get_dispatch_05_amd")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_host_code_under_asan():
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as d:
        pkg = os.path.join(d, "combine_get_dispatch_05_amd")
        os.makedirs(pkg)
        for f in ("__init__.py", "abi.py", "buffer.py"):
            shutil.copy(os.path.join(PKG, f), pkg)
        srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))

        def compile_one(src):
            obj = os.path.join(d, os.path.basename(src)[:-4] + ".o")
            subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], check=True,
                           capture_output=True)
            return obj

        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            objs = list(ex.map(compile_one, srcs))
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-o", os.path.join(pkg, "libep.so"), *objs],
                       check=True, capture_output=True)
        preload = rt + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
        env = dict(os.environ, PYTHONPATH=os.pathsep.join([d, ROOT]), LD_PRELOAD=preload,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:"
                                "detect_odr_violation=0")
        # the child must load the sanitized copy, not the library in the tree
        which = subprocess.run([sys.executable, "-c", "from combine_get_dispatch_05_amd import abi; "
                                "print(abi.LIB_PATH)"], env=env, capture_output=True, text=True,
                               timeout=300, cwd=d)
        assert which.stdout.strip() == os.path.join(pkg, "libep.so"), which.stdout + which.stderr
        r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                                                                         "test_abi_cpu.py"),
                            "-q", "-p", "no:cacheprovider", "-k", "not plain_c_program and not probe",
                            "-m", "not gpu"],
                           env=env, capture_output=True, text=True, timeout=600, cwd=d)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out
    assert " passed" in r.stdout
