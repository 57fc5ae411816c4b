"""Build libep.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc,
and libep_probe.so (the measurement kernels of include/ep_probe.h).

    python combine_get_dispatch_05_amd/build.py

(run it as a script: importing the package loads libep.so, which this builds)

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel), then all objects are linked into ``combine_get_dispatch_05_amd/libep.so``;
``probe/*.hip`` likewise into ``libep_probe.so``.  Packed-fp32 instructions are
switched off for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROBE = os.path.join(PKG, "probe")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libep.so")
PROBE_LIB = os.path.join(PKG, "libep_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def sources(d: str = CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _compile(src: str) -> str:
    sub = os.path.basename(os.path.dirname(src))
    obj = os.path.join(BUILD, sub + "_" + os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs, psrcs = sources(CSRC), sources(PROBE)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
