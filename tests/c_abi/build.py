"""Build tests/c_abi/abi_check (plain C against include/ep.h and libep.so).

    python tests/c_abi/build.py

Test infrastructure: the binary finds libep.so through an $ORIGIN-relative
run path and the HIP runtime under /opt/rocm/lib.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_check.c")
BIN = os.path.join(HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "combine_get_dispatch_05_amd")
    tmp = BIN + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-o", tmp, SRC,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-L", pkg, "-lep", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../combine_get_dispatch_05_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.check_call(cmd)
    os.replace(tmp, BIN)  # a reader never sees a half-written binary
    return BIN


if __name__ == "__main__":
    print(build(), file=sys.stderr)
