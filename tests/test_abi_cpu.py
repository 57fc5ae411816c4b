"""The C ABI without a GPU: the library loads, exports exactly what
include/ep.h declares, and rejects bad arguments before touching the device.
No call here reaches a HIP runtime call."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")

from combine_get_dispatch_05_amd import abi  # noqa: E402

L = abi.lib()
S = None  # NULL stream; never used by these calls


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_0-9]+)\s*\(", text)))


def test_every_header_is_checked():
    """include/ holds the library's ABI and the measurement probes' ABI."""
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["ep.h", "ep_probe.h"]


def test_probe_header_matches_its_binding_and_library():
    from combine_get_dispatch_05_amd import probe_abi
    hdr = os.path.join(ROOT, "include", "ep_probe.h")
    assert declared_functions(hdr) == sorted(probe_abi.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", probe_abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    P = probe_abi.lib()
    for name in probe_abi.EXPORTS:
        assert name in exported, name
    # argument checks run before anything touches the device
    assert P.ep_probe_write(None, 16, None) == abi.EP_ERR_INVALID
    assert P.ep_probe_write(ctypes.c_void_p(0x1008), 16, None) == abi.EP_ERR_ALIGN
    assert P.ep_probe_empty(0, 64, None) == abi.EP_ERR_INVALID
    assert P.ep_probe_empty(1, 65, None) == abi.EP_ERR_INVALID
    assert P.ep_probe_pack(None, 4, 8, None, 1, None, None) == abi.EP_ERR_INVALID
    assert P.ep_probe_ll_copy(ctypes.c_void_p(0x1000), 4, 12, 2, ctypes.c_void_p(0x1000),
                              None) == abi.EP_ERR_ALIGN


def test_header_matches_binding():
    assert declared_functions() == sorted(abi.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(abi, "LIB_PATH", "/nonexistent/libep.so")
    with pytest.raises(ImportError):
        abi._load()


def test_product_package_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "combine_get_dispatch_05_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+(oracle|gen)\b", src, re.M), f
                assert "liboracle" not in src, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            src = open(os.path.join(ROOT, "oracle", f)).read()
            assert "combine_get_dispatch_05_amd" not in src and "libep" not in src, f


def test_version_and_status_text():
    assert abi.version() == (2, 4)
    for code in range(8):
        assert L.ep_status_str(code)
    assert L.ep_status_str(99) == b"unknown status"


def test_max_recv_rows():
    assert L.ep_max_recv_rows(ctypes.byref(abi.dims(4096, 7168, 8, 256, 64, 10))) == 4096 * 8
    assert L.ep_max_recv_rows(ctypes.byref(abi.dims(128, 256, 4, 16, 2, 4))) == 128 * 2
    assert L.ep_max_recv_rows(ctypes.byref(abi.dims(10, 7168, 8, 255, 64, 10))) == -1


@pytest.mark.parametrize("dims,code", [
    ((-1, 64, 2, 8, 4, 1), abi.EP_ERR_INVALID),
    ((8, 0, 2, 8, 4, 1), abi.EP_ERR_INVALID),
    ((8, 12, 2, 8, 4, 1), abi.EP_ERR_ALIGN),       # a row is not whole 16-byte vectors
    ((8, 64, 0, 8, 4, 1), abi.EP_ERR_INVALID),
    ((8, 64, 65, 128, 4, 1), abi.EP_ERR_INVALID),
    ((8, 64, 2, 10, 4, 1), abi.EP_ERR_INVALID),   # E not a multiple of R
    ((8, 64, 2, 1024, 1024, 1), abi.EP_ERR_INVALID),  # R above 512
    ((8, 64, 2, 8, 4, 0), abi.EP_ERR_INVALID),
    ((8, 64, 2, 8, 4, 5000), abi.EP_ERR_INVALID),
])
def test_dims_rejected(dims, code):
    d = abi.dims(*dims)
    h = ctypes.c_void_p()
    rc = L.ep_dispatch(ctypes.byref(d), None, None, None, None, ctypes.byref(h), None, None, None,
                       0, None, S)
    assert rc == code
    assert h.value is None
    rc = L.ep_get_dispatch_layout(ctypes.byref(d), None, None, None, ctypes.byref(h), S)
    assert rc == code


def test_argument_rules_rejected_before_device_work():
    d = abi.dims(16, 64, 2, 8, 4, 1)
    h = ctypes.c_void_p()
    hp = ctypes.byref(h)
    fake = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10008)  # 8-byte aligned, not 16

    def disp(x, topk, w, mask, handle, recv_x, rw, cap):
        # (dims, x, topk_idx, topk_weights, rank_mask, handle, recv_x,
        #  recv_topk_idx, recv_topk_weights, recv_cap, num_recv, stream)
        return L.ep_dispatch(ctypes.byref(d), x, topk, w, mask, handle, recv_x, None, rw, cap,
                             None, S)

    assert disp(fake, fake, None, None, None, fake, None, 64) == abi.EP_ERR_INVALID  # no handle slot
    assert disp(mis, fake, None, None, hp, fake, None, 64) == abi.EP_ERR_ALIGN  # misaligned x
    assert disp(fake, fake, None, None, hp, mis, None, 64) == abi.EP_ERR_ALIGN  # misaligned recv_x
    assert disp(fake, ctypes.c_void_p(0x10004), None, None, hp, fake, None,
                64) == abi.EP_ERR_ALIGN  # misaligned topk_idx
    assert disp(fake, fake, None, ctypes.c_void_p(0x10002), hp, fake, None,
                64) == abi.EP_ERR_ALIGN  # misaligned rank mask
    assert disp(None, fake, None, None, hp, fake, None, 64) == abi.EP_ERR_INVALID  # recv_x, no x
    assert disp(fake, fake, None, None, hp, fake, fake,
                64) == abi.EP_ERR_INVALID  # recv weights without topk weights
    assert disp(fake, None, None, None, hp, fake, None, 64) == abi.EP_ERR_INVALID  # no routing
    assert disp(fake, fake, None, None, hp, fake, None, -1) == abi.EP_ERR_INVALID  # capacity < 0
    assert h.value is None
    # layout with nothing to produce; misaligned rank mask
    assert L.ep_get_dispatch_layout(ctypes.byref(d), fake, None, None, None, S) == abi.EP_ERR_INVALID
    assert L.ep_get_dispatch_layout(ctypes.byref(d), fake, ctypes.c_void_p(0x10002), None, hp,
                                    S) == abi.EP_ERR_ALIGN
    # combine: misaligned rank mask is refused before the handle is used
    assert L.ep_combine(ctypes.c_void_p(0x10000), 64, fake, 0, None, None, None,
                        ctypes.c_void_p(0x10002), fake, None, S) == abi.EP_ERR_ALIGN


def test_combine_and_handle_calls_without_handle():
    assert L.ep_combine(None, 64, None, 0, None, None, None, None, None, None,
                        S) == abi.EP_ERR_HANDLE
    n = ctypes.c_int64()
    assert L.ep_handle_num_recv(None, ctypes.byref(n)) == abi.EP_ERR_HANDLE
    assert L.ep_handle_copy_layout(None, None, S) == abi.EP_ERR_HANDLE
    assert L.ep_handle_dims(None, None) == abi.EP_ERR_HANDLE
    assert L.ep_handle_nbytes(None) == 0
    L.ep_handle_free(None)  # no-op


def test_low_latency_rules():
    d = abi.dims(129, 64, 2, 8, 4, 1)
    fake = ctypes.c_void_p(0x10000)
    # more tokens than slots per (local expert, rank)
    assert L.ep_ll_dispatch(ctypes.byref(d), 128, fake, fake, None, fake, fake, fake, fake,
                            S) == abi.EP_ERR_CAPACITY
    assert L.ep_ll_combine(ctypes.byref(d), 128, fake, fake, fake, fake, None, fake,
                           S) == abi.EP_ERR_CAPACITY
    d = abi.dims(16, 64, 2, 8, 4, 1)
    assert L.ep_ll_dispatch(ctypes.byref(d), 0, fake, fake, None, fake, fake, fake, fake,
                            S) == abi.EP_ERR_INVALID
    assert L.ep_ll_dispatch(ctypes.byref(d), 5000, fake, fake, None, fake, fake, fake, fake,
                            S) == abi.EP_ERR_INVALID
    # missing metadata outputs
    assert L.ep_ll_dispatch(ctypes.byref(d), 16, fake, fake, None, fake, None, fake, fake,
                            S) == abi.EP_ERR_INVALID
    # misaligned packed buffer / mask
    assert L.ep_ll_dispatch(ctypes.byref(d), 16, fake, fake, None, ctypes.c_void_p(0x10008), fake,
                            fake, fake, S) == abi.EP_ERR_ALIGN
    assert L.ep_ll_dispatch(ctypes.byref(d), 16, fake, fake, ctypes.c_void_p(0x10002), fake, fake,
                            fake, fake, S) == abi.EP_ERR_ALIGN
    assert L.ep_ll_combine(ctypes.byref(d), 16, fake, fake, fake, fake, None, None,
                           S) == abi.EP_ERR_INVALID
    # FP8: rows must be whole 128-element blocks; scales required
    assert L.ep_ll_dispatch_fp8(ctypes.byref(d), 16, fake, fake, None, fake, fake, fake, fake,
                                fake, S) == abi.EP_ERR_ALIGN
    d = abi.dims(16, 128, 2, 8, 4, 1)
    assert L.ep_ll_dispatch_fp8(ctypes.byref(d), 16, fake, fake, None, fake, None, fake, fake,
                                fake, S) == abi.EP_ERR_INVALID


def test_mask_and_load_balance_rules():
    fake = ctypes.c_void_p(0x10000)
    assert L.ep_mask_update(None, 4, 0, 1, S) == abi.EP_ERR_INVALID
    assert L.ep_mask_update(fake, 4, 4, 1, S) == abi.EP_ERR_INVALID
    assert L.ep_mask_update(fake, 4, -1, 1, S) == abi.EP_ERR_INVALID
    assert L.ep_mask_clean(fake, 0, S) == abi.EP_ERR_INVALID
    assert L.ep_mask_query(fake, 4, None, S) == abi.EP_ERR_INVALID
    assert L.ep_mask_update(ctypes.c_void_p(0x10002), 4, 1, 1, S) == abi.EP_ERR_ALIGN
    for fn in (L.ep_lb_reduce_grads, L.ep_lb_prefetch_weights):
        assert fn(fake, fake, fake, 4, 8, 12, S) == abi.EP_ERR_ALIGN      # rows not 16-byte vectors
        assert fn(fake, fake, fake, -1, 8, 16, S) == abi.EP_ERR_INVALID
        assert fn(fake, fake, fake, 70000, 8, 16, S) == abi.EP_ERR_INVALID
        assert fn(None, fake, fake, 4, 8, 16, S) == abi.EP_ERR_INVALID
        assert fn(fake, fake, ctypes.c_void_p(0x10004), 4, 8, 16, S) == abi.EP_ERR_ALIGN


@pytest.mark.parametrize("op", ["ll", "layout"])
def test_path_tuning_modes(op):
    assert abi.tunings(op) == [(0, 0, 0), (1, 0, 0), (2, 0, 0)]
    assert L.ep_set_tuning(op.encode(), 3, 0, 0) == abi.EP_ERR_INVALID
    assert L.ep_set_tuning(op.encode(), 1, 1, 0) == abi.EP_ERR_INVALID
    assert L.ep_set_tuning(op.encode(), 2, 0, 0) == abi.EP_OK
    abi.set_tuning(op)  # back to automatic


def test_plain_c_program_uses_the_abi():
    """include/ep.h and libep.so from a C program (no Python binding): static
    calls and argument validation."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_abi_build",
                                                  os.path.join(ROOT, "tests", "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "abi_check cpu: ok" in r.stdout


def test_noalloc_layout_rules_without_device():
    """ep_get_dispatch_layout_noalloc refuses bad arguments, short buffers
    and problems beyond its static scratch before any device call."""
    d = abi.dims(16, 64, 2, 8, 4, 1)
    fake = ctypes.c_void_p(0x10000)
    f = L.ep_get_dispatch_layout_noalloc
    assert f(ctypes.byref(d), fake, None, None, S) == abi.EP_ERR_INVALID  # out is required
    o = abi.LayoutOut()
    assert f(ctypes.byref(d), None, None, ctypes.byref(o), S) == abi.EP_ERR_INVALID  # no table
    o = abi.LayoutOut(None, None, None, None, None, None, 0x10004, None, 0)
    assert f(ctypes.byref(d), fake, None, ctypes.byref(o), S) == abi.EP_ERR_ALIGN  # send_head
    o = abi.LayoutOut(None, None, 0x10002, None, None, None, None, None, 0)
    assert f(ctypes.byref(d), fake, None, ctypes.byref(o), S) == abi.EP_ERR_ALIGN  # membership
    o = abi.LayoutOut(None, None, None, None, None, None, None, 0x10000, 31)
    assert f(ctypes.byref(d), fake, None, ctypes.byref(o), S) == abi.EP_ERR_CAPACITY  # 32 rows
    big = abi.dims(1 << 20, 64, 8, 512, 512, 1)  # [T][R] alone is 512 MiB
    o = abi.LayoutOut()
    assert f(ctypes.byref(big), fake, None, ctypes.byref(o), S) == abi.EP_ERR_TOO_LARGE
    assert L.ep_status_str(abi.EP_ERR_TOO_LARGE).startswith(b"problem needs more")
