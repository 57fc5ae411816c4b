"""CPU oracle for the expert-parallel layout / dispatch / combine path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does.  The
arithmetic lives in ``oracle.c`` (plain single-threaded C, built with gcc);
this module only marshals numpy arrays into it.  Nothing here shares code
with the HIP library.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math, no
    FP contraction: every rounding step is the one the C source spells out)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_f32_to_bf16.argtypes = [p, p, i64]
    lib.oracle_f32_to_bf16.restype = None
    lib.oracle_layout.argtypes = [i64] * 5 + [p] * 10 + [i64]
    lib.oracle_layout.restype = i64
    lib.oracle_dispatch.argtypes = [i64] * 5 + [p] * 8
    lib.oracle_dispatch.restype = None
    lib.oracle_combine.argtypes = [i64] * 4 + [p] * 9
    lib.oracle_combine.restype = None
    lib.oracle_ll_dispatch.argtypes = [i64] * 6 + [p] * 7
    lib.oracle_ll_dispatch.restype = ctypes.c_int
    lib.oracle_ll_combine.argtypes = [i64] * 6 + [p] * 6
    lib.oracle_ll_combine.restype = ctypes.c_int
    lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_e4m3_array.argtypes = [p, p, i64]
    lib.oracle_f32_to_e4m3_array.restype = None
    lib.oracle_ll_dispatch_fp8.argtypes = [i64] * 6 + [p] * 8
    lib.oracle_ll_dispatch_fp8.restype = ctypes.c_int
    lib.oracle_ll_combine_fp8.argtypes = [i64] * 6 + [p] * 7
    lib.oracle_ll_combine_fp8.restype = ctypes.c_int
    lib.oracle_lb_reduce_grads.argtypes = [i64] * 3 + [p] * 3
    lib.oracle_lb_reduce_grads.restype = None
    lib.oracle_lb_prefetch_weights.argtypes = [i64] * 3 + [p] * 3
    lib.oracle_lb_prefetch_weights.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns (round to nearest even)."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16(_ptr(f), _ptr(out), f.size)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Layout:
    num_tokens_per_rank: np.ndarray  # int32 [R]
    num_tokens_per_expert: np.ndarray  # int32 [E]
    is_token_in_rank: np.ndarray  # uint8 [T, R]
    rank_prefix_matrix: np.ndarray  # int32 [R]
    channel_prefix_matrix: np.ndarray  # int32 [R, C]
    recv_channel_prefix_matrix: np.ndarray  # int32 [R, C]
    send_head: np.ndarray  # int32 [T, R]
    recv_src_idx: np.ndarray  # int32 [N]

    @property
    def num_recv(self) -> int:
        return int(self.recv_src_idx.shape[0])


def layout(topk_idx: np.ndarray, E: int, R: int, C: int, rank_mask=None) -> Layout:
    """rank_mask: optional int32 [R], nonzero = masked rank (its slots act as
    masked slots)."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    m = _mask(rank_mask, R)
    T, K = topk_idx.shape
    cap = T * min(K, R)
    ntpr = np.empty(R, np.int32)
    ntpe = np.empty(E, np.int32)
    itr = np.empty((T, R), np.uint8)
    rpm = np.empty(R, np.int32)
    cpm = np.empty((R, C), np.int32)
    rcpm = np.empty((R, C), np.int32)
    sh = np.empty((T, R), np.int32)
    rsi = np.empty(max(cap, 1), np.int32)
    n = _load().oracle_layout(T, K, E, R, C, _ptr(topk_idx), _ptr(m), _ptr(ntpr), _ptr(ntpe), _ptr(itr),
                              _ptr(rpm), _ptr(cpm), _ptr(rcpm), _ptr(sh), _ptr(rsi), cap)
    if n < 0:
        raise ValueError("oracle_layout rejected its arguments")
    return Layout(ntpr, ntpe, itr, rpm, cpm, rcpm, sh, rsi[:n].copy())


def dispatch(x: np.ndarray, topk_idx, topk_weights, E: int, R: int, lay: Layout,
             with_topk: bool = True):
    """Returns (recv_x, recv_topk_idx, recv_topk_weights); topk outputs are None
    when ``with_topk`` is false (the handle-reuse dispatch)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, H = x.shape
    N = lay.num_recv
    recv_x = np.zeros((N, H), np.uint16)
    rti = rtw = None
    ti = tw = None
    K = 1
    if with_topk:
        ti = np.ascontiguousarray(topk_idx, dtype=np.int64)
        K = ti.shape[1]
        tw = np.ascontiguousarray(topk_weights, dtype=np.float32)
        rti = np.empty((N, K), np.int64)
        rtw = np.empty((N, K), np.float32)
    _load().oracle_dispatch(T, H, K, E, R, _ptr(x), _ptr(ti), _ptr(tw),
                            _ptr(lay.rank_prefix_matrix), _ptr(lay.send_head),
                            _ptr(recv_x), _ptr(rti), _ptr(rtw))
    return recv_x, rti, rtw


def combine(y: np.ndarray, lay: Layout, recv_topk_weights=None, K: int = 0, bias0=None,
            bias1=None, rank_mask=None):
    """Returns (out bf16 bits [T, H], combined_topk_weights [T, K] or None).
    bias0 / bias1: optional bf16 bits [T, H] added after the rank sum.
    rank_mask: optional int32 [R]; masked ranks are skipped."""
    y = np.ascontiguousarray(y, dtype=np.uint16)
    T, R = lay.send_head.shape
    H = y.shape[1]
    out = np.empty((T, H), np.uint16)
    cw = None
    rw = None
    if recv_topk_weights is not None:
        rw = np.ascontiguousarray(recv_topk_weights, dtype=np.float32)
        K = rw.shape[1]
        cw = np.empty((T, K), np.float32)
    b0 = None if bias0 is None else np.ascontiguousarray(bias0, dtype=np.uint16)
    b1 = None if bias1 is None else np.ascontiguousarray(bias1, dtype=np.uint16)
    for b in (b0, b1):
        assert b is None or b.shape == (T, H)
    m = _mask(rank_mask, R)
    _load().oracle_combine(T, H, max(K, 1), R, _ptr(y), _ptr(rw), _ptr(lay.rank_prefix_matrix),
                           _ptr(lay.send_head), _ptr(b0), _ptr(b1), _ptr(m), _ptr(out), _ptr(cw))
    return out, cw


def _mask(rank_mask, R):
    if rank_mask is None:
        return None
    m = np.ascontiguousarray(rank_mask, dtype=np.int32)
    assert m.shape == (R,)
    return m


def ll_dispatch(x: np.ndarray, topk_idx: np.ndarray, E: int, R: int, num_slots: int,
                with_buf: bool = True, rank_mask=None):
    """Returns (buf [E/R, R, slots, H] bits or None, counts [E/R, R],
    src_info [E/R, R, slots], topk_slot [T, K]).  rank_mask: int32 [R],
    nonzero = masked rank."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ti = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = ti.shape
    H = x.shape[1]
    epr = E // R
    buf = np.zeros((epr, R, num_slots, H), np.uint16) if with_buf else None
    counts = np.empty((epr, R), np.int32)
    src = np.empty((epr, R, num_slots), np.int32)
    ts = np.empty((T, K), np.int32)
    m = _mask(rank_mask, R)
    rc = _load().oracle_ll_dispatch(T, H, K, E, R, num_slots, _ptr(x), _ptr(ti), _ptr(m),
                                    _ptr(buf), _ptr(counts), _ptr(src), _ptr(ts))
    if rc != 0:
        raise ValueError("oracle_ll_dispatch rejected its arguments")
    return buf, counts, src, ts


def ll_combine(buf: np.ndarray, topk_idx: np.ndarray, topk_weights: np.ndarray, E: int, R: int,
               rank_mask=None, combine_mask=None):
    """rank_mask: the mask the dispatch used (slots); combine_mask: ranks
    masked at combine time (skipped)."""
    buf = np.ascontiguousarray(buf, dtype=np.uint16)
    epr, R2, num_slots, H = buf.shape
    assert R2 == R and epr == E // R
    ti = np.ascontiguousarray(topk_idx, dtype=np.int64)
    tw = np.ascontiguousarray(topk_weights, dtype=np.float32)
    T, K = ti.shape
    out = np.empty((T, H), np.uint16)
    m = _mask(rank_mask, R)
    cm = _mask(combine_mask, R)
    rc = _load().oracle_ll_combine(T, H, K, E, R, num_slots, _ptr(buf), _ptr(ti), _ptr(tw),
                                   _ptr(m), _ptr(cm), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_ll_combine rejected its arguments")
    return out


def ll_combine_fp8(q: np.ndarray, scale: np.ndarray, topk_idx: np.ndarray,
                   topk_weights: np.ndarray, E: int, R: int, rank_mask=None, combine_mask=None):
    """The LL combine of an FP8 payload: codes q [E/R, R, slots, H] (uint8)
    and per-128-block scales [E/R, R, slots, H/128] decoded in the sum."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sc = np.ascontiguousarray(scale, dtype=np.float32)
    epr, R2, num_slots, H = q.shape
    assert R2 == R and epr == E // R and sc.shape == (epr, R, num_slots, H // 128)
    ti = np.ascontiguousarray(topk_idx, dtype=np.int64)
    tw = np.ascontiguousarray(topk_weights, dtype=np.float32)
    T, K = ti.shape
    out = np.empty((T, H), np.uint16)
    m = _mask(rank_mask, R)
    cm = _mask(combine_mask, R)
    rc = _load().oracle_ll_combine_fp8(T, H, K, E, R, num_slots, _ptr(q), _ptr(sc), _ptr(ti),
                                       _ptr(tw), _ptr(m), _ptr(cm), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_ll_combine_fp8 rejected its arguments")
    return out


def e4m3_to_f32(code: int) -> float:
    return float(_load().oracle_e4m3_to_f32(int(code)))


def f32_to_e4m3(f: np.ndarray) -> np.ndarray:
    """fp32 -> FP8 E4M3 codes, round to nearest even, saturating at +-448."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint8)
    _load().oracle_f32_to_e4m3_array(_ptr(f), _ptr(out), f.size)
    return out


def ll_dispatch_fp8(x: np.ndarray, topk_idx: np.ndarray, E: int, R: int, num_slots: int,
                    rank_mask=None):
    """Returns (q [E/R, R, slots, H] uint8, scale [E/R, R, slots, H/128] fp32,
    counts, src_info, topk_slot).  Unused cells of q / scale are zero."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ti = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = ti.shape
    H = x.shape[1]
    epr = E // R
    q = np.zeros((epr, R, num_slots, H), np.uint8)
    sc = np.zeros((epr, R, num_slots, H // 128), np.float32)
    counts = np.empty((epr, R), np.int32)
    src = np.empty((epr, R, num_slots), np.int32)
    ts = np.empty((T, K), np.int32)
    m = _mask(rank_mask, R)
    rc = _load().oracle_ll_dispatch_fp8(T, H, K, E, R, num_slots, _ptr(x), _ptr(ti), _ptr(m),
                                        _ptr(q), _ptr(sc), _ptr(counts), _ptr(src), _ptr(ts))
    if rc != 0:
        raise ValueError("oracle_ll_dispatch_fp8 rejected its arguments")
    return q, sc, counts, src, ts


def lb_reduce_grads(redundant_grads: np.ndarray, expert_grads: np.ndarray,
                    mapping: np.ndarray) -> np.ndarray:
    """Returns new expert gradients (bf16 bits [E, P]); the input is not changed."""
    rg = np.ascontiguousarray(redundant_grads, dtype=np.uint16)
    eg = np.array(expert_grads, dtype=np.uint16, copy=True, order="C")
    mp = np.ascontiguousarray(mapping, dtype=np.int64)
    assert rg.shape == (len(mp), eg.shape[1])
    _load().oracle_lb_reduce_grads(len(mp), eg.shape[0], eg.shape[1], _ptr(rg), _ptr(eg), _ptr(mp))
    return eg


def lb_prefetch_weights(expert_weights: np.ndarray, redundant_weights: np.ndarray,
                        mapping: np.ndarray) -> np.ndarray:
    """Returns new replica weights (bf16 bits [n_rep, P])."""
    ew = np.ascontiguousarray(expert_weights, dtype=np.uint16)
    rw = np.array(redundant_weights, dtype=np.uint16, copy=True, order="C")
    mp = np.ascontiguousarray(mapping, dtype=np.int64)
    assert rw.shape == (len(mp), ew.shape[1])
    _load().oracle_lb_prefetch_weights(len(mp), ew.shape[0], ew.shape[1], _ptr(ew), _ptr(rw),
                                       _ptr(mp))
    return rw
