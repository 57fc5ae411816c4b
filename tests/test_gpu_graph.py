"""HIP graph capture of the launch-bound calls.

The low-latency decode step (dispatch + combine, with a device rank mask) and
the handle-reuse normal path (cached dispatch + combine) issue only kernel
launches, so they can be captured once and replayed.  Each replay here gets
new inputs written into the captured buffers (and, for the decode step, a
changed rank mask), with the program's own eager work and synchronizations in
between, and every replay is checked against the oracle.
"""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from gen import config_inputs, random_case, random_rows
from gpu_util import assert_bf16_close, dev, dev_bf16, host_bits

pytestmark = pytest.mark.gpu

import combine_get_dispatch_05_amd as epm  # noqa: E402
from combine_get_dispatch_05_amd import abi  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-test] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _eager_noise():
    a = torch.randn(1 << 20, device="cuda")
    (a * 2 + 1).sum().item()
    torch.cuda.synchronize()


def test_ll_decode_step_graph(ll_mode):
    base = config_inputs(3)
    E, R, S, T, H, K = base.E, base.R, base.slots, base.T, base.H, base.K
    epr = E // R
    L, P = abi.lib(), abi.ptr
    d = abi.dims(T, H, K, E, R, 1)
    x = dev_bf16(base.x)
    topk = dev(base.topk_idx)
    w = dev(base.topk_weights)
    mask = torch.zeros(R, dtype=torch.int32, device="cuda")
    packed = torch.empty((epr, R, S, H), dtype=torch.bfloat16, device="cuda")
    cnt = torch.empty((epr, R), dtype=torch.int32, device="cuda")
    src = torch.empty((epr, R, S), dtype=torch.int32, device="cuda")
    slot = torch.empty((T, K), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step():
        s = abi.current_stream()
        abi.check(L.ep_ll_dispatch(ctypes.byref(d), S, P(x), P(topk), P(mask), P(packed), P(cnt),
                                   P(src), P(slot), s), "ll dispatch")
        abi.check(L.ep_ll_combine(ctypes.byref(d), S, P(packed), P(topk), P(w), P(slot), P(mask),
                                  P(out), s), "ll combine")

    step()  # eager once before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i in range(4):
        inp = random_case(40 + i, T, H, E, K, R, 1, mask=0.05, slots=S)
        m = np.zeros(R, np.int32)
        if i % 2:
            m[[i, 2 * i + 7, R - 1]] = 1
        x.copy_(dev_bf16(inp.x))
        topk.copy_(dev(inp.topk_idx))
        w.copy_(dev(inp.topk_weights))
        s = abi.current_stream()
        abi.check(L.ep_mask_clean(P(mask), R, s), "mask clean")
        for r in np.nonzero(m)[0]:
            abi.check(L.ep_mask_update(P(mask), R, int(r), 1, s), "mask update")
        g.replay()
        torch.cuda.synchronize()
        o_buf, o_cnt, o_src, o_slot = oracle.ll_dispatch(inp.x, inp.topk_idx, E, R, S, rank_mask=m)
        np.testing.assert_array_equal(cnt.cpu().numpy(), o_cnt)
        np.testing.assert_array_equal(src.cpu().numpy(), o_src)
        np.testing.assert_array_equal(slot.cpu().numpy(), o_slot)
        o_out = oracle.ll_combine(o_buf, inp.topk_idx, inp.topk_weights, E, R, rank_mask=m)
        assert_bf16_close(host_bits(out), o_out, what=f"graph replay {i}")
        _eager_noise()


def test_cached_dispatch_and_combine_graph():
    inp = config_inputs(0)
    E, R, C, T, H, K = inp.E, inp.R, inp.C, inp.T, inp.H, inp.K
    L, P = abi.lib(), abi.ptr
    buf = epm.Buffer(R, E, C)
    _, _, rtw, _, h, _ = buf.dispatch(dev_bf16(inp.x), dev(inp.topk_idx), dev(inp.topk_weights))
    ora = oracle.layout(inp.topk_idx, E, R, C)
    _, _, o_rtw = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, E, R, ora)
    d = abi.dims(T, H, K, E, R, C)
    cap = int(L.ep_max_recv_rows(ctypes.byref(d)))   # worst case: no host sync inside
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    recv = torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    cw = torch.empty((T, K), dtype=torch.float32, device="cuda")
    raw = ctypes.c_void_p(h.raw.value)

    def step():
        s = abi.current_stream()
        abi.check(L.ep_dispatch(ctypes.byref(d), P(x), None, None, None, ctypes.byref(raw),
                                P(recv), None, None, cap, None, s), "cached dispatch")
        abi.check(L.ep_combine(raw, H, P(recv), cap, P(rtw), None, None, None, P(out), P(cw), s),
                  "combine")

    x.copy_(dev_bf16(inp.x))
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        xi = random_rows(T, H, 50 + i, tag=3)
        x.copy_(dev_bf16(xi))
        g.replay()
        torch.cuda.synchronize()
        o_rx, _, _ = oracle.dispatch(xi, None, None, E, R, ora, with_topk=False)
        np.testing.assert_array_equal(host_bits(recv[:ora.num_recv]), o_rx)
        o_out, o_cw = oracle.combine(o_rx, ora, o_rtw)
        assert_bf16_close(host_bits(out), o_out, what=f"graph replay {i}")
        np.testing.assert_array_equal(cw.cpu().numpy().view(np.uint32), o_cw.view(np.uint32))
        _eager_noise()
    h.free()
