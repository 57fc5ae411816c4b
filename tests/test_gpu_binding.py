"""The Python binding refuses tensors whose extents disagree before any launch.

The C ABI takes bare device pointers and cannot see a tensor's size, so the
binding checks every extent a kernel will index.  Each refusal below would
otherwise let a kernel read or write past the end of a tensor.  After the
refusals the same Buffer still gives the oracle's results."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from gen import random_case
from gpu_util import assert_bf16_close, dev, dev_bf16, f32_bits, host, host_bits

pytestmark = pytest.mark.gpu

import combine_get_dispatch_05_amd as epm  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-test] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _case():
    return random_case(31, 70, 256, 16, 4, 8, 4, mask=0.1, dup=0.0, slots=70)


def test_normal_path_refuses_mismatched_extents():
    inp = _case()
    E, R = inp.E, inp.R
    buf = epm.Buffer(R, E, inp.C)
    x, topk, w = dev_bf16(inp.x), dev(inp.topk_idx), dev(inp.topk_weights)
    with pytest.raises(ValueError, match="topk_weights"):
        buf.dispatch(x, topk, w[:, :-1].contiguous())
    with pytest.raises(ValueError, match="number of tokens"):
        buf.dispatch(x[:-1].contiguous(), topk, w)

    rx, rti, rtw, _, h, _ = buf.dispatch(x, topk, w)
    with pytest.raises(ValueError, match="topk_weights needs topk_idx"):
        buf.dispatch(x, None, w, handle=h)
    with pytest.raises(ValueError, match="topk_weights"):
        buf.combine(rx, h, rtw[:-1].contiguous())
    with pytest.raises(ValueError, match="topk_weights"):
        buf.combine(rx, h, rtw[:, :-1].contiguous())
    with pytest.raises(ValueError, match="bias"):
        buf.combine(rx, h, bias=x[:-1].contiguous())

    # the refusals left nothing behind: the same handle still combines right
    ora = oracle.layout(inp.topk_idx, E, R, inp.C)
    o_rx, _, o_rtw = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, E, R, ora)
    np.testing.assert_array_equal(host_bits(rx), o_rx)
    out, cw, _ = buf.combine(rx, h, rtw)
    o_out, o_cw = oracle.combine(o_rx, ora, o_rtw)
    assert_bf16_close(host_bits(out), o_out, what="combine after refusals")
    np.testing.assert_array_equal(f32_bits(host(cw)), f32_bits(o_cw))
    h.free()


def test_low_latency_refuses_mismatched_extents():
    inp = _case()
    E, R, S = inp.E, inp.R, inp.slots
    buf = epm.Buffer(R, E)
    x, topk, w = dev_bf16(inp.x), dev(inp.topk_idx), dev(inp.topk_weights)
    with pytest.raises(ValueError, match="number of tokens"):
        buf.low_latency_dispatch(x, topk[:-1].contiguous(), S, E)

    packed, _, hdl, _, _ = buf.low_latency_dispatch(x, topk, S, E)
    with pytest.raises(ValueError, match="shape"):
        buf.low_latency_combine(packed[:, :, :-1].contiguous(), topk, w, hdl)
    with pytest.raises(ValueError, match="shape"):
        buf.low_latency_combine(packed[:-1].contiguous(), topk, w, hdl)
    with pytest.raises(ValueError, match="topk_weights"):
        buf.low_latency_combine(packed, topk, w[:-1].contiguous(), hdl)
    with pytest.raises(ValueError, match="topk_slot"):
        buf.low_latency_combine(packed, topk[:-1].contiguous(), w[:-1].contiguous(), hdl)

    (q, sc), _, hdl8, _, _ = buf.low_latency_dispatch(x, topk, S, E, use_fp8=True)
    with pytest.raises(ValueError, match="codes"):
        buf.low_latency_combine((q.view(torch.uint8)[:, :, :-1].contiguous(),
                                 sc[:, :, :-1].contiguous()), topk, w, hdl8)
    with pytest.raises(ValueError, match="scales"):
        buf.low_latency_combine((q, sc[..., :-1].contiguous()), topk, w, hdl8)

    # a valid combine still matches the oracle
    y = packed.clone()
    out, _, _ = buf.low_latency_combine(y, topk, w, hdl)
    o_buf, _, _, _ = oracle.ll_dispatch(inp.x, inp.topk_idx, E, R, S)
    o_out = oracle.ll_combine(o_buf, inp.topk_idx, inp.topk_weights, E, R)
    assert_bf16_close(host_bits(out), o_out, what="ll combine after refusals")


def test_lb_refuses_mismatched_extents():
    n_exp, n_rep, P = 6, 5, 1024
    g = torch.Generator().manual_seed(5)
    ew = torch.randn(n_exp, P, generator=g).to(torch.bfloat16).cuda()
    rw = torch.zeros(n_rep, P, dtype=torch.bfloat16, device="cuda")
    mapping = torch.tensor([3, 0, 3, 5, 1], dtype=torch.int64, device="cuda")
    buf = epm.Buffer(2, 4)
    with pytest.raises(ValueError, match="one row per"):
        buf.lb_prefetch_weights(rw[:-1].contiguous(), ew, mapping)
    with pytest.raises(ValueError, match="same shape"):
        buf.lb_prefetch_weights(rw, ew[:, :-8].contiguous(), mapping)
    with pytest.raises(ValueError, match="one row per"):
        buf.lb_reduce_grads(rw, ew, mapping[:-1].contiguous())
    with pytest.raises(ValueError, match="same shape"):
        buf.lb_reduce_grads(rw[:, :-8].contiguous(), ew, mapping)

    buf.lb_prefetch_weights(rw, ew, mapping)
    np.testing.assert_array_equal(host_bits(rw), host_bits(ew)[mapping.cpu().numpy()])
