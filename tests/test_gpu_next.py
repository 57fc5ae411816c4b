"""HIP path against the oracle for the NEXT rows: low-latency rank masking,
combine bias terms, the FP8 low-latency dispatch and the load-balance
operations over redundant experts.  Integer / byte outputs bit-exact; bf16
reductions within 1 ulp (and equal, as both sides round the same sums)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pinlib
from gen import config_inputs, random_case, random_rows
from gpu_util import assert_bf16_close, dev, dev_bf16, host, host_bits

pytestmark = pytest.mark.gpu

import combine_get_dispatch_05_amd as epm  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-test] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


# ------------------------------------------------------------ rank masking


@pytest.mark.parametrize("case", ["decode", "random"])
def test_ll_rank_mask(case):
    if case == "decode":
        inp = config_inputs(3)
        masked = [3, 17, 31]
    else:
        inp = random_case(8, 50, 136, 16, 4, 8, 1, mask=0.1, dup=0.3, slots=60)
        masked = [1, 4, 5]
    E, R, S = inp.E, inp.R, inp.slots
    m = np.zeros(R, np.int32)
    m[masked] = 1
    buf = epm.Buffer(R, E)
    for r in masked:
        buf.low_latency_update_mask_buffer(r, mask=True)
    buf.low_latency_update_mask_buffer(0, mask=True)
    buf.low_latency_update_mask_buffer(0, mask=False)
    status = torch.empty(R, dtype=torch.int32)
    buf.low_latency_query_mask_buffer(status)
    np.testing.assert_array_equal(status.numpy(), m)

    x, topk, w = dev_bf16(inp.x), dev(inp.topk_idx), dev(inp.topk_weights)
    packed, count, hdl, _, _ = buf.low_latency_dispatch(x, topk, S, E)
    o_buf, o_cnt, o_src, o_slot = oracle.ll_dispatch(inp.x, inp.topk_idx, E, R, S, rank_mask=m)
    np.testing.assert_array_equal(host(count), o_cnt)
    np.testing.assert_array_equal(host(hdl.src_info), o_src)
    np.testing.assert_array_equal(host(hdl.topk_slot), o_slot)
    pk = host_bits(packed)
    used = np.minimum(o_cnt, S)
    for le in range(E // R):
        for r in range(R):
            np.testing.assert_array_equal(pk[le, r, :used[le, r]], o_buf[le, r, :used[le, r]])
    y = random_rows((E // R) * R * S, inp.H, 3, tag=13).reshape(E // R, R, S, inp.H)
    out, _, _ = buf.low_latency_combine(dev_bf16(y), topk, w, hdl)
    assert_bf16_close(host_bits(out), oracle.ll_combine(y, inp.topk_idx, inp.topk_weights, E, R,
                                                        rank_mask=m), what="masked ll combine")

    # mask cleared: dispatch everything; then a rank fails before the combine
    buf.low_latency_clean_mask_buffer()
    buf.low_latency_query_mask_buffer(status)
    assert int(status.sum()) == 0
    packed, count, hdl, _, _ = buf.low_latency_dispatch(x, topk, S, E)
    buf.low_latency_update_mask_buffer(masked[0], mask=True)
    cm = np.zeros(R, np.int32)
    cm[masked[0]] = 1
    out, _, _ = buf.low_latency_combine(dev_bf16(y), topk, w, hdl)
    assert_bf16_close(host_bits(out), oracle.ll_combine(y, inp.topk_idx, inp.topk_weights, E, R,
                                                        combine_mask=cm),
                      what="combine-time mask")


# -------------------------------------------------------------- combine bias


@pytest.mark.parametrize("cfg", [0, 1])
def test_combine_bias(cfg):
    inp = config_inputs(cfg)
    E, R, C, T, H = inp.E, inp.R, inp.C, inp.T, inp.H
    ora = oracle.layout(inp.topk_idx, E, R, C)
    buf = epm.Buffer(R, E, C)
    _, _, rtw, _, h, _ = buf.dispatch(dev_bf16(inp.x), dev(inp.topk_idx), dev(inp.topk_weights))
    y = random_rows(ora.num_recv, H, cfg, tag=12)
    b0 = random_rows(T, H, cfg, tag=21)
    b1 = random_rows(T, H, cfg, tag=22)
    o_rx, _, o_rtw = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, E, R, ora)
    yd = dev_bf16(y)
    for bias, ob in (((dev_bf16(b0), dev_bf16(b1)), (b0, b1)), (dev_bf16(b0), (b0, None))):
        out, cw, _ = buf.combine(yd, h, rtw, bias=bias)
        o_out, o_cw = oracle.combine(y, ora, o_rtw, bias0=ob[0], bias1=ob[1])
        assert_bf16_close(host_bits(out), o_out, what="combine with bias")
        np.testing.assert_array_equal(f32_bits(host(cw)), f32_bits(o_cw))
    h.free()


# ------------------------------------------------------------------- FP8 LL


@pytest.mark.parametrize("case", ["decode", "edge", "nonfinite", "masked"])
def test_ll_dispatch_fp8(case):
    if case == "decode":
        inp, m = config_inputs(3), None
    elif case == "edge":
        inp, m = pinlib.fp8_edge_case(), None
    elif case == "nonfinite":
        inp, m = pinlib.fp8_nonfinite_case(), None
    else:
        inp = random_case(4, 40, 1024, 16, 4, 4, 1, mask=0.2, slots=40)
        m = np.array([0, 1, 0, 0], np.int32)
    E, R, S = inp.E, inp.R, inp.slots
    buf = epm.Buffer(R, E)
    if m is not None:
        for r in np.nonzero(m)[0]:
            buf.low_latency_update_mask_buffer(int(r), mask=True)
    (q, sc), count, hdl, _, _ = buf.low_latency_dispatch(dev_bf16(inp.x), dev(inp.topk_idx), S, E,
                                                          use_fp8=True)
    assert q.dtype == torch.float8_e4m3fn
    o_q, o_sc, o_cnt, o_src, o_slot = oracle.ll_dispatch_fp8(inp.x, inp.topk_idx, E, R, S,
                                                             rank_mask=m)
    np.testing.assert_array_equal(host(count), o_cnt)
    np.testing.assert_array_equal(host(hdl.src_info), o_src)
    np.testing.assert_array_equal(host(hdl.topk_slot), o_slot)
    qh = q.view(torch.uint8).cpu().numpy()
    sch = sc.cpu().numpy()
    used = o_src >= 0
    # NaN codes: IEEE 754 leaves a NaN's sign open, so both 0x7F and 0xFF pass
    nan_o = pinlib.e4m3_is_nan(o_q)
    np.testing.assert_array_equal(pinlib.e4m3_is_nan(qh)[used], nan_o[used])
    np.testing.assert_array_equal(np.where(nan_o, 0x7F, qh)[used], np.where(nan_o, 0x7F, o_q)[used])
    np.testing.assert_array_equal(f32_bits(sch[used]), f32_bits(o_sc[used]))
    if case != "nonfinite":
        assert not nan_o[used].any()


# ------------------------------------------------------------ load balancing


def _mapping_from_large_config():
    inp = config_inputs(4, with_x=False)
    table = inp.extra["redundancy"]  # logical expert -> replica id or -1
    n_rep = int((table >= 0).sum())
    mapping = np.full(n_rep, -1, np.int64)
    for e, rep in enumerate(table):
        if rep >= 0:
            mapping[rep - (inp.E - n_rep)] = e
    return mapping, inp.E - n_rep


@pytest.mark.parametrize("P", [8, 2056, 4096 * 3 + 8])
def test_lb_ops(P):
    mapping, E = _mapping_from_large_config()
    # add a second replica of expert mapping[0], and an ignored entry
    mapping = np.concatenate([mapping, [mapping[0], -1, E + 5]]).astype(np.int64)
    n_rep = len(mapping)
    ew = random_rows(E, P, P, tag=31)
    rg = random_rows(n_rep, P, P, tag=32)
    buf = epm.Buffer(1, 1)
    mp = dev(mapping)
    # prefetch
    ewd = dev_bf16(ew)
    rwd = dev_bf16(random_rows(n_rep, P, P, tag=33))
    before = host_bits(rwd)
    buf.lb_prefetch_weights(rwd, ewd, mp)
    exp = oracle.lb_prefetch_weights(ew, before, mapping)
    np.testing.assert_array_equal(host_bits(rwd), exp)
    # reduce (in place)
    egd = dev_bf16(ew)
    buf.lb_reduce_grads(dev_bf16(rg), egd, mp)
    exp = oracle.lb_reduce_grads(rg, ew, mapping)
    assert_bf16_close(host_bits(egd), exp, what="lb_reduce_grads")
