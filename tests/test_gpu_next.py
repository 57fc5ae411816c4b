"""HIP path against the oracle for the NEXT rows: low-latency rank masking,
combine bias terms, the FP8 low-latency dispatch and the load-balance
operations over redundant experts.  Integer / byte outputs bit-exact; bf16
reductions within 1 ulp (and equal, as both sides round the same sums)."""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import pinlib
from gen import config_inputs, random_case, random_rows
from gpu_util import assert_bf16_close, compare_layout, dev, dev_bf16, f32_bits, host, host_bits

pytestmark = pytest.mark.gpu

import combine_get_dispatch_05_amd as epm  # noqa: E402
from combine_get_dispatch_05_amd import abi  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-test] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------ rank masking


@pytest.mark.parametrize("case", ["decode", "random", "random_two_rounds"])
def test_ll_rank_mask(case, ll_mode):
    if case == "decode":
        inp = config_inputs(3)
        masked = [3, 17, 31]
    elif case == "random_two_rounds":
        # T*K = 10000 top-k entries: the slot scan reads the table in two rounds
        inp = random_case(9, 2500, 64, 32, 4, 8, 1, mask=0.05, dup=0.2, slots=2500)
        masked = [2, 6]
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


# --------------------------------------------- rank masking, normal path


def _normal_mask_case(case):
    if case == "tiny":
        return config_inputs(0), [1]
    if case == "skewed":
        return config_inputs(2), [0, 7, 31]
    if case == "large":
        return config_inputs(4), [3, 64, 130, 143]   # ranks in all three 64-rank words
    if case == "T20000":   # the layout's separate scan kernel (more than 32 count blocks)
        return random_case(32, 20000, 72, 96, 6, 24, 9, mask=0.05, dup=0.1), [0, 5, 23]
    return random_case(31, 257, 136, 512, 8, 512, 7, mask=0.05, dup=0.1), [0, 63, 64, 300, 511]


@pytest.mark.parametrize("case", ["tiny", "skewed", "large", "R512", "T20000"])
def test_normal_path_rank_mask(case, layout_mode):
    """Ranks masked before the layout receive nothing (layout, dispatch and
    handle bit-exact with the oracle's masked layout); a rank masked later,
    before the combine, drops out of both combine sums."""
    inp, masked = _normal_mask_case(case)
    E, R, C, H = inp.E, inp.R, inp.C, inp.H
    m = np.zeros(R, np.int32)
    m[masked] = 1
    ora = oracle.layout(inp.topk_idx, E, R, C, rank_mask=m)
    buf = epm.Buffer(R, E, C)
    for r in masked:
        buf.low_latency_update_mask_buffer(r, mask=True)
    x, topk, w = dev_bf16(inp.x), dev(inp.topk_idx), dev(inp.topk_weights)

    ntpr, ntpe, itr, _ = buf.get_dispatch_layout(topk)
    np.testing.assert_array_equal(host(ntpr), ora.num_tokens_per_rank)
    np.testing.assert_array_equal(host(ntpe), ora.num_tokens_per_expert)
    np.testing.assert_array_equal(host(itr).astype(np.uint8), ora.is_token_in_rank)

    rx, rti, rtw, counts, h, _ = buf.dispatch(x, topk, w)
    assert h.num_recv == ora.num_recv
    compare_layout(h.layout(), ora)
    o_rx, o_rti, o_rtw = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, E, R, ora)
    np.testing.assert_array_equal(host_bits(rx), o_rx)
    np.testing.assert_array_equal(host(rti), o_rti)
    np.testing.assert_array_equal(f32_bits(host(rtw)), f32_bits(o_rtw))

    y = random_rows(ora.num_recv, H, 5, tag=12)
    out, cw, _ = buf.combine(dev_bf16(y), h, rtw)
    o_out, o_cw = oracle.combine(y, ora, o_rtw, rank_mask=m)
    assert_bf16_close(host_bits(out), o_out, what="combine, mask set at dispatch")
    np.testing.assert_array_equal(f32_bits(host(cw)), f32_bits(o_cw))

    # one more rank fails after the dispatch
    live = [r for r in range(R) if m[r] == 0 and ora.num_tokens_per_rank[r] > 0]
    extra = live[len(live) // 2]
    buf.low_latency_update_mask_buffer(extra, mask=True)
    m2 = m.copy()
    m2[extra] = 1
    out2, cw2, _ = buf.combine(dev_bf16(y), h, rtw)
    o_out2, o_cw2 = oracle.combine(y, ora, o_rtw, rank_mask=m2)
    assert_bf16_close(host_bits(out2), o_out2, what="combine, rank masked at combine time")
    np.testing.assert_array_equal(f32_bits(host(cw2)), f32_bits(o_cw2))
    assert not np.array_equal(o_out2, o_out)

    if case == "tiny":
        # a mask cannot be applied to a handle's existing layout
        d = abi.dims(inp.T, H, inp.K, E, R, C)
        raw = ctypes.c_void_p(h.raw.value)
        rc = abi.lib().ep_dispatch(ctypes.byref(d), abi.ptr(x), None, None, abi.ptr(buf._mask),
                                   ctypes.byref(raw), abi.ptr(rx), None, None, rx.shape[0], None,
                                   abi.current_stream())
        assert rc == abi.EP_ERR_INVALID
    h.free()


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


@pytest.mark.parametrize("case", ["decode", "edge", "nonfinite", "masked", "max_slots",
                                  "long_row"])
def test_ll_dispatch_fp8(case, ll_mode):
    if case == "decode":
        inp, m = config_inputs(3), None
    elif case == "max_slots":  # the largest slot count the library accepts
        inp, m = random_case(6, 4096, 128, 8, 1, 4, 1, slots=4096), None
    elif case == "long_row":  # the longest row (H = 2^20: 8192 scale blocks)
        inp, m = random_case(9, 3, 1 << 20, 8, 2, 4, 1, slots=3), None
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


def _fp8_sweep_rows(amax_bits: int, H: int = 2048):
    """Rows that enumerate every bf16 magnitude from 0 up to the bf16 value
    `amax_bits`, with both signs, 127 per 128-element block; the first
    element of every block is +amax itself, so every block's amax (after the
    1e-4 floor) and hence its scale is fixed.  Trailing unused elements
    repeat +0."""
    mags = np.arange(0, amax_bits + 1, dtype=np.uint32)
    vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    per = 127
    nblk = -(-vals.size // per)
    vals = np.concatenate([vals, np.zeros(nblk * per - vals.size, np.uint16)])
    blocks = np.concatenate([np.full((nblk, 1), amax_bits, np.uint16), vals.reshape(nblk, per)],
                            axis=1)
    bpr = H // 128
    T = -(-nblk // bpr)
    pad = np.zeros((T * bpr - nblk, 128), np.uint16)
    pad[:, 0] = amax_bits
    return np.ascontiguousarray(np.concatenate([blocks, pad]).reshape(T, H))


# bf16 block maxima: 448 (scale exactly 1: the codes are the e4m3 rounding of
# the bf16 values themselves, every e4m3 tie and subnormal tie included);
# 300 and 1.203 (scales that are not powers of two); 446 (products a hair
# above 448 hit the saturation edge); 9.98e-5 (below the 1e-4 floor).
@pytest.mark.parametrize("amax_bits", [0x43E0, 0x4396, 0x3F9A, 0x43DF, 0x38D1])
def test_ll_dispatch_fp8_conversion_sweep(amax_bits, ll_mode):
    """The FP8 dispatch's codes on rows that sweep every bf16 magnitude up to
    each block's amax, against the oracle's e4m3 round to nearest even, bit
    for bit.  Finite blocks are quantized by the hardware's packed
    fp32->e4m3 conversion, so this pins that conversion to the definition
    on every value the dispatch can feed it at these scales."""
    x = _fp8_sweep_rows(amax_bits)
    T, H = x.shape
    E, R, K = 8, 2, 2
    topk = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], axis=1).astype(np.int64)
    S = T
    buf = epm.Buffer(R, E)
    (q, sc), count, hdl, _, _ = buf.low_latency_dispatch(dev_bf16(x), dev(topk), S, E,
                                                          use_fp8=True)
    o_q, o_sc, o_cnt, o_src, o_slot = oracle.ll_dispatch_fp8(x, topk, E, R, S)
    np.testing.assert_array_equal(host(count), o_cnt)
    np.testing.assert_array_equal(host(hdl.src_info), o_src)
    used = o_src >= 0
    qh = q.view(torch.uint8).cpu().numpy()
    assert not pinlib.e4m3_is_nan(o_q[used]).any()
    np.testing.assert_array_equal(qh[used], o_q[used])
    np.testing.assert_array_equal(f32_bits(sc.cpu().numpy()[used]), f32_bits(o_sc[used]))
    if amax_bits == 0x43E0:
        # scale 1: the e4m3 midpoints among the inputs (values halfway between
        # two neighbouring codes) were all rounded to the even code
        xf = oracle.bf16_to_f32(x.reshape(-1))
        lo = np.array([oracle.e4m3_to_f32(c) for c in range(0x7F)], np.float64)
        mids = (lo[:-1] + lo[1:]) / 2
        n_ties = int(np.isin(np.abs(xf.astype(np.float64)), mids).sum())
        assert n_ties > 200, n_ties


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


def test_lb_ops_many_replicas():
    """300 replicas over 40 experts: repeated experts and invalid entries
    spread over several 64-entry scans of the mapping."""
    rng = np.random.default_rng(77)
    E, n_rep, P = 40, 300, 136
    mapping = rng.integers(-1, E + 3, n_rep).astype(np.int64)
    mapping[:5] = 7   # one expert replicated in a run, and again later
    mapping[250] = 7
    buf = epm.Buffer(1, 1)
    mp = dev(mapping)
    ew = random_rows(E, P, 5, tag=41)
    rw0 = random_rows(n_rep, P, 5, tag=42)
    rwd = dev_bf16(rw0)
    buf.lb_prefetch_weights(rwd, dev_bf16(ew), mp)
    np.testing.assert_array_equal(host_bits(rwd), oracle.lb_prefetch_weights(ew, rw0, mapping))
    rg = random_rows(n_rep, P, 5, tag=43)
    egd = dev_bf16(ew)
    buf.lb_reduce_grads(dev_bf16(rg), egd, mp)
    assert_bf16_close(host_bits(egd), oracle.lb_reduce_grads(rg, ew, mapping), what="many replicas")


# ------------------------------------------------------------ FP8 LL combine


@pytest.mark.parametrize("case", ["decode", "random_codes", "masked", "nonfinite"])
def test_ll_combine_fp8(case, ll_mode):
    """The FP8 payload decoded with its scales inside the LL combine, against
    the oracle: the FP8 dispatch's own output, and random codes with
    power-of-two scales; a rank masked at combine time; non-finite blocks
    (NaN outputs compared as NaN)."""
    if case == "decode":
        inp, m = config_inputs(3), None
    elif case == "random_codes":
        inp, m = random_case(13, 40, 384, 16, 4, 4, 1, mask=0.1, dup=0.2, slots=40), None
    elif case == "masked":
        inp = random_case(14, 40, 512, 16, 4, 4, 1, mask=0.1, slots=40)
        m = np.array([0, 1, 0, 0], np.int32)
    else:
        inp, m = pinlib.fp8_nonfinite_case(), None
    E, R, S = inp.E, inp.R, inp.slots
    buf = epm.Buffer(R, E)
    x, topk, w = dev_bf16(inp.x), dev(inp.topk_idx), dev(inp.topk_weights)
    (q, sc), _, hdl, _, _ = buf.low_latency_dispatch(x, topk, S, E, use_fp8=True)
    if case == "random_codes":
        rng = np.random.default_rng(5)
        qh = rng.integers(0, 256, tuple(q.shape)).astype(np.uint8)
        qh[(qh & 0x7F) == 0x7F] = 0x21
        sh = np.ldexp(np.ones(tuple(sc.shape)), rng.integers(-4, 5, tuple(sc.shape))).astype(np.float32)
        q = torch.from_numpy(qh).cuda().view(torch.float8_e4m3fn)
        sc = torch.from_numpy(sh).cuda()
    else:
        qh = q.view(torch.uint8).cpu().numpy()
        sh = sc.cpu().numpy()
    if m is not None:
        buf.low_latency_update_mask_buffer(int(np.nonzero(m)[0][0]), mask=True)
    out, _, _ = buf.low_latency_combine((q, sc), topk, w, hdl)
    # the oracle combines the same codes and scales (unused cells never read)
    exp = oracle.ll_combine_fp8(qh, sh, inp.topk_idx, inp.topk_weights, E, R, combine_mask=m)
    got = host_bits(out)
    nan_e = (exp & 0x7FFF) > 0x7F80
    np.testing.assert_array_equal((got & 0x7FFF) > 0x7F80, nan_e)
    assert_bf16_close(np.where(nan_e, 0, got), np.where(nan_e, 0, exp), what=f"fp8 combine {case}")
    if case != "nonfinite":
        assert not nan_e.any()


# ---------------------------------------------------- crafted rounding cases


def _rows_f32(values, H=8):
    return pinlib.bits_from_f32_exact(np.repeat(np.asarray(values, np.float32)[:, None], H, axis=1))


def test_crafted_sum_order_and_fma_on_gpu():
    """The crafted cases the oracle is pinned with, through the HIP kernels:
    summation order (ranks, slots, replicas ascending), the fused
    multiply-add of the LL combines and the bias order of the combine.  Each
    case has one right answer, and the wrong orders or an unfused product give
    another."""
    terms = np.array([1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24], np.float32)
    fwd, rev = np.float32(1.0), np.float32(1.0 + 2.0 ** -7)
    fused = np.float32(2.0 ** -17 + 2.0 ** -24)

    def values(t):
        return pinlib.f32_from_bits(host_bits(t))

    # normal combine: one token on experts 0..3, one per rank
    buf = epm.Buffer(4, 4, 1)
    idx = dev(np.array([[0, 1, 2, 3]], np.int64))
    x = dev_bf16(_rows_f32([1.0]))
    _, _, _, _, h, _ = buf.dispatch(x, idx)
    for t, want in ((terms, fwd), (terms[::-1].copy(), rev)):
        out, _, _ = buf.combine(dev_bf16(_rows_f32(t)), h)
        assert (values(out) == want).all(), "combine rank order"
    h.free()
    # bias after the rank sum: ranks 0, 1 hold 1 and 2^-8, two biases of 2^-24
    buf = epm.Buffer(2, 2, 1)
    _, _, _, _, h, _ = buf.dispatch(x, dev(np.array([[0, 1]], np.int64)))
    bias = dev_bf16(_rows_f32([2.0 ** -24]))
    out, _, _ = buf.combine(dev_bf16(_rows_f32([1.0, 2.0 ** -8])), h, bias=(bias, bias))
    assert (values(out) == fwd).all(), "bias after the rank sum"
    h.free()

    # LL combines: experts 0, 1 on one rank, one slot each
    buf = epm.Buffer(1, 2)
    lidx = dev(np.array([[0, 1]], np.int64))
    w = dev(np.array([[1.0, 1.0 + 2.0 ** -17]], np.float32))
    _, _, hdl, _, _ = buf.low_latency_dispatch(dev_bf16(_rows_f32([1.0], H=128)), lidx, 1, 2)
    y = _rows_f32([-(1.0 + 2.0 ** -7), 1.0 + 2.0 ** -7], H=128).reshape(2, 1, 1, 128)
    out, _, _ = buf.low_latency_combine(dev_bf16(y), lidx, w, hdl)
    assert (values(out) == fused).all(), "LL combine fma"
    q = np.zeros((2, 1, 1, 128), np.uint8)
    q[0], q[1] = 0xB8, 0x38  # e4m3 codes of -1 and 1
    sc = np.full((2, 1, 1, 1), 1.0 + 2.0 ** -7, np.float32)
    out, _, _ = buf.low_latency_combine((dev(q), dev(sc)), lidx, w, hdl)
    assert (values(out) == fused).all(), "FP8 LL combine fma"
    # and the slot order: unit weights over four slots
    buf = epm.Buffer(1, 4)
    lidx = dev(np.array([[0, 1, 2, 3]], np.int64))
    ones = dev(np.ones((1, 4), np.float32))
    _, _, hdl, _, _ = buf.low_latency_dispatch(x, lidx, 1, 4)
    for t, want in ((terms, fwd), (terms[::-1].copy(), rev)):
        out, _, _ = buf.low_latency_combine(dev_bf16(_rows_f32(t).reshape(4, 1, 1, 8)), lidx, ones,
                                            hdl)
        assert (values(out) == want).all(), "LL combine slot order"

    # lb_reduce_grads: own gradient 0, four replicas of expert 0
    for t, want in ((terms, fwd), (terms[::-1].copy(), rev)):
        eg = dev_bf16(_rows_f32([0.0]))
        buf.lb_reduce_grads(dev_bf16(_rows_f32(t)), eg, dev(np.zeros(4, np.int64)))
        assert (values(eg) == want).all(), "lb_reduce_grads replica order"
