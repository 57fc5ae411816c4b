"""Property tests of the oracle over shapes the fixed pins do not reach.

Hypothesis draws a routing table and its shape: up to 40 tokens, up to 6
slots, 1 to 8 ranks, 1 to 4 experts per rank, channel counts above the token
count, repeated experts and masked slots, and an optional rank mask.  It then
checks the oracle against definitions computed another way:
- the layout against the sorted (rank, token) pair listing, of the
  slot-masked table when a rank mask is given;
- the dispatch rows, the remapped ids and weights, and the combine of
  small-integer rows (exact in fp32) against the same listing;
- the low-latency slots against a per-expert listing of the (token, slot)
  pairs.
On failure Hypothesis shrinks to a minimal table."""

from __future__ import annotations

import numpy as np
from hypothesis import given, settings, HealthCheck
from hypothesis import strategies as st

import oracle as O
from pinlib import bits_from_f32_exact, brute_layout, f32_from_bits, masked_topk, _compare_layout


@st.composite
def routing(draw):
    R = draw(st.integers(1, 8))
    epr = draw(st.integers(1, 4))
    E = R * epr
    T = draw(st.integers(0, 40))
    K = draw(st.integers(1, 6))
    C = draw(st.integers(1, 50))
    ids = draw(st.lists(st.integers(-1, E - 1), min_size=T * K, max_size=T * K))
    idx = np.array(ids, np.int64).reshape(T, K)
    mask = None
    if draw(st.booleans()):
        mask = np.array(draw(st.lists(st.integers(0, 1), min_size=R, max_size=R)), np.int32)
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return idx, E, R, C, mask, seed


@settings(max_examples=300, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(routing())
def test_layout_dispatch_combine_match_the_pair_listing(case):
    idx, E, R, C, mask, seed = case
    T, K = idx.shape
    epr = E // R
    L = O.layout(idx, E, R, C, rank_mask=mask)
    live = idx if mask is None else masked_topk(idx, E, R, mask)
    B = brute_layout(live, E, R, C)
    _compare_layout(L, B, T, R, C)

    rng = np.random.default_rng(seed)
    H = 8
    w = rng.random((T, K)).astype(np.float32)
    xf = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
    x = bits_from_f32_exact(xf)
    rx, rti, rtw = O.dispatch(x, idx, w, E, R, L)
    assert rx.shape[0] == len(B["pairs"])
    for i, (r, t) in enumerate(B["pairs"]):
        np.testing.assert_array_equal(rx[i], x[t])
        for k in range(K):
            e = int(live[t, k])
            if e >= 0 and e // epr == r:
                assert rti[i, k] == e - r * epr and rtw[i, k] == w[t, k]
            else:
                assert rti[i, k] == -1 and rtw[i, k] == 0.0
    yf = rng.integers(-8, 9, size=(len(B["pairs"]), H)).astype(np.float32)
    out, cw = O.combine(bits_from_f32_exact(yf), L, rtw)
    exp = np.zeros((T, H), np.float32)
    expw = np.zeros((T, K), np.float32)
    for i, (r, t) in enumerate(B["pairs"]):
        exp[t] += yf[i]
        expw[t] += rtw[i]
    np.testing.assert_array_equal(f32_from_bits(out), exp)
    np.testing.assert_array_equal(cw, expw)


@settings(max_examples=300, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(routing(), st.integers(1, 12))
def test_low_latency_slots_match_the_expert_listing(case, S):
    idx, E, R, _, mask, _ = case
    T, K = idx.shape
    if T > S:
        S = T  # the LL path needs a slot for every token
    epr = E // R
    _, cnt, src, slot = O.ll_dispatch(np.zeros((T, 8), np.uint16), idx, E, R, S, with_buf=False,
                                      rank_mask=mask)
    exp_cnt = np.zeros((epr, R), np.int32)
    exp_src = np.full((epr, R, S), -1, np.int32)
    exp_slot = np.full((T, K), -1, np.int32)
    for e in range(E):
        r = e // epr
        if mask is not None and mask[r]:
            continue
        pairs = [(t, k) for t in range(T) for k in range(K) if idx[t, k] == e]
        exp_cnt[e % epr, r] = len(pairs)
        for s, (t, k) in enumerate(pairs[:S]):
            exp_src[e % epr, r, s] = t
            exp_slot[t, k] = s
    np.testing.assert_array_equal(cnt, exp_cnt)
    np.testing.assert_array_equal(src, exp_src)
    np.testing.assert_array_equal(slot, exp_slot)
