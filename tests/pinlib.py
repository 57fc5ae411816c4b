"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with an
independent fact: a worked example derived by hand, brute force by a
different algorithm, closed forms, invariants, library rounding, or an fp64
evaluation within a stated error bound.  ``tests/test_oracle_pins.py`` runs
them on the real oracle; ``tests/test_oracle_mutants.py`` runs them on copies
of the oracle with a planted mistake and requires that some pin fails.
"""

from __future__ import annotations

import itertools
import json
import os

import numpy as np
import torch

import oracle as O
from gen import generate, random_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32_from_bits(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bits_from_f32_exact(f):
    """bf16 bits of values that are exactly representable in bf16."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> np.uint32(16)).astype(np.uint16)


def torch_bf16_bits(f):
    """Library round-to-nearest-even of fp32 (or fp64 via fp32-free path) to bf16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(f))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------ worked example


def check_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    idx = np.array(g["topk_idx"], np.int64)
    w = np.array(g["topk_weights"], np.float32)
    x = bits_from_f32_exact(np.array(g["x"], np.float32))
    E, R, C = g["E"], g["R"], g["C"]
    L = O.layout(idx, E, R, C)
    for name in ["num_tokens_per_expert", "is_token_in_rank", "num_tokens_per_rank",
                 "rank_prefix_matrix", "channel_prefix_matrix", "recv_channel_prefix_matrix",
                 "send_head", "recv_src_idx"]:
        np.testing.assert_array_equal(getattr(L, name), np.array(g[name]), err_msg=name)
    rx, rti, rtw = O.dispatch(x, idx, w, E, R, L)
    np.testing.assert_array_equal(f32_from_bits(rx), np.array(g["recv_x"], np.float32))
    np.testing.assert_array_equal(rti, np.array(g["recv_topk_idx"]))
    np.testing.assert_array_equal(rtw, np.array(g["recv_topk_weights"], np.float32))
    out, cw = O.combine(rx, L, rtw)
    np.testing.assert_array_equal(f32_from_bits(out), np.array(g["combine_of_recv_x"], np.float32))
    np.testing.assert_array_equal(cw, np.array(g["combined_topk_weights"], np.float32))
    buf, counts, src, ts = O.ll_dispatch(x, idx, E, R, g["slots"])
    np.testing.assert_array_equal(counts, np.array(g["ll_counts"]))
    np.testing.assert_array_equal(ts, np.array(g["ll_topk_slot"]))
    np.testing.assert_array_equal(src, np.array(g["ll_src_info"]))
    out = O.ll_combine(buf, idx, w, E, R)
    np.testing.assert_array_equal(f32_from_bits(out),
                                  np.array(g["ll_combine_of_identity"], np.float32))


# -------------------------------------------------------------- brute force


def brute_layout(idx, E, R, C):
    """Layout by a different algorithm: list the (rank, token) pairs, sort
    them by (rank, token); a pair's packed row is its index in that list."""
    T, K = idx.shape
    epr = E // R
    pairs = sorted({(int(e) // epr, t) for t in range(T) for e in idx[t] if e >= 0})
    pos = {p: i for i, p in enumerate(pairs)}
    ntpe = [int(np.sum(idx == e)) for e in range(E)]
    ntpr = [sum(1 for (r, _) in pairs if r == rr) for rr in range(R)]
    first = {}
    for i, (r, t) in enumerate(pairs):
        first.setdefault(r, i)
    send_head = [[pos[(r, t)] - first[r] if (r, t) in pos else -1 for r in range(R)]
                 for t in range(T)]
    in_rank = [[1 if (r, t) in pos else 0 for r in range(R)] for t in range(T)]
    rank_prefix = [sum(ntpr[:r + 1]) for r in range(R)]
    per = -(-T // C) if T > 0 else 1
    chan = [[sum(1 for (r2, t) in pairs if r2 == r and t // per <= c) for c in range(C)]
            for r in range(R)]
    rchan = [[sum(1 for (r2, t) in pairs if r2 == r and t // per < c) for c in range(C)]
             for r in range(R)]
    src = [t for (_, t) in pairs]
    return dict(num_tokens_per_expert=ntpe, num_tokens_per_rank=ntpr, send_head=send_head,
                is_token_in_rank=in_rank, rank_prefix_matrix=rank_prefix,
                channel_prefix_matrix=chan, recv_channel_prefix_matrix=rchan,
                recv_src_idx=src, pairs=pairs)


def _compare_layout(L, B, T, R, C):
    np.testing.assert_array_equal(L.num_tokens_per_expert, B["num_tokens_per_expert"])
    np.testing.assert_array_equal(L.num_tokens_per_rank, B["num_tokens_per_rank"])
    np.testing.assert_array_equal(L.rank_prefix_matrix, B["rank_prefix_matrix"])
    np.testing.assert_array_equal(L.send_head.reshape(T, R), np.array(B["send_head"]).reshape(T, R))
    np.testing.assert_array_equal(L.is_token_in_rank.reshape(T, R),
                                  np.array(B["is_token_in_rank"]).reshape(T, R))
    np.testing.assert_array_equal(L.channel_prefix_matrix, np.array(B["channel_prefix_matrix"]))
    np.testing.assert_array_equal(L.recv_channel_prefix_matrix,
                                  np.array(B["recv_channel_prefix_matrix"]))
    np.testing.assert_array_equal(L.recv_src_idx, np.array(B["recv_src_idx"], np.int64))


def check_bruteforce_exhaustive(T=3, K=2, E=4, Rs=(1, 2, 4), stride=1):
    """Every topk_idx table over {-1, 0..E-1} for the given T, K (every
    ``stride``-th one), each rank count, C in {1, 2, T+1}; layout against
    the sorted-pair brute force; dispatch and combine rows against it too."""
    vals = list(range(-1, E))
    n = 0
    for i, flat in enumerate(itertools.product(vals, repeat=T * K)):
        if i % stride:
            continue
        idx = np.array(flat, np.int64).reshape(T, K)
        for R in Rs:
            for C in sorted({1, 2, T + 1}):
                L = O.layout(idx, E, R, C)
                B = brute_layout(idx, E, R, C)
                _compare_layout(L, B, T, R, C)
                n += 1
    return n


def check_bruteforce_dispatch_combine(seed=0, cases=200):
    """Dispatch rows and combine sums on random tiny tables, against the
    sorted-pair listing.  Token rows hold small integers, so every fp32 sum is
    exact and the expected combine is the plain integer sum."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        T = int(rng.integers(0, 6))
        K = int(rng.integers(1, 4))
        R = int(rng.choice([1, 2, 3, 6]))
        E = R * int(rng.integers(1, 3))
        C = int(rng.integers(1, 5))
        H = 8
        idx = rng.integers(-1, E, size=(T, K)).astype(np.int64)
        w = rng.random((T, K)).astype(np.float32)
        xf = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
        x = bits_from_f32_exact(xf)
        L = O.layout(idx, E, R, C)
        B = brute_layout(idx, E, R, C)
        _compare_layout(L, B, T, R, C)
        rx, rti, rtw = O.dispatch(x, idx, w, E, R, L)
        epr = E // R
        for i, (r, t) in enumerate(B["pairs"]):
            np.testing.assert_array_equal(rx[i], x[t])
            for k in range(K):
                e = int(idx[t, k])
                if e >= 0 and e // epr == r:
                    assert rti[i, k] == e - r * epr and rtw[i, k] == w[t, k]
                else:
                    assert rti[i, k] == -1 and rtw[i, k] == 0.0
        # y rows: small integers, different per packed row
        yf = rng.integers(-8, 9, size=(len(B["pairs"]), H)).astype(np.float32)
        out, _ = O.combine(bits_from_f32_exact(yf), L)
        exp = np.zeros((T, H), np.float32)
        for i, (r, t) in enumerate(B["pairs"]):
            exp[t] += yf[i]
        np.testing.assert_array_equal(f32_from_bits(out), exp)


# ---------------------------------------------------------------- invariants


def check_layout_invariants(inp):
    idx, E, R, C = inp.topk_idx, inp.E, inp.R, inp.C
    T = idx.shape[0]
    epr = E // R
    L = O.layout(idx, E, R, C)
    itr = L.is_token_in_rank.astype(np.int64)
    ntpr = L.num_tokens_per_rank.astype(np.int64)
    ntpe = L.num_tokens_per_expert.astype(np.int64)
    assert ntpr.sum() == itr.sum() == L.num_recv
    assert ntpe.sum() == int(np.sum(idx >= 0))
    per_rank_e = ntpe.reshape(R, epr)
    assert np.all(per_rank_e.max(axis=1) <= ntpr) and np.all(ntpr <= per_rank_e.sum(axis=1))
    rp = L.rank_prefix_matrix.astype(np.int64)
    assert np.all(np.diff(rp) >= 0) and rp[-1] == L.num_recv
    np.testing.assert_array_equal(np.diff(np.concatenate([[0], rp])), ntpr)
    cp = L.channel_prefix_matrix.astype(np.int64)
    assert np.all(np.diff(cp, axis=1) >= 0)
    np.testing.assert_array_equal(cp[:, -1], ntpr)
    np.testing.assert_array_equal(L.recv_channel_prefix_matrix[:, 1:], cp[:, :-1])
    assert np.all(L.recv_channel_prefix_matrix[:, 0] == 0)
    sh = L.send_head
    assert np.array_equal(sh >= 0, itr.astype(bool))
    S = np.concatenate([[0], rp[:-1]])
    rsi = L.recv_src_idx.astype(np.int64)
    for r in range(R):
        seg = rsi[S[r]:rp[r]]
        assert np.all(np.diff(seg) > 0), "segment not in token order"
        np.testing.assert_array_equal(seg, np.nonzero(itr[:, r])[0])
        ts = np.nonzero(sh[:, r] >= 0)[0]
        np.testing.assert_array_equal(rsi[S[r] + sh[ts, r]], ts)
    # membership recomputed from the definition with numpy
    ranks = np.where(idx >= 0, idx // epr, -1)
    ref = np.zeros((T, R), bool)
    for k in range(idx.shape[1]):
        ok = ranks[:, k] >= 0
        ref[np.nonzero(ok)[0], ranks[ok, k]] = True
    np.testing.assert_array_equal(L.is_token_in_rank.astype(bool), ref)
    return L


def check_special_cases(seed=0):
    # R = E, distinct experts: tokens per rank equal tokens per expert
    inp = generate(64, 8, 16, 4, 16, 3, seed=seed, with_x=False)
    L = O.layout(inp.topk_idx, 16, 16, 3)
    np.testing.assert_array_equal(L.num_tokens_per_rank, L.num_tokens_per_expert)
    # R = 1: every token with a valid slot goes to rank 0, in order
    inp = random_case(seed, 50, 8, 12, 3, 1, 4, mask=0.4)
    L = O.layout(inp.topk_idx, 12, 1, 4)
    valid = np.nonzero((inp.topk_idx >= 0).any(axis=1))[0]
    assert L.num_tokens_per_rank[0] == len(valid)
    np.testing.assert_array_equal(L.recv_src_idx, valid)
    # K = 1: N equals the number of valid tokens; each row's local expert is e % epr
    inp = random_case(seed + 1, 40, 8, 12, 1, 4, 2, mask=0.3)
    L = O.layout(inp.topk_idx, 12, 4, 2)
    assert L.num_recv == int(np.sum(inp.topk_idx >= 0))
    rx, rti, _ = O.dispatch(np.zeros((40, 8), np.uint16), inp.topk_idx, inp.topk_weights, 12, 4, L)
    np.testing.assert_array_equal(rti[:, 0], inp.topk_idx[L.recv_src_idx, 0] % 3)
    # C = 1: the single channel column is the per-rank total
    inp = random_case(seed + 2, 33, 8, 8, 2, 4, 1, mask=0.2)
    L = O.layout(inp.topk_idx, 8, 4, 1)
    np.testing.assert_array_equal(L.channel_prefix_matrix[:, 0], L.num_tokens_per_rank)
    # C >= T: one token per channel, so column c counts hits among tokens 0..c
    T = 9
    for C in (T, T + 3):
        inp = random_case(seed + 3, T, 8, 8, 2, 4, C, mask=0.2)
        L = O.layout(inp.topk_idx, 8, 4, C)
        csum = np.cumsum(L.is_token_in_rank.astype(np.int64), axis=0)  # [T, R]
        for c in range(C):
            np.testing.assert_array_equal(L.channel_prefix_matrix[:, c], csum[min(c, T - 1)])
    # T = 0: everything empty
    L = O.layout(np.zeros((0, 4), np.int64), 8, 4, 2)
    assert L.num_recv == 0 and np.all(L.channel_prefix_matrix == 0)


# ------------------------------------------------------------------ dispatch


def check_dispatch_props(inp):
    L = O.layout(inp.topk_idx, inp.E, inp.R, inp.C)
    rx, rti, rtw = O.dispatch(inp.x, inp.topk_idx, inp.topk_weights, inp.E, inp.R, L)
    src = L.recv_src_idx
    np.testing.assert_array_equal(rx, inp.x[src])
    epr = inp.E // inp.R
    rank_of_row = np.searchsorted(L.rank_prefix_matrix, np.arange(L.num_recv), side="right")
    e = inp.topk_idx[src]
    mine = (e >= 0) & (e // epr == rank_of_row[:, None])
    np.testing.assert_array_equal(rti, np.where(mine, e - rank_of_row[:, None] * epr, -1))
    np.testing.assert_array_equal(rtw, np.where(mine, inp.topk_weights[src], np.float32(0)))
    # handle reuse: a second x through the same layout is the same gather
    x2 = np.ascontiguousarray(inp.x[::-1])
    rx2, _, _ = O.dispatch(x2, None, None, inp.E, inp.R, L, with_topk=False)
    np.testing.assert_array_equal(rx2, x2[src])
    return L, rx, rtw


# ------------------------------------------------------------------- combine


def check_identity_combine(inp):
    """combine(dispatch(x)) = bf16(n_t * x_t): n_t <= 8 copies of an 8-bit
    mantissa value sum exactly in fp32, so only the final rounding acts; the
    expected value is rounded by torch's bf16 conversion."""
    L, rx, rtw = check_dispatch_props(inp)
    out, cw = O.combine(rx, L, rtw)
    n = L.is_token_in_rank.astype(np.float32).sum(axis=1)
    exp = torch_bf16_bits(f32_from_bits(inp.x) * n[:, None])
    np.testing.assert_array_equal(f32_from_bits(out), f32_from_bits(exp))
    # weight round trip: exactly one nonzero term per valid slot
    np.testing.assert_array_equal(cw, np.where(inp.topk_idx >= 0, inp.topk_weights, np.float32(0)))


def _bf16_ulp(v):
    v = np.abs(np.asarray(v, np.float64))
    v = np.maximum(v, 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(v)) - 7)


def check_combine_fp64(seed=0, T=64, H=96, K=8, E=32, R=8, C=3):
    """Random N(0,1) rows: the oracle's sequential fp32 sum then RNE must be
    within sum-error bound (n-1) * 2^-24 * sum|v| plus half a bf16 ulp of the
    exact fp64 sum (a standard bound for recursive summation); where no
    cancellation occurs this is within one bf16 ulp."""
    inp = random_case(seed, T, H, E, K, R, C, mask=0.1)
    L = O.layout(inp.topk_idx, E, R, C)
    rng = np.random.default_rng(seed + 7)
    yf = rng.standard_normal((L.num_recv, H)).astype(np.float32)
    y = (yf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out, _ = O.combine(y, L)
    v = f32_from_bits(y).astype(np.float64)
    exact = np.zeros((T, H))
    absum = np.zeros((T, H))
    for r in range(R):
        S = L.rank_prefix_matrix[r - 1] if r > 0 else 0
        ts = np.nonzero(L.send_head[:, r] >= 0)[0]
        rows = S + L.send_head[ts, r]
        exact[ts] += v[rows]
        absum[ts] += np.abs(v[rows])
    n = L.is_token_in_rank.sum(axis=1).astype(np.float64)[:, None]
    got = f32_from_bits(out).astype(np.float64)
    err = np.abs(got - exact)
    bound = np.maximum(n - 1, 0) * 2.0 ** -24 * absum * 1.0001 + 0.5 * _bf16_ulp(np.maximum(np.abs(got), np.abs(exact)))
    assert np.all(err <= bound), float((err - bound).max())
    well = np.abs(exact) >= np.maximum(n - 1, 0) * 2.0 ** -16 * absum
    assert np.all(err[well] <= _bf16_ulp(exact)[well])


# ----------------------------------------------------------------------- LL


def check_ll(inp):
    """Slots by a different algorithm (stable sort of the pairs by expert),
    counts equal per-expert counts, buffer rows are the source rows, and a
    combine of identity experts with softmax weights returns x bit-exactly
    (sum of weights is 1 within a few fp32 ulps, far inside half a bf16 ulp)."""
    E, R, slots = inp.E, inp.R, inp.slots
    epr = E // R
    T, K = inp.topk_idx.shape
    buf, counts, src, ts = O.ll_dispatch(inp.x, inp.topk_idx, E, R, slots)
    flat = inp.topk_idx.reshape(-1)
    order = np.argsort(np.where(flat >= 0, flat, E), kind="stable")
    exp_slot = np.full(T * K, -1, np.int64)
    seen = {}
    for p in order:
        e = int(flat[p])
        if e < 0:
            continue
        exp_slot[p] = seen.get(e, 0)
        seen[e] = exp_slot[p] + 1
    exp_slot = np.where(exp_slot < slots, exp_slot, -1)
    np.testing.assert_array_equal(ts.reshape(-1), exp_slot)
    cnt = np.bincount(flat[flat >= 0], minlength=E)
    np.testing.assert_array_equal(counts, cnt.reshape(R, epr).T)
    for le in range(epr):
        for r in range(R):
            c = min(int(counts[le, r]), slots)
            s = src[le, r]
            assert np.all(s[c:] == -1) and np.all(np.diff(s[:c]) >= 0)
            np.testing.assert_array_equal(buf[le, r, :c], inp.x[s[:c]])
    out = O.ll_combine(buf, inp.topk_idx, inp.topk_weights, E, R)
    if np.all(inp.topk_idx >= 0) and np.all(cnt <= slots):
        np.testing.assert_array_equal(out, inp.x)
    return buf, counts, src, ts


def check_ll_fp64(seed=0, T=32, H=64, K=4, E=16, R=4, slots=32):
    inp = random_case(seed, T, H, E, K, R, 1, mask=0.15, slots=slots)
    rng = np.random.default_rng(seed + 11)
    epr = E // R
    bf = rng.standard_normal((epr, R, slots, H)).astype(np.float32)
    buf = (bf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    w = rng.standard_normal((T, K)).astype(np.float32)
    out = O.ll_combine(buf, inp.topk_idx, w, E, R)
    _, _, _, ts = O.ll_dispatch(np.zeros((T, H), np.uint16), inp.topk_idx, E, R, slots)
    v = f32_from_bits(buf).astype(np.float64)
    exact = np.zeros((T, H))
    absum = np.zeros((T, H))
    nk = np.zeros((T, 1))
    for t in range(T):
        for k in range(K):
            e = int(inp.topk_idx[t, k])
            if e < 0:
                continue
            row = v[e % epr, e // epr, ts[t, k]]
            exact[t] += float(w[t, k]) * row
            absum[t] += abs(float(w[t, k])) * np.abs(row)
            nk[t] += 1
    got = f32_from_bits(out).astype(np.float64)
    err = np.abs(got - exact)
    bound = nk * 2.0 ** -24 * absum * 1.0001 + 0.5 * _bf16_ulp(np.maximum(np.abs(got), np.abs(exact)))
    assert np.all(err <= bound), float((err - bound).max())


# --------------------------------------------------------------------- bf16


def check_bf16_patterns(step=1, chunk=1 << 24):
    """fp32 -> bf16 round-to-nearest-even against torch's conversion on every
    ``step``-th fp32 bit pattern (step=1: all 2^32).  NaNs must stay NaN."""
    for start in range(0, 1 << 32, chunk * step):
        u = (np.arange(chunk, dtype=np.uint64) * step + start).astype(np.uint32)
        f = u.view(np.float32)
        got = O.f32_to_bf16(f)
        exp = torch_bf16_bits(f)
        nan = np.isnan(f)
        assert np.array_equal(got[~nan], exp[~nan]), hex(int(u[~nan][np.argmax(got[~nan] != exp[~nan])]))
        g = got[nan]
        assert np.all(((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0) | ((g & 0x7FC0) == 0x7FC0))


def check_bf16_edges():
    cases = {
        0x3F808000: 0x3F80,  # 1 + half ulp, kept lsb even: ties to even, down
        0x3F818000: 0x3F82,  # 1 + 1.5 ulp: ties to even, up
        0x3F808001: 0x3F81,  # just above half: up
        0x3F807FFF: 0x3F80,  # just below half: down
        0x3FFF8000: 0x4000,  # carry out of the mantissa into the exponent
        0x7F7FFFFF: 0x7F80,  # past the largest finite bf16: infinity
        0x80000000: 0x8000,  # -0 stays -0
        0x00000001: 0x0000,  # smallest denormal rounds to +0
        0x7F800000: 0x7F80,  # +inf
    }
    u = np.array(list(cases.keys()), np.uint32)
    got = O.f32_to_bf16(u.view(np.float32))
    np.testing.assert_array_equal(got, np.array(list(cases.values()), np.uint16))
