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


# ------------------------------------------------------------ rank masking


def masked_topk(topk_idx, E, R, rank_mask):
    """topk_idx with every slot whose expert sits on a masked rank set to -1."""
    epr = E // R
    idx = topk_idx.copy()
    ranks = np.where(idx >= 0, idx // epr, 0)
    idx[(idx >= 0) & (np.asarray(rank_mask)[ranks] != 0)] = -1
    return idx


def check_ll_rank_mask(inp, rank_mask):
    """Masking a rank is the same as masking every slot that names one of its
    experts: counts, slots, src_info, rows and the combine all agree."""
    E, R, S = inp.E, inp.R, inp.slots
    m = np.asarray(rank_mask, np.int32)
    a = O.ll_dispatch(inp.x, inp.topk_idx, E, R, S, rank_mask=m)
    idx2 = masked_topk(inp.topk_idx, E, R, m)
    b = O.ll_dispatch(inp.x, idx2, E, R, S)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    out_a = O.ll_combine(a[0], inp.topk_idx, inp.topk_weights, E, R, rank_mask=m)
    out_b = O.ll_combine(b[0], idx2, inp.topk_weights, E, R)
    np.testing.assert_array_equal(out_a, out_b)
    # masked ranks receive nothing
    epr = E // R
    for r in np.nonzero(m)[0]:
        assert np.all(a[1][:, r] == 0) and np.all(a[2][:, r] == -1)
    # a rank masked only at combine time drops exactly its pairs' terms
    out_c = O.ll_combine(b[0], idx2, inp.topk_weights, E, R, combine_mask=m)
    np.testing.assert_array_equal(out_c, out_b)
    full = O.ll_dispatch(inp.x, inp.topk_idx, E, R, S)
    out_d = O.ll_combine(full[0], inp.topk_idx, inp.topk_weights, E, R, combine_mask=m)
    w2 = np.where(idx2 >= 0, inp.topk_weights, np.float32(0))
    out_e = O.ll_combine(full[0], inp.topk_idx, w2, E, R)
    np.testing.assert_array_equal(f32_from_bits(out_d), f32_from_bits(out_e))
    return a


def check_ll_mask_extremes(inp):
    E, R, S = inp.E, inp.R, inp.slots
    none = O.ll_dispatch(inp.x, inp.topk_idx, E, R, S, rank_mask=np.zeros(R, np.int32))
    plain = O.ll_dispatch(inp.x, inp.topk_idx, E, R, S)
    for u, v in zip(none, plain):
        np.testing.assert_array_equal(u, v)
    allm = O.ll_dispatch(inp.x, inp.topk_idx, E, R, S, rank_mask=np.ones(R, np.int32))
    assert np.all(allm[1] == 0) and np.all(allm[2] == -1) and np.all(allm[3] == -1)
    out = O.ll_combine(allm[0], inp.topk_idx, inp.topk_weights, E, R, rank_mask=np.ones(R, np.int32))
    assert np.all((out & 0x7FFF) == 0)


def check_layout_rank_mask(inp, rank_mask):
    """Normal-path masking: the masked layout is the sorted-pair brute force
    of the table whose slots on masked ranks are set to -1; masked ranks get
    no tokens, their experts count 0, and the dispatch rows follow."""
    E, R, C, T = inp.E, inp.R, inp.C, inp.T
    m = np.asarray(rank_mask, np.int32)
    L = O.layout(inp.topk_idx, E, R, C, rank_mask=m)
    idx2 = masked_topk(inp.topk_idx, E, R, m)
    _compare_layout(L, brute_layout(idx2, E, R, C), T, R, C)
    epr = E // R
    for r in np.nonzero(m)[0]:
        assert L.num_tokens_per_rank[r] == 0
        assert np.all(L.is_token_in_rank[:, r] == 0) and np.all(L.send_head[:, r] == -1)
        assert np.all(L.num_tokens_per_expert[r * epr:(r + 1) * epr] == 0)
    # dispatch of the masked layout = dispatch of the slot-masked table
    a = O.dispatch(inp.x, inp.topk_idx, inp.topk_weights, E, R, L)
    L2 = O.layout(idx2, E, R, C)
    b = O.dispatch(inp.x, idx2, inp.topk_weights, E, R, L2)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    return L


def check_combine_rank_mask(seed=0, T=80, H=48, E=24, K=4, R=6, C=3):
    """A rank masked at combine time contributes nothing: the result equals
    the unmasked combine of rows (and weights) in which that rank's segment
    holds +0.  The fp32 accumulator starts at +0 and so never becomes -0;
    adding +0 then leaves every value unchanged, which makes the two
    bit-identical.  The identity combine counts only unmasked hits."""
    inp = random_case(seed, T, H, E, K, R, C, mask=0.15)
    L, rx, rtw = check_dispatch_props(inp)
    rng = np.random.default_rng(seed + 11)
    m = (rng.random(R) < 0.4).astype(np.int32)
    m[0], m[-1] = 1, 0
    yf = rng.standard_normal((L.num_recv, H)).astype(np.float32)
    y = (yf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out, cw = O.combine(y, L, rtw, rank_mask=m)
    y0, w0 = y.copy(), rtw.copy()
    for r in np.nonzero(m)[0]:
        a = L.rank_prefix_matrix[r - 1] if r > 0 else 0
        b = L.rank_prefix_matrix[r]
        y0[a:b] = 0
        w0[a:b] = 0
    out0, cw0 = O.combine(y0, L, w0)
    np.testing.assert_array_equal(out, out0)
    np.testing.assert_array_equal(cw.view(np.uint32), cw0.view(np.uint32))
    # identity: n'_t unmasked copies of x_t sum exactly
    outi, cwi = O.combine(rx, L, rtw, rank_mask=m)
    n = (L.is_token_in_rank.astype(np.float32) * (1 - m)[None, :]).sum(axis=1)
    exp = torch_bf16_bits(f32_from_bits(inp.x) * n[:, None])
    np.testing.assert_array_equal(f32_from_bits(outi), f32_from_bits(exp))
    epr = E // R
    live = (inp.topk_idx >= 0) & (m[np.maximum(inp.topk_idx, 0) // epr] == 0)
    np.testing.assert_array_equal(cwi, np.where(live, inp.topk_weights, np.float32(0)))
    # nothing masked = the plain combine
    outn, cwn = O.combine(y, L, rtw, rank_mask=np.zeros(R, np.int32))
    outp, cwp = O.combine(y, L, rtw)
    np.testing.assert_array_equal(outn, outp)
    np.testing.assert_array_equal(cwn, cwp)
    return m


# -------------------------------------------------------------- combine bias


def check_combine_bias(seed=0, T=96, H=40, E=24, K=4, R=6, C=3):
    inp = random_case(seed, T, H, E, K, R, C, mask=0.2)
    L = O.layout(inp.topk_idx, E, R, C)
    rng = np.random.default_rng(seed + 21)
    y = (rng.standard_normal((L.num_recv, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    zero = np.zeros((T, H), np.uint16)
    a, _ = O.combine(y, L)
    b, _ = O.combine(y, L, bias0=zero, bias1=zero)
    np.testing.assert_array_equal(f32_from_bits(a), f32_from_bits(b))  # +0 bias changes nothing
    # zero rows: the output is the bias sum, exact for small integers
    b0 = rng.integers(-20, 21, (T, H)).astype(np.float32)
    b1 = rng.integers(-20, 21, (T, H)).astype(np.float32)
    out, _ = O.combine(np.zeros_like(y), L, bias0=bits_from_f32_exact(b0),
                       bias1=bits_from_f32_exact(b1))
    np.testing.assert_array_equal(f32_from_bits(out), b0 + b1)
    # integer rows and integer biases: exact total
    yi = rng.integers(-8, 9, (L.num_recv, H)).astype(np.float32)
    out, _ = O.combine(bits_from_f32_exact(yi), L, bias0=bits_from_f32_exact(b0))
    exp = b0.copy()
    for r in range(R):
        S = L.rank_prefix_matrix[r - 1] if r > 0 else 0
        ts = np.nonzero(L.send_head[:, r] >= 0)[0]
        exp[ts] += yi[S + L.send_head[ts, r]]
    np.testing.assert_array_equal(f32_from_bits(out), exp)
    # only bias1 given: the same as bias0 alone with those values
    o1, _ = O.combine(y, L, bias1=bits_from_f32_exact(b1))
    o0, _ = O.combine(y, L, bias0=bits_from_f32_exact(b1))
    np.testing.assert_array_equal(f32_from_bits(o1), f32_from_bits(o0))


# ------------------------------------------------------------ load balancing


def check_lb_ops(seed=0, E=12, n_rep=7, P=37):
    rng = np.random.default_rng(seed)
    mapping = rng.integers(-1, E, n_rep).astype(np.int64)
    mapping[0] = E + 3  # an invalid entry is ignored
    mapping[1] = mapping[n_rep - 1] = 2  # an expert with two replicas, far apart
    ew = rng.integers(-30, 31, (E, P)).astype(np.float32)
    rg = rng.integers(-30, 31, (n_rep, P)).astype(np.float32)
    # reduce: small integers sum exactly; replicas in any order give the same
    out = f32_from_bits(O.lb_reduce_grads(bits_from_f32_exact(rg), bits_from_f32_exact(ew), mapping))
    exp = ew.copy()
    for j in range(n_rep):
        if 0 <= mapping[j] < E:
            exp[mapping[j]] += rg[j]
    np.testing.assert_array_equal(out, exp)
    # zero replica gradients leave every expert bitwise unchanged (even -0)
    egb = (rng.standard_normal((E, P)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out0 = O.lb_reduce_grads(np.zeros((n_rep, P), np.uint16), egb, mapping)
    np.testing.assert_array_equal(f32_from_bits(out0), f32_from_bits(egb))
    # fp64 bound on random values: n terms summed in fp32 then rounded once
    rgb = (rng.standard_normal((n_rep, P)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = f32_from_bits(O.lb_reduce_grads(rgb, egb, mapping)).astype(np.float64)
    ex = f32_from_bits(egb).astype(np.float64)
    ab = np.abs(ex).copy()
    cnt = np.ones(E)
    for j in range(n_rep):
        if 0 <= mapping[j] < E:
            v = f32_from_bits(rgb[j]).astype(np.float64)
            ex[mapping[j]] += v
            ab[mapping[j]] += np.abs(v)
            cnt[mapping[j]] += 1
    err = np.abs(got - ex)
    bound = (cnt[:, None] - 1) * 2.0 ** -24 * ab * 1.0001 + 0.5 * _bf16_ulp(np.maximum(np.abs(got), np.abs(ex)))
    assert np.all(err <= bound)
    # prefetch copies each replica's source row; invalid entries stay as they were
    rw0 = rng.integers(0, 65535, (n_rep, P)).astype(np.uint16)
    rw = O.lb_prefetch_weights(egb, rw0, mapping)
    for j in range(n_rep):
        if 0 <= mapping[j] < E:
            np.testing.assert_array_equal(rw[j], egb[mapping[j]])
        else:
            np.testing.assert_array_equal(rw[j], rw0[j])
    # prefetch then reduce of the copied values doubles each replicated row
    once = np.bincount(mapping[(mapping >= 0) & (mapping < E)], minlength=E)
    ewi = rng.integers(-30, 31, (E, P)).astype(np.float32)
    rwi = O.lb_prefetch_weights(bits_from_f32_exact(ewi), np.zeros((n_rep, P), np.uint16), mapping)
    red = f32_from_bits(O.lb_reduce_grads(rwi, bits_from_f32_exact(ewi), mapping))
    np.testing.assert_array_equal(red, ewi * (1 + once)[:, None])


# ---------------------------------------------------------------------- FP8


def e4m3_table():
    """The 256 codes decoded from the format definition (sign, 4-bit exponent
    with bias 7, 3-bit mantissa, subnormals at exponent 0, 0x7F/0xFF NaN)."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        ex, m = (c >> 3) & 15, c & 7
        if ex == 15 and m == 7:
            vals[c] = np.nan
        elif ex == 0:
            vals[c] = s * m * 2.0 ** -9
        else:
            vals[c] = s * (1 + m / 8) * 2.0 ** (ex - 7)
    return vals


def brute_e4m3(f):
    """Nearest finite code by exhaustive search; ties go to the even code
    (mantissa lsb 0); values beyond 448 saturate; sign of zero kept."""
    vals = e4m3_table()
    out = np.empty(f.shape, np.uint8)
    fin = np.arange(256)[~np.isnan(vals)]
    for i, v in enumerate(np.asarray(f, np.float64).ravel()):
        if np.isnan(v):
            out.flat[i] = 0x7F
            continue
        v2 = min(max(v, -448.0), 448.0)
        d = np.abs(vals[fin] - v2)
        best = fin[d == d.min()]
        if len(best) > 1:
            best = best[(best & 1) == 0]
            if len(best) > 1:  # +0 / -0: keep the sign of the input
                best = best[(best & 0x80) == (0x80 if np.signbit(v) else 0)]
        out.flat[i] = best[0]
    return out


def check_e4m3(seed=0):
    vals = e4m3_table()
    for c in range(256):
        got = O.e4m3_to_f32(c)
        assert (np.isnan(got) and np.isnan(vals[c])) or got == vals[c], c
    # torch's own float8_e4m3fn decoding agrees with the format definition
    tv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ok = ~np.isnan(vals)
    np.testing.assert_array_equal(tv[ok], vals[ok].astype(np.float32))
    # every code, every midpoint between neighbours (ties), and points next to them
    fin = np.sort(np.unique(vals[~np.isnan(vals)]))
    mids = (fin[:-1] + fin[1:]) / 2
    pts = np.concatenate([fin, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                          np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
                          [449.0, 463.9, 464.0, 465.0, 1e6, -1e6, 1e-12, -1e-12, -0.0]])
    rng = np.random.default_rng(seed)
    rnd = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000))).astype(np.float32)
    pts = np.concatenate([pts.astype(np.float32), rnd])
    np.testing.assert_array_equal(O.f32_to_e4m3(pts), brute_e4m3(pts))
    # torch's rounding conversion agrees inside the finite range
    inr = pts[np.abs(pts) <= 448]
    tq = torch.from_numpy(inr).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.f32_to_e4m3(inr), tq)
    # the format has no infinity: NaN encodes to a NaN code (0x7F or 0xFF, the
    # sign is left open), and infinities saturate to +-448 like any value
    # past the largest finite one
    nan_codes = O.f32_to_e4m3(np.array([np.nan, -np.nan], np.float32))
    assert all(int(c) & 0x7F == 0x7F for c in nan_codes), nan_codes
    np.testing.assert_array_equal(O.f32_to_e4m3(np.array([np.inf, -np.inf], np.float32)),
                                  np.array([0x7E, 0xFE], np.uint8))


def check_ll_fp8(inp, rank_mask=None):
    """Metadata equals the bf16 dispatch's; each block's scale is amax/448
    (amax clamped at 1e-4); every code is the rounding of x * (448/amax); and
    dequantized rows are within half an e4m3 step (times the scale) of x."""
    E, R, S = inp.E, inp.R, inp.slots
    q, sc, cnt, src, ts = O.ll_dispatch_fp8(inp.x, inp.topk_idx, E, R, S, rank_mask=rank_mask)
    _, cnt2, src2, ts2 = O.ll_dispatch(inp.x, inp.topk_idx, E, R, S, with_buf=False,
                                       rank_mask=rank_mask)
    np.testing.assert_array_equal(cnt, cnt2)
    np.testing.assert_array_equal(src, src2)
    np.testing.assert_array_equal(ts, ts2)
    H = inp.x.shape[1]
    vals = e4m3_table()
    used = src >= 0
    xs = f32_from_bits(inp.x)[src[used]]                     # [n, H]
    qs = q[used].astype(np.int64)
    ss = sc[used]                                            # [n, H/128]
    blocks = xs.reshape(len(xs), H // 128, 128)
    amax = np.maximum(np.abs(blocks).max(axis=2), np.float32(1e-4)).astype(np.float32)
    np.testing.assert_array_equal(ss, (amax / np.float32(448.0)).astype(np.float32))
    sinv = (np.float32(448.0) / amax).astype(np.float32)
    scaled = (blocks * sinv[:, :, None]).astype(np.float32)
    np.testing.assert_array_equal(qs.reshape(scaled.shape), O.f32_to_e4m3(scaled).astype(np.int64))
    deq = vals[qs].reshape(scaled.shape) * ss[:, :, None]
    # half a step of e4m3 around the scaled value: step = 2^(e-3) for normals, 2^-9 below
    a = np.maximum(np.abs(scaled.astype(np.float64)), 2.0 ** -6)
    step = 2.0 ** (np.floor(np.log2(a)) - 3)
    err = np.abs(deq - blocks)
    assert np.all(err <= (0.5 * step + 1e-6 * a) * ss[:, :, None] * 1.0001 + 1e-30)
    assert np.all(q[~used] == 0)
    return q, sc


def fp8_nonfinite_case(seed=5):
    """A decode batch with infinities and NaNs in some 128-element blocks:
    a lone +inf, a lone -inf, lone NaNs of both signs, an all-NaN block and
    a block holding both an infinity and a NaN."""
    inp = random_case(seed, 40, 512, 16, 4, 4, 1, slots=40)
    x = inp.x.copy()
    x[0, 5] = 0x7F80        # +inf in block 0
    x[0, 200] = 0xFF80      # -inf in block 1
    x[1, 300] = 0x7FC0      # NaN in block 2
    x[1, 301] = 0xFFC1      # negative NaN, same block
    x[2, 0:128] = 0x7FC0    # a block of NaNs only
    x[3, 384] = 0x7F80      # +inf and NaN in block 3
    x[3, 385] = 0xFFC0
    inp.x = x
    return inp


def e4m3_is_nan(code):
    return (np.asarray(code) & 0x7F) == 0x7F


def check_ll_fp8_nonfinite():
    """IEEE arithmetic carried through the FP8 recipe: NaNs do not raise a
    block's amax (max ignores them), an infinite amax makes the scale infinite
    and 448/amax zero, so finite values become signed zeros and infinities
    (inf * 0) and NaNs become NaN codes.  The sign of a NaN is not fixed by
    IEEE 754, so only NaN-ness is checked there."""
    inp = fp8_nonfinite_case()
    E, R, S = inp.E, inp.R, inp.slots
    q, sc, _, src, _ = O.ll_dispatch_fp8(inp.x, inp.topk_idx, E, R, S)
    xf = f32_from_bits(inp.x)
    checked = 0
    for le in range(E // R):
        for r in range(R):
            for s_ in range(S):
                t = src[le, r, s_]
                if t < 0 or t > 3:
                    continue
                for b in range(inp.x.shape[1] // 128):
                    blk = xf[t, b * 128:(b + 1) * 128]
                    code = q[le, r, s_, b * 128:(b + 1) * 128].astype(np.int64)
                    fin = np.isfinite(blk)
                    finite_amax = np.abs(blk[~np.isnan(blk)]).max(initial=0.0)
                    if np.isinf(finite_amax):
                        assert np.isinf(sc[le, r, s_, b])
                        assert np.all(e4m3_is_nan(code[~fin]))
                        assert np.all(code[fin] == np.where(np.signbit(blk[fin]), 0x80, 0))
                    else:
                        amax = np.float32(max(finite_amax, np.float32(1e-4)))
                        assert sc[le, r, s_, b] == np.float32(amax / np.float32(448.0))
                        assert np.all(e4m3_is_nan(code[np.isnan(blk)]))
                        sinv = np.float32(np.float32(448.0) / amax)
                        exp = O.f32_to_e4m3((blk[fin] * sinv).astype(np.float32)).astype(np.int64)
                        np.testing.assert_array_equal(code[fin], exp)
                    checked += 1
    assert checked >= 16
    return q, sc


def check_ll_combine_fp8(inp, rank_mask=None, seed=0):
    """The FP8 LL combine reduces to the (pinned) bf16 LL combine: every
    e4m3 value is exact in bf16, and a power-of-two scale keeps it exact, so
    with such scales the decoded, scaled payload is a bf16 buffer and both
    combines must agree bit for bit.  Each 128-element block gets its own
    scale 2^k (k from -3 to 3), which pins the scale indexing.  A dispatch /
    combine round trip stays within the quantization error of the bf16 one."""
    E, R, S = inp.E, inp.R, inp.slots
    H = inp.x.shape[1]
    epr = E // R
    nb = H // 128
    rng = np.random.default_rng(seed + 91)
    q = rng.integers(0, 256, (epr, R, S, H)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3A          # no NaN codes in this pin
    k = rng.integers(-3, 4, (epr, R, S, nb))
    sc = np.ldexp(np.ones((epr, R, S, nb)), k).astype(np.float32)
    vals = e4m3_table()
    deq = (vals[q.astype(np.int64)] * np.repeat(sc, 128, axis=3)).astype(np.float32)
    buf = bits_from_f32_exact(deq.reshape(-1, H)).reshape(deq.shape)
    w = inp.topk_weights
    a = O.ll_combine_fp8(q, sc, inp.topk_idx, w, E, R, rank_mask=rank_mask)
    b = O.ll_combine(buf, inp.topk_idx, w, E, R, rank_mask=rank_mask)
    np.testing.assert_array_equal(a, b)
    # unit scales: the codes' own values
    ones = np.ones_like(sc)
    buf1 = bits_from_f32_exact(vals[q.astype(np.int64)].astype(np.float32).reshape(-1, H))
    np.testing.assert_array_equal(O.ll_combine_fp8(q, ones, inp.topk_idx, w, E, R, rank_mask=rank_mask),
                                  O.ll_combine(buf1.reshape(q.shape), inp.topk_idx, w, E, R,
                                               rank_mask=rank_mask))
    # combine-time mask: a masked rank's terms drop out as in the bf16 combine
    cm = np.zeros(R, np.int32)
    cm[R // 2] = 1
    np.testing.assert_array_equal(
        O.ll_combine_fp8(q, sc, inp.topk_idx, w, E, R, combine_mask=cm),
        O.ll_combine(buf, inp.topk_idx, w, E, R, combine_mask=cm))
    # round trip through the FP8 dispatch
    fq, fs, _, _, _ = O.ll_dispatch_fp8(inp.x, inp.topk_idx, E, R, S, rank_mask=rank_mask)
    rt = f32_from_bits(O.ll_combine_fp8(fq, fs, inp.topk_idx, w, E, R, rank_mask=rank_mask))
    bq, _, _, _ = O.ll_dispatch(inp.x, inp.topk_idx, E, R, S, rank_mask=rank_mask)
    ref = f32_from_bits(O.ll_combine(bq, inp.topk_idx, w, E, R, rank_mask=rank_mask))
    # each term moves by at most half an e4m3 step of its block (<= 2^-4 of
    # the block's amax); the weights of a token sum to at most 1
    xs = np.abs(f32_from_bits(inp.x)).reshape(inp.T, nb, 128).max(axis=2)
    bound = np.repeat(xs.max(axis=0, keepdims=True), 128, axis=1) * 2.0 ** -4 + 2.0 ** -6 * np.abs(ref)
    assert np.all(np.abs(rt - ref) <= bound * 1.01 + 1e-6)
    return a


# -------------------------------------------------------- exact tie rounding


def check_tie_rounding():
    """Sums that land exactly on a bf16 tie (halfway between neighbours) must
    round to the even neighbour; any perturbation of the sum (a scaled term, a
    lost term, a different rounding) moves it off the tie and flips the
    result.  Every term and partial sum here is exact in fp32."""
    # normal combine: token 0 sends to ranks 0 and 1 of R=2 (experts 0, 1)
    idx = np.array([[0, 1], [1, -1], [-1, -1]], np.int64)
    L = O.layout(idx, 2, 2, 1)
    rows = np.array([[1.0, 1.0, -3.0, 256.0],             # row of (token 0, rank 0)
                     [2.0 ** -8, 3 * 2.0 ** -8, -2.0 ** -7 * 3, 1.0],  # (token 0, rank 1)
                     [1.0 + 2.0 ** -7, 0.0, 0.0, 0.0]], np.float32)    # (token 1, rank 1)
    # rows are in segment order: rank 0 = [t0], rank 1 = [t0, t1]
    out, _ = O.combine(bits_from_f32_exact(rows), L)
    got = f32_from_bits(out)
    # 1 + 2^-8: tie between 1 and 1 + 2^-7 -> even 1;  1 + 3*2^-8: tie -> even 1 + 2^-6
    # -3 - 3*2^-7 = -3.0234375: tie between -3.015625 (odd mantissa) and -3.03125 (even) ->
    # -3.03125;  256 + 1: tie between 256 (even) and 258 -> 256
    np.testing.assert_array_equal(got[0], np.array([1.0, 1.0 + 2.0 ** -6, -3.03125, 256.0], np.float32))
    np.testing.assert_array_equal(got[1], rows[2])
    # LL combine: one token, experts 0, 1, 2 on one rank, one slot each
    idx = np.array([[0, 1, 2]], np.int64)
    w = np.array([[0.5, 0.5, 0.0]], np.float32)
    b = np.zeros((3, 1, 1, 8), np.float32)
    b[1, 0, 0, 0] = 1.0
    # 0.5 * (1 + 2^-7) + 0.5 * 1 = 1 + 2^-8: a tie -> even 1.0
    b[0, 0, 0, 0] = 1.0 + 2.0 ** -7
    out = f32_from_bits(O.ll_combine(bits_from_f32_exact(b), idx, w, 3, 1))
    assert out[0, 0] == np.float32(1.0)
    # 0.5 * (1 + 3*2^-7) + 0.5 = 1 + 3*2^-8: a tie between 1 + 2^-7 and 1 + 2^-6 -> even 1 + 2^-6
    b[0, 0, 0, 0] = 1.0 + 3 * 2.0 ** -7
    out = f32_from_bits(O.ll_combine(bits_from_f32_exact(b), idx, w, 3, 1))
    assert out[0, 0] == np.float32(1.0 + 2.0 ** -6)
    # lb_reduce_grads: the same two ties
    eg = bits_from_f32_exact(np.array([[1.0, -3.0]], np.float32))
    rg = bits_from_f32_exact(np.array([[2.0 ** -8, -3 * 2.0 ** -7]], np.float32))
    got = f32_from_bits(O.lb_reduce_grads(rg, eg, np.array([0], np.int64)))
    np.testing.assert_array_equal(got, np.array([[1.0, -3.03125]], np.float32))


def check_sum_order():
    """Every sum's order is fixed by a reading: the combine adds ranks in
    ascending order, the LL combine slots k in ascending order, and
    lb_reduce_grads the expert's own gradient and then its replicas in
    ascending order.  fp32 sums depend on that order when small terms land on
    ties.  With the terms 1, 2^-8, 2^-24, 2^-24 in that order, each 2^-24 is
    exactly half an fp32 ulp of 1 + 2^-8 and is dropped (ties to even).  That
    leaves 1 + 2^-8, a bf16 tie that rounds to 1.0.  In the opposite order the
    two 2^-24 first make 2^-23, the total 1 + 2^-8 + 2^-23 is exact and above
    the tie, and it rounds to 1 + 2^-7.  Each case checks both orders of the
    input, so the pin also shows that the order matters."""
    terms = np.array([1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24], np.float32)
    fwd, rev = np.float32(1.0), np.float32(1.0 + 2.0 ** -7)
    # normal combine: one token on experts 0..3, one expert per rank (R = 4);
    # the packed row of rank r holds terms[r]
    L = O.layout(np.array([[0, 1, 2, 3]], np.int64), 4, 4, 1)
    for t, want in ((terms, fwd), (terms[::-1], rev)):
        rows = np.repeat(np.ascontiguousarray(t)[:, None], 8, axis=1)
        out, _ = O.combine(bits_from_f32_exact(rows), L)
        assert (f32_from_bits(out) == want).all(), "combine rank order"
    # LL combine: one token, experts 0..3 on one rank, one slot each, unit weights
    idx = np.array([[0, 1, 2, 3]], np.int64)
    w = np.ones((1, 4), np.float32)
    for t, want in ((terms, fwd), (terms[::-1], rev)):
        b = np.repeat(np.ascontiguousarray(t)[:, None], 8, axis=1).reshape(4, 1, 1, 8)
        out = f32_from_bits(O.ll_combine(bits_from_f32_exact(b), idx, w, 4, 1))
        assert (out == want).all(), "LL combine slot order"
    # lb_reduce_grads: own gradient 0, then four replicas of expert 0
    for t, want in ((terms, fwd), (terms[::-1], rev)):
        rg = bits_from_f32_exact(np.repeat(np.ascontiguousarray(t)[:, None], 8, axis=1))
        eg = bits_from_f32_exact(np.zeros((1, 8), np.float32))
        got = f32_from_bits(O.lb_reduce_grads(rg, eg, np.zeros(4, np.int64)))
        assert (got == want).all(), "lb_reduce_grads replica order"


def check_fma_and_bias_order():
    """Two more fixed roundings.  The LL combines add each weighted term with
    one fused multiply-add: with slot 0 holding -(1 + 2^-7) at weight 1 and
    slot 1 holding 1 + 2^-7 at weight 1 + 2^-17, the exact product of slot 1
    is 1 + 2^-7 + 2^-17 + 2^-24, so the fused sum is 2^-17 + 2^-24 (exact in
    bf16).  A separate product would first round the 2^-24 away (an fp32 tie)
    and give 2^-17.  The FP8 combine gets the same terms from the codes of
    -1 and 1 with the block scale 1 + 2^-7, whose product is exact in fp32.
    The normal combine adds the bias terms after the rank sum: rank rows 1 and
    2^-8 then two biases of 2^-24 give 1 + 2^-8 (each bias lost at a tie), so
    bf16 1.0.  Biases added first would make 2^-23 and give 1 + 2^-7."""
    fused = np.float32(2.0 ** -17 + 2.0 ** -24)
    idx = np.array([[0, 1]], np.int64)
    w = np.array([[1.0, 1.0 + 2.0 ** -17]], np.float32)
    # bf16 LL combine: experts 0, 1 on one rank, one slot each
    b = np.zeros((2, 1, 1, 8), np.float32)
    b[0] = -(1.0 + 2.0 ** -7)
    b[1] = 1.0 + 2.0 ** -7
    out = f32_from_bits(O.ll_combine(bits_from_f32_exact(b), idx, w, 2, 1))
    assert (out == fused).all(), "LL combine fma"
    # FP8 LL combine: codes of -1 (0xB8) and 1 (0x38), scale 1 + 2^-7
    assert O.e4m3_to_f32(0x38) == 1.0 and O.e4m3_to_f32(0xB8) == -1.0
    q = np.zeros((2, 1, 1, 128), np.uint8)
    q[0] = 0xB8
    q[1] = 0x38
    sc = np.full((2, 1, 1, 1), 1.0 + 2.0 ** -7, np.float32)
    out = f32_from_bits(O.ll_combine_fp8(q, sc, idx, w, 2, 1))
    assert (out == fused).all(), "FP8 LL combine fma"
    # normal combine: one token on experts 0, 1 (ranks 0, 1), two biases
    L = O.layout(idx, 2, 2, 1)
    rows = bits_from_f32_exact(np.repeat(np.array([[1.0], [2.0 ** -8]], np.float32), 8, axis=1))
    bias = bits_from_f32_exact(np.full((1, 8), 2.0 ** -24, np.float32))
    out, _ = O.combine(rows, L, bias0=bias, bias1=bias)
    assert (f32_from_bits(out) == np.float32(1.0)).all(), "bias after the rank sum"


def fp8_edge_case(seed=4):
    """A decode batch whose rows hold an all-zero block and a block of values
    far below the amax floor, next to ordinary blocks."""
    inp = random_case(seed, 40, 256, 16, 4, 4, 1, mask=0.2, slots=40)
    x = inp.x.copy()
    x[0, :128] = 0
    x[1, 128:] = bits_from_f32_exact(np.full(128, 2.0 ** -20, np.float32))
    x[2, :64] = 0x8000  # -0
    inp.x = x
    return inp
