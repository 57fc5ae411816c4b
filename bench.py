#!/usr/bin/env python3
"""Benchmark of the expert-parallel hot path on one MI355X.

One step = one pass of every hot-path operation over one batch of synthetic
input, all on torch's current stream, through the C ABI:

  training-scale batch (T=4096, H=7168, E=256, K=8, R=64 ranks, C=10 channels)
    1. layout            ep_get_dispatch_layout   -> handle
    2. dispatch          ep_dispatch(handle, x, topk_idx, topk_weights)   rows + top-k outputs
    3. cached dispatch   ep_dispatch(handle, x2)                          rows only
    4. combine           ep_combine(handle, y = rows of 2, weights of 2)
    5. handle free
  low-latency decode batch (T=128, H=7168, E=256, K=8, R=32, 128 slots)
    6. LL dispatch       ep_ll_dispatch
    7. LL combine        ep_ll_combine(packed rows of 6)

Inputs are generated and copied to HBM before timing; successive steps use
four copies of the token batches in turn (470 MB, more than the last-level
cache), so each dispatch reads its rows from HBM, and two copies of each
packed-row buffer, so no dispatch overwrites rows still dirty in a cache.  Device buffers are sized
for the worst case (T*min(K,R) rows), so no step synchronizes the host.
``value`` is whole-job throughput: the algorithmic bytes of all operations
divided by the wall time of the timed steps, which hold no event (an event
marker costs the stream about 5 us).  A second pass of the same steps brackets
only the dispatch call, which launches one kernel, with HIP events on the
launch stream: that is the roofline figure.  Per-operation times come from a
third, instrumented pass with events around every call (each call launches
one kernel, except the layout: two); for the cached dispatch, the combine and
the two LL operations ``back_to_back_us`` adds the time per call of the same
operation timed back to back (one event pair around many calls).

Algorithmic bytes (what the method must move; x read once, only the N copied
rows' positions read):
  dispatch        (T+N)*H*2 + N*4 + T*K*12 + N*K*12
  cached dispatch (T+N)*H*2 + N*4
  combine         (N+T)*H*2 + N*4 + N*K*4 + T*K*4
  layout          T*K*8 + T*R*5 + N*4
  LL dispatch     T*H*2 + M*H*2 + T*K*12 + M*4      (M valid (token, slot) pairs)
  LL combine      M*H*2 + T*H*2 + T*K*16
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch & combine HBM GB/s (% of peak) at T=4096,H=7168,K=8,R=64; layout Mtok/s"
HBM_PEAK_GBS = 8000.0
TRAIN = dict(T=4096, H=7168, E=256, K=8, R=64, C=10)
DECODE = dict(T=128, H=7168, E=256, K=8, R=32, slots=128)
PROFILES = os.path.join(ROOT, "profiles")
NBUF = 4


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU work budget of the oracle baseline leg (0 = skip)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the skewed and large workloads (profiling runs: their launches "
                        "would mix into the per-kernel figures of the training-scale batch)")
    return p.parse_args()


def kernel_source_sha(name: str) -> str:
    path = os.path.join(ROOT, "combine_get_dispatch_05_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_file: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "traffic_training_T4096_H7168_K8_R64.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_sha") != kernel_source_sha(kernel_file):
        return None
    return ent.get("hbm_bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the hot path on one GPU only (the R ranks are logical "
              "partitions of one GPU's HBM); --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_get_dispatch_05_amd as epm
    from combine_get_dispatch_05_amd import abi
    from gen import config_inputs, random_rows

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    L = abi.lib()
    dev = torch.device("cuda", 0)

    def to_dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return t.view(dtype) if dtype is not None else t

    # ---------------------------------------------------------------- inputs
    tr = config_inputs(1)
    assert (tr.T, tr.H, tr.E, tr.K, tr.R, tr.C) == tuple(TRAIN[k] for k in "THEKRC")
    T, H, E, K, R, C = tr.T, tr.H, tr.E, tr.K, tr.R, tr.C
    # NBUF copies of each token batch, used in turn: 4 x (x, x2) = 470 MB is
    # more than the 256 MB last-level cache, so every dispatch reads its rows
    # from HBM rather than from rows a previous step left in the cache.
    x0 = to_dev(tr.x.view(np.int16), torch.bfloat16)
    x20 = to_dev(random_rows(T, H, 0, tag=11).view(np.int16), torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(NBUF - 1)]
    x2s = [x20] + [x20.clone() for _ in range(NBUF - 1)]
    topk = to_dev(tr.topk_idx)
    w = to_dev(tr.topk_weights)
    d = abi.dims(T, H, K, E, R, C)
    cap = int(L.ep_max_recv_rows(ctypes.byref(d)))
    # Two packed-row buffers per dispatch, used in turn, so a dispatch never
    # overwrites rows that the previous step may still hold dirty in a cache.
    recv_xs = [torch.empty((cap, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    recv_x2s = [torch.empty((cap, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    rti = torch.empty((cap, K), dtype=torch.int64, device=dev)
    rtw = torch.empty((cap, K), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    cw = torch.empty((T, K), dtype=torch.float32, device=dev)

    dc = config_inputs(3)
    dd = abi.dims(dc.T, dc.H, dc.K, dc.E, dc.R, 1)
    S = dc.slots
    epr = dc.E // dc.R
    lx = to_dev(dc.x.view(np.int16), torch.bfloat16)
    ltopk = to_dev(dc.topk_idx)
    lw = to_dev(dc.topk_weights)
    packed = torch.empty((epr, dc.R, S, dc.H), dtype=torch.bfloat16, device=dev)
    lcount = torch.empty((epr, dc.R), dtype=torch.int32, device=dev)
    lsrc = torch.empty((epr, dc.R, S), dtype=torch.int32, device=dev)
    lslot = torch.empty((dc.T, dc.K), dtype=torch.int32, device=dev)
    lout = torch.empty((dc.T, dc.H), dtype=torch.bfloat16, device=dev)

    P = abi.ptr
    ops = ["layout", "dispatch", "dispatch_cached", "combine", "ll_dispatch", "ll_combine"]

    counter = [0]

    def step(events=None, roof_events=None):
        s = abi.current_stream()
        x = xs[counter[0] % NBUF]
        x2 = x2s[counter[0] % NBUF]
        recv_x = recv_xs[counter[0] % 2]
        recv_x2 = recv_x2s[counter[0] % 2]
        counter[0] += 1

        def mark(i):
            if events is not None:
                events[i].record()

        h = ctypes.c_void_p()
        mark(0)
        abi.check(L.ep_get_dispatch_layout(ctypes.byref(d), P(topk), None, None, ctypes.byref(h),
                                           s), "layout")
        mark(1)
        if roof_events is not None:
            roof_events[0].record()
        abi.check(L.ep_dispatch(ctypes.byref(d), P(x), P(topk), P(w), None, ctypes.byref(h),
                                P(recv_x), P(rti), P(rtw), cap, None, s), "dispatch")
        if roof_events is not None:
            roof_events[1].record()
        mark(2)
        abi.check(L.ep_dispatch(ctypes.byref(d), P(x2), None, None, None, ctypes.byref(h),
                                P(recv_x2), None, None, cap, None, s), "cached dispatch")
        mark(3)
        abi.check(L.ep_combine(h, H, P(recv_x), cap, P(rtw), None, None, None, P(out), P(cw), s),
                  "combine")
        mark(4)
        L.ep_handle_free(h)
        abi.check(L.ep_ll_dispatch(ctypes.byref(dd), S, P(lx), P(ltopk), None, P(packed),
                                   P(lcount), P(lsrc), P(lslot), s), "ll dispatch")
        mark(5)
        abi.check(L.ep_ll_combine(ctypes.byref(dd), S, P(packed), P(ltopk), P(lw), P(lslot),
                                  None, P(lout), s), "ll combine")
        mark(6)

    # N and M for the byte counts
    step()
    torch.cuda.synchronize()
    h = ctypes.c_void_p()
    abi.check(L.ep_get_dispatch_layout(ctypes.byref(d), P(topk), None, None, ctypes.byref(h),
                                       abi.current_stream()), "layout")
    n = ctypes.c_int64()
    abi.check(L.ep_handle_num_recv(h, ctypes.byref(n)), "num_recv")
    L.ep_handle_free(h)
    N = int(n.value)
    M = int((dc.topk_idx >= 0).sum())

    by = {
        "layout": T * K * 8 + T * R * 5 + N * 4,
        "dispatch": (T + N) * H * 2 + N * 4 + T * K * 12 + N * K * 12,
        "dispatch_cached": (T + N) * H * 2 + N * 4,
        "combine": (N + T) * H * 2 + N * 4 + N * K * 4 + T * K * 4,
        "ll_dispatch": dc.T * dc.H * 2 + M * dc.H * 2 + dc.T * dc.K * 12 + M * 4,
        "ll_combine": M * dc.H * 2 + dc.T * dc.H * 2 + dc.T * dc.K * 16,
    }
    step_bytes = sum(by.values())

    # ---------------------------------------------------------------- timing
    # Timed region: K whole steps with no event inside (every event marker
    # costs the stream about 5 us, which is measurement, not work).  The
    # roofline pass then runs the same K steps again with HIP events around
    # the dispatch pack call only (one kernel, on the stream it runs on); the
    # per-operation table comes from a third, fully instrumented pass.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    roof = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(roof_events=roof[i])
    torch.cuda.synchronize()
    roof_us = [1e3 * e[0].elapsed_time(e[1]) for e in roof]

    # Instrumented pass (not part of ``value``): events around every operation.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events=ev[i])
    torch.cuda.synchronize()

    per_op_ms = {op: [] for op in ops}
    for e in ev:
        for j, op in enumerate(ops):
            per_op_ms[op].append(e[j].elapsed_time(e[j + 1]))
    avg_us = {op: 1e3 * float(np.mean(v)) for op, v in per_op_ms.items()}
    med_us = {op: 1e3 * float(np.median(v)) for op, v in per_op_ms.items()}
    min_us = {op: 1e3 * float(np.min(v)) for op, v in per_op_ms.items()}

    ms_per_step = 1e3 * wall / args.steps
    value = step_bytes / (wall / args.steps) / 1e9

    op_report = {}
    for op in ops:
        gbs = by[op] / (avg_us[op] * 1e-6) / 1e9
        op_report[op] = {"avg_us": round(avg_us[op], 2), "median_us": round(med_us[op], 2),
                         "min_us": round(min_us[op], 2), "bytes": by[op], "gbs": round(gbs, 1),
                         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    op_report["layout"]["mtok_s"] = round(T / (avg_us["layout"] * 1e-6) / 1e6, 2)
    op_report["layout"]["kernels"] = 2

    # Roofline of the dominant kernel (the dispatch pack with top-k outputs,
    # the largest byte count of the step), timed with events over K steps.
    dom_us = float(np.mean(roof_us))
    achieved = by["dispatch"] / (dom_us * 1e-6) / 1e9
    traffic = load_traffic("dispatch.hip", "dispatch:dispatch_scatter_kernel")
    roofline = {"bound": "hbm", "kernel": "dispatch_scatter_kernel (dispatch with top-k outputs)",
                "avg_us": round(dom_us, 2), "timed_over": f"{args.steps} steps, events around the "
                "dispatch call only", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}

    # ------------------------------------------- plain-copy practical ceiling
    # A device-to-device copy of a known size: its rate is the practical HBM
    # ceiling for read+write streams, and the HBM byte counters of this kernel
    # calibrate the counter readings of the path's kernels.
    copy_bytes = 512 << 20
    src = torch.empty(copy_bytes // 2, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record()
    for _ in range(10):
        dst.copy_(src)
    ce[1].record()
    torch.cuda.synchronize()
    copy_us = ce[0].elapsed_time(ce[1]) * 1e3 / 10
    copy_gbs = 2 * copy_bytes / (copy_us * 1e-6) / 1e9
    del src, dst

    # --------------------------------------------- same-traffic ceilings
    ceilings = measure_ceilings(args, L, abi, tr, d, xs, x2s, recv_xs, recv_x2s, rtw, out, cw,
                                cap, N, by, dc, dd, S, lx, ltopk, lw, packed, lcount, lsrc, lslot,
                                lout, topk, w)

    # ------------------------------------------- NEXT rows (not in ``value``)
    next_report = measure_next(args, L, abi, tr, dc, xs[0], topk, w, d, cap, recv_xs[0], rtw,
                               out, cw, packed, lcount, lsrc, lslot, lout, lx, ltopk, lw, dd, S,
                               epr)

    workloads = None if args.no_workloads else measure_workloads(args, L, abi)

    # The same operations timed back to back (one event pair around many
    # calls): for the latency-bound ones the per-call event markers above
    # cost as much as the kernel.
    for op in ("dispatch_cached", "combine", "ll_dispatch", "ll_combine"):
        if isinstance(ceilings, dict) and isinstance(ceilings.get(op), dict):
            op_report[op]["back_to_back_us"] = ceilings[op]["avg_us"]

    # ---------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        cpu = cpu_baseline(tr, dc, x2_bits=random_rows(T, H, 0, tag=11), budget=args.cpu_seconds,
                           step_bytes=step_bytes, op_bytes=by)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "training-scale EP layout+dispatch+cached dispatch+combine "
                        "(T=4096,H=7168,E=256,K=8,R=64,C=10, uniform distinct top-8) + "
                        "low-latency decode dispatch+combine (T=128,H=7168,E=256,K=8,R=32,"
                        "128 slots), one GPU",
            "T": T, "H": H, "E": E, "K": K, "R": R, "C": C, "N": N,
            "ll": {"T": dc.T, "R": dc.R, "slots": S, "M": M},
            "step_bytes": step_bytes,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "next": next_report,
        "workloads": workloads,
        "copy_ceiling": {"bytes_read_plus_written": 2 * copy_bytes, "avg_us": round(copy_us, 2),
                         "gbs": round(copy_gbs, 1),
                         "frac_hbm_peak": round(copy_gbs / HBM_PEAK_GBS, 4)},
        "ceilings": ceilings,
        "ops": op_report,
    }
    print(json.dumps(rec))


def measure_ceilings(args, L, abi, tr, d, xs, x2s, recv_xs, recv_x2s, rtw, out, cw, cap, N, by,
                     dc, dd, S, lx, ltopk, lw, packed, lcount, lsrc, lslot, lout, topk, w):
    """Each operation beside a probe kernel (libep_probe.so) that moves the
    same bytes in the simplest pattern there is, both timed back to back over
    ``args.steps`` calls with HIP events at the ends, on the same rotating
    inputs:
      cached dispatch  vs  pack probe (read each token row once, store it to
                           n_t planes) and write probe (the N rows' stores alone)
      combine          vs  reduce probe (read n_t planes per token, fp32 sum,
                           store one row)
      LL dispatch      vs  LL copy probe (the same grid and copy, cells known in
                           advance) and an empty kernel of the same grid
      LL combine       vs  LL reduce probe (the same grid, cells known)
    ``frac_of_ceiling`` = probe time / operation time."""
    import numpy as np
    import torch
    from combine_get_dispatch_05_amd import probe_abi

    PL = probe_abi.lib()
    P = abi.ptr
    dev = torch.device("cuda", 0)
    s = abi.current_stream()
    T, H, K, R = tr.T, tr.H, tr.K, tr.R
    n = args.steps

    def b2b(fn):
        for i in range(max(args.warmup, 2)):
            fn(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for i in range(n):
            fn(i)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / n

    # the dispatch's rows per token, from the layout
    h = ctypes.c_void_p()
    abi.check(L.ep_dispatch(ctypes.byref(d), P(xs[0]), P(topk), P(w), None, ctypes.byref(h),
                            P(recv_xs[0]), None, P(rtw), cap, None, s), "dispatch")
    itr = torch.empty((T, R), dtype=torch.uint8, device=dev)
    o = abi.LayoutOut(None, None, itr.data_ptr(), None, None, None, None, None, 0)
    abi.check(L.ep_handle_copy_layout(h, ctypes.byref(o), s), "copy layout")
    rows = itr.to(torch.int32).sum(dim=1).to(torch.int32).contiguous()
    kmax = min(K, R)
    assert int(rows.sum()) == N
    planes = [torch.empty((kmax, T, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    nb = len(xs)

    rep = {}

    def entry(name, us, nbytes):
        rep[name] = {"avg_us": round(us, 2), "bytes": nbytes,
                     "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}

    us_op = b2b(lambda i: abi.check(L.ep_dispatch(
        ctypes.byref(d), P(x2s[i % nb]), None, None, None, ctypes.byref(h), P(recv_x2s[i % 2]),
        None, None, cap, None, s), "cached dispatch"))
    entry("dispatch_cached", us_op, by["dispatch_cached"])
    us_pr = b2b(lambda i: probe_abi.check(PL.ep_probe_pack(P(x2s[i % nb]), T, H, P(rows), kmax,
                                                           P(planes[i % 2]), s), "pack probe"))
    entry("pack_probe", us_pr, (T + N) * H * 2)
    us_w = b2b(lambda i: probe_abi.check(PL.ep_probe_write(P(recv_x2s[i % 2]), N * H * 2, s),
                                         "write probe"))
    entry("write_probe", us_w, N * H * 2)
    us_c = b2b(lambda i: abi.check(L.ep_combine(h, H, P(recv_xs[i % 2]), cap, P(rtw), None, None,
                                                None, P(out), P(cw), s), "combine"))
    entry("combine", us_c, by["combine"])
    us_rp = b2b(lambda i: probe_abi.check(PL.ep_probe_reduce(P(planes[i % 2]), T, H, P(rows),
                                                             kmax, P(out), s), "reduce probe"))
    entry("reduce_probe", us_rp, (N + T) * H * 2)
    L.ep_handle_free(h)
    del planes

    # low-latency decode batch
    Td, Hd, Kd, Ed = dc.T, dc.H, dc.K, dc.E
    cells = torch.empty((Td * Kd, Hd), dtype=torch.bfloat16, device=dev)
    us_ld = b2b(lambda i: abi.check(L.ep_ll_dispatch(ctypes.byref(dd), S, P(lx), P(ltopk), None,
                                                     P(packed), P(lcount), P(lsrc), P(lslot), s),
                                    "ll dispatch"))
    entry("ll_dispatch", us_ld, by["ll_dispatch"])
    us_lp = b2b(lambda i: probe_abi.check(PL.ep_probe_ll_copy(P(lx), Td, Hd, Kd, P(cells), s),
                                          "ll copy probe"))
    entry("ll_copy_probe", us_lp, Td * Hd * 2 + Td * Kd * Hd * 2)
    # the LL dispatch's grid: T x 2 row slices + E/8 expert workgroups of 512 threads
    V = Hd // 8
    grid = Td * ((V + 511) // 512) + (Ed + 7) // 8
    us_le = b2b(lambda i: probe_abi.check(PL.ep_probe_empty(grid, 512, s), "empty"))
    rep["ll_empty_kernel"] = {"avg_us": round(us_le, 2), "blocks": grid, "threads": 512}
    us_lc = b2b(lambda i: abi.check(L.ep_ll_combine(ctypes.byref(dd), S, P(packed), P(ltopk),
                                                    P(lw), P(lslot), None, P(lout), s),
                                    "ll combine"))
    entry("ll_combine", us_lc, by["ll_combine"])
    us_lr = b2b(lambda i: probe_abi.check(PL.ep_probe_ll_reduce(P(cells), P(lw), Td, Hd, Kd,
                                                                P(lout), s), "ll reduce probe"))
    entry("ll_reduce_probe", us_lr, Td * Kd * Hd * 2 + Td * Hd * 2 + Td * Kd * 4)
    del cells

    rep["frac_of_ceiling"] = {
        "dispatch_cached_vs_pack_probe": round(us_pr / us_op, 4),
        "combine_vs_reduce_probe": round(us_rp / us_c, 4),
        "ll_dispatch_vs_ll_copy_probe": round(us_lp / us_ld, 4),
        "ll_combine_vs_ll_reduce_probe": round(us_lr / us_lc, 4),
    }
    rep["timed_over"] = f"{n} calls back to back, HIP events at the ends"
    return rep


def measure_next(args, L, abi, tr, dc, x, topk, w, d, cap, recv_x, rtw, out, cw, packed, lcount,
                 lsrc, lslot, lout, lx, ltopk, lw, dd, S, epr):
    """Per-call times (HIP events, mean of ``args.steps`` calls after warmup)
    of the operations beyond the step: low-latency calls with three ranks
    masked, the FP8 low-latency dispatch, combine with two bias rows, and the
    load-balance operations over the large workload's 32 redundant experts."""
    import numpy as np
    import torch
    from gen import config_inputs, random_rows

    P = abi.ptr
    dev = torch.device("cuda", 0)

    def timed(fn, n):
        for _ in range(max(args.warmup, 2)):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(n):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / n

    rep = {}
    T, H, K = tr.T, tr.H, tr.K
    s = abi.current_stream()
    # The layout with the N readback a fresh dispatch of unknown size needs
    # (ep_dispatch asked for N only: the count kernel stores N into pinned
    # host memory and the host polls it), host wall time per call, in a loop
    # and on an idle stream; and the same through a handle made without it
    # (N copied back later, one stream sync).
    def fresh_size_query():
        hl = ctypes.c_void_p()
        nn = ctypes.c_int64()
        abi.check(L.ep_dispatch(ctypes.byref(d), None, P(topk), None, None, ctypes.byref(hl), None,
                                None, None, 0, ctypes.byref(nn), s), "size query")
        L.ep_handle_free(hl)

    def layout_then_n():
        hl = ctypes.c_void_p()
        abi.check(L.ep_get_dispatch_layout(ctypes.byref(d), P(topk), None, None, ctypes.byref(hl),
                                           s), "layout")
        nn = ctypes.c_int64()
        abi.check(L.ep_handle_num_recv(hl, ctypes.byref(nn)), "num_recv")
        L.ep_handle_free(hl)

    def host_us(fn):
        for _ in range(max(args.warmup, 2)):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        return (time.perf_counter() - t0) * 1e6 / args.steps
    def idle_us(fn):
        for _ in range(max(args.warmup, 2)):
            fn()
        tot = 0.0
        for _ in range(args.steps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            tot += time.perf_counter() - t0
        torch.cuda.synchronize()
        return tot * 1e6 / args.steps
    us = host_us(fresh_size_query)
    us_idle = idle_us(fresh_size_query)
    rep["layout_with_n_readback"] = {"avg_us": round(us, 2), "mtok_s": round(T / us, 2),
                                     "idle_stream_us": round(us_idle, 2),
                                     "how": "ep_dispatch size query (the count kernel stores N "
                                            "into pinned host memory, the host polls it); "
                                            "avg_us: calls back to back, idle_stream_us: each "
                                            "call made on an idle stream"}
    us = host_us(layout_then_n)
    rep["layout_then_handle_num_recv"] = {"avg_us": round(us, 2),
                                          "how": "ep_get_dispatch_layout, then ep_handle_num_recv "
                                                 "(N copied into pinned memory, which the host "
                                                 "polls)"}
    # combine with two bias rows
    h = ctypes.c_void_p()
    abi.check(L.ep_dispatch(ctypes.byref(d), P(x), P(topk), P(w), None, ctypes.byref(h),
                            P(recv_x), None, P(rtw), cap, None, s), "dispatch")
    n = ctypes.c_int64()
    abi.check(L.ep_handle_num_recv(h, ctypes.byref(n)), "num_recv")
    N = int(n.value)
    b0 = torch.from_numpy(random_rows(T, H, 0, tag=21).view(np.int16)).to(dev)
    b1 = torch.from_numpy(random_rows(T, H, 0, tag=22).view(np.int16)).to(dev)
    us = timed(lambda: abi.check(L.ep_combine(h, H, P(recv_x), cap, P(rtw), P(b0), P(b1), None,
                                              P(out), P(cw), s), "combine"), args.steps)
    byt = (N + T) * H * 2 + N * 4 + N * K * 4 + T * K * 4 + 2 * T * H * 2
    rep["combine_with_bias"] = {"avg_us": round(us, 2), "bytes": byt,
                                "gbs": round(byt / (us * 1e-6) / 1e9, 1)}
    L.ep_handle_free(h)

    # low-latency with three ranks masked
    mask = torch.zeros(dc.R, dtype=torch.int32, device=dev)
    for r in (3, 17, 31):
        abi.check(L.ep_mask_update(P(mask), dc.R, r, 1, s), "mask")
    us_d = timed(lambda: abi.check(L.ep_ll_dispatch(ctypes.byref(dd), S, P(lx), P(ltopk), P(mask),
                                                    P(packed), P(lcount), P(lsrc), P(lslot), s),
                                   "ll"), args.steps)
    us_c = timed(lambda: abi.check(L.ep_ll_combine(ctypes.byref(dd), S, P(packed), P(ltopk), P(lw),
                                                   P(lslot), P(mask), P(lout), s), "ll"),
                 args.steps)
    rep["ll_dispatch_masked3"] = {"avg_us": round(us_d, 2)}
    rep["ll_combine_masked3"] = {"avg_us": round(us_c, 2)}

    # FP8 low-latency dispatch
    q = torch.empty((epr, dc.R, S, dc.H), dtype=torch.uint8, device=dev)
    sc = torch.empty((epr, dc.R, S, dc.H // 128), dtype=torch.float32, device=dev)
    us = timed(lambda: abi.check(L.ep_ll_dispatch_fp8(ctypes.byref(dd), S, P(lx), P(ltopk), None,
                                                      P(q), P(sc), P(lcount), P(lsrc), P(lslot),
                                                      s), "fp8"), args.steps)
    M = int((dc.topk_idx >= 0).sum())
    byt = dc.T * dc.H * 2 + M * dc.H + M * (dc.H // 128) * 4 + dc.T * dc.K * 12 + M * 4
    rep["ll_dispatch_fp8"] = {"avg_us": round(us, 2), "bytes": byt,
                              "gbs": round(byt / (us * 1e-6) / 1e9, 1)}
    # FP8 LL combine of that payload (codes and scales decoded in the sum)
    us = timed(lambda: abi.check(L.ep_ll_combine_fp8(ctypes.byref(dd), S, P(q), P(sc), P(ltopk),
                                                     P(lw), P(lslot), None, P(lout), s), "fp8c"),
               args.steps)
    byt = M * dc.H + M * (dc.H // 128) * 4 + dc.T * dc.H * 2 + dc.T * dc.K * 16
    rep["ll_combine_fp8"] = {"avg_us": round(us, 2), "bytes": byt,
                             "gbs": round(byt / (us * 1e-6) / 1e9, 1)}

    # load balancing: 32 replicas of the large workload's most popular experts
    big = config_inputs(4, with_x=False)
    table = big.extra["redundancy"]
    n_rep = int((table >= 0).sum())
    e_log = big.E - n_rep
    mapping = np.full(n_rep, -1, np.int64)
    for e, r in enumerate(table):
        if r >= 0:
            mapping[r - e_log] = e
    elems = 4 << 20  # 4 Mi bf16 per expert (8 MiB)
    ew = torch.empty((e_log, elems), dtype=torch.bfloat16, device=dev).normal_()
    rw = torch.empty((n_rep, elems), dtype=torch.bfloat16, device=dev)
    mp = torch.from_numpy(mapping).to(dev)
    us = timed(lambda: abi.check(L.ep_lb_prefetch_weights(P(ew), P(rw), P(mp), n_rep, e_log,
                                                          elems, s), "lb"), max(args.steps // 5, 3))
    byt = 2 * n_rep * elems * 2
    rep["lb_prefetch_weights"] = {"avg_us": round(us, 2), "bytes": byt,
                                  "gbs": round(byt / (us * 1e-6) / 1e9, 1),
                                  "replicas": n_rep, "elems_per_expert": elems}
    us = timed(lambda: abi.check(L.ep_lb_reduce_grads(P(rw), P(ew), P(mp), n_rep, e_log, elems, s),
                                 "lb"), max(args.steps // 5, 3))
    n_targets = len(set(mapping.tolist()))
    byt = (n_rep + 2 * n_targets) * elems * 2
    rep["lb_reduce_grads"] = {"avg_us": round(us, 2), "bytes": byt,
                              "gbs": round(byt / (us * 1e-6) / 1e9, 1)}
    del ew, rw

    # the decode step (LL dispatch + LL combine) replayed from a HIP graph,
    # against the same two calls launched one by one
    def ll_step():
        st = abi.current_stream()
        abi.check(L.ep_ll_dispatch(ctypes.byref(dd), S, P(lx), P(ltopk), None, P(packed),
                                   P(lcount), P(lsrc), P(lslot), st), "ll")
        abi.check(L.ep_ll_combine(ctypes.byref(dd), S, P(packed), P(ltopk), P(lw), P(lslot), None,
                                  P(lout), st), "ll")
    eager = timed(ll_step, args.steps)
    ll_step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ll_step()
    torch.cuda.synchronize()
    graph = timed(g.replay, args.steps)
    rep["ll_step_graph"] = {"eager_us": round(eager, 2), "graph_replay_us": round(graph, 2)}
    return rep


def measure_workloads(args, L, abi):
    """The skewed (Zipf 1.2, 10 % masked, R=32) and large (R=144, 32 redundant
    experts) workloads: layout, fresh dispatch (layout + pack with top-k),
    cached dispatch and combine, each timed over back-to-back calls with HIP
    events at the ends (not in ``value``)."""
    import numpy as np
    import torch
    from gen import config_inputs

    P = abi.ptr
    dev = torch.device("cuda", 0)
    s = abi.current_stream()
    n = max(args.steps // 2, 3)

    def timed(fn):
        for _ in range(max(args.warmup, 2)):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(n):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / n

    rep = {}
    for cfg in (2, 4):
        inp = config_inputs(cfg)
        T, H, E, K, R, C = inp.T, inp.H, inp.E, inp.K, inp.R, inp.C
        d = abi.dims(T, H, K, E, R, C)
        cap = int(L.ep_max_recv_rows(ctypes.byref(d)))
        x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).to(dev)
        topk = torch.from_numpy(inp.topk_idx).to(dev)
        w = torch.from_numpy(inp.topk_weights).to(dev)
        recv = torch.empty((cap, H), dtype=torch.int16, device=dev)
        rti = torch.empty((cap, K), dtype=torch.int64, device=dev)
        rtw = torch.empty((cap, K), dtype=torch.float32, device=dev)
        out = torch.empty((T, H), dtype=torch.int16, device=dev)
        cw = torch.empty((T, K), dtype=torch.float32, device=dev)

        def layout():
            h = ctypes.c_void_p()
            abi.check(L.ep_get_dispatch_layout(ctypes.byref(d), P(topk), None, None,
                                               ctypes.byref(h), s), "layout")
            L.ep_handle_free(h)

        def fresh():
            h = ctypes.c_void_p()
            abi.check(L.ep_dispatch(ctypes.byref(d), P(x), P(topk), P(w), None, ctypes.byref(h),
                                    P(recv), P(rti), P(rtw), cap, None, s), "dispatch")
            L.ep_handle_free(h)

        h = ctypes.c_void_p()
        abi.check(L.ep_dispatch(ctypes.byref(d), P(x), P(topk), P(w), None, ctypes.byref(h),
                                P(recv), P(rti), P(rtw), cap, None, s), "dispatch")
        nn = ctypes.c_int64()
        abi.check(L.ep_handle_num_recv(h, ctypes.byref(nn)), "num_recv")
        N = int(nn.value)
        us_lay = timed(layout)
        us_fresh = timed(fresh)
        us_cached = timed(lambda: abi.check(L.ep_dispatch(
            ctypes.byref(d), P(x), None, None, None, ctypes.byref(h), P(recv), None, None, cap,
            None, s), "cached dispatch"))
        us_comb = timed(lambda: abi.check(L.ep_combine(h, H, P(recv), cap, P(rtw), None, None,
                                                       None, P(out), P(cw), s), "combine"))
        L.ep_handle_free(h)
        b_cached = (T + N) * H * 2 + N * 4
        b_comb = (N + T) * H * 2 + N * 4 + N * K * 4 + T * K * 4
        rep[inp.name] = {
            "T": T, "H": H, "E": E, "K": K, "R": R, "C": C, "N": N,
            "layout_us": round(us_lay, 2), "layout_mtok_s": round(T / us_lay, 2),
            "dispatch_fresh_us": round(us_fresh, 2),
            "dispatch_cached_us": round(us_cached, 2),
            "dispatch_cached_gbs": round(b_cached / (us_cached * 1e-6) / 1e9, 1),
            "combine_us": round(us_comb, 2),
            "combine_gbs": round(b_comb / (us_comb * 1e-6) / 1e9, 1),
        }
        del x, recv, rti, rtw, out, cw

    # low-latency batch past the one-launch limit (T*K = 8192): slot scan +
    # token-major copy, then the LL combine
    from gen import generate
    inp = generate(1024, 7168, 256, 8, 32, 1, seed=0, slots=1024, name="ll_large")
    T, H, E, K, R, S = inp.T, inp.H, inp.E, inp.K, inp.R, inp.slots
    epr = E // R
    d = abi.dims(T, H, K, E, R, 1)
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).to(dev)
    topk = torch.from_numpy(inp.topk_idx).to(dev)
    w = torch.from_numpy(inp.topk_weights).to(dev)
    packed = torch.empty((epr, R, S, H), dtype=torch.int16, device=dev)
    cnt = torch.empty((epr, R), dtype=torch.int32, device=dev)
    src = torch.empty((epr, R, S), dtype=torch.int32, device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    M = int((inp.topk_idx >= 0).sum())
    us_d = timed(lambda: abi.check(L.ep_ll_dispatch(ctypes.byref(d), S, P(x), P(topk), None,
                                                    P(packed), P(cnt), P(src), P(slot), s), "ll"))
    us_c = timed(lambda: abi.check(L.ep_ll_combine(ctypes.byref(d), S, P(packed), P(topk), P(w),
                                                   P(slot), None, P(out), s), "ll"))
    b_d = T * H * 2 + M * H * 2 + T * K * 12 + M * 4
    b_c = M * H * 2 + T * H * 2 + T * K * 16
    rep["ll_large"] = {"T": T, "H": H, "E": E, "K": K, "R": R, "slots": S, "M": M,
                       "ll_dispatch_us": round(us_d, 2), "ll_dispatch_bytes": b_d,
                       "ll_dispatch_gbs": round(b_d / (us_d * 1e-6) / 1e9, 1),
                       "ll_combine_us": round(us_c, 2), "ll_combine_bytes": b_c,
                       "ll_combine_gbs": round(b_c / (us_c * 1e-6) / 1e9, 1)}
    del packed
    return rep


def cpu_baseline(tr, dc, x2_bits, budget: float, step_bytes: int, op_bytes=None,
                 workloads=(0, 2, 4)):
    """The oracle, as it stands, on the same rows of the same workload:
    whole passes (layout, dispatch, cached dispatch, combine, LL dispatch,
    LL combine) until ``budget`` seconds of CPU work are spent, with the
    process pinned to one core.  Also the median time of each operation over
    the passes (and its rate on the same algorithmic bytes), and the median
    of three runs of layout, dispatch and combine on each of ``workloads``
    (workload ids of the input generator)."""
    import oracle
    from gen import config_inputs
    pinned = None
    old_aff = None
    if hasattr(os, "sched_setaffinity"):
        try:
            old_aff = os.sched_getaffinity(0)
            pinned = min(old_aff)
            os.sched_setaffinity(0, {pinned})
        except OSError:
            pinned = None
    names = ["layout", "dispatch", "dispatch_cached", "combine", "ll_dispatch", "ll_combine"]
    times = {n: [] for n in names}
    passes = 0
    t0 = time.perf_counter()
    try:
        while True:
            c0 = time.perf_counter()
            lay = oracle.layout(tr.topk_idx, tr.E, tr.R, tr.C)
            c1 = time.perf_counter()
            rx, rti, rtw = oracle.dispatch(tr.x, tr.topk_idx, tr.topk_weights, tr.E, tr.R, lay)
            c2 = time.perf_counter()
            oracle.dispatch(x2_bits, None, None, tr.E, tr.R, lay, with_topk=False)
            c3 = time.perf_counter()
            oracle.combine(rx, lay, rtw)
            c4 = time.perf_counter()
            buf, _, _, _ = oracle.ll_dispatch(dc.x, dc.topk_idx, dc.E, dc.R, dc.slots)
            c5 = time.perf_counter()
            oracle.ll_combine(buf, dc.topk_idx, dc.topk_weights, dc.E, dc.R)
            c6 = time.perf_counter()
            for n, (u, v) in zip(names, [(c0, c1), (c1, c2), (c2, c3), (c3, c4), (c4, c5),
                                         (c5, c6)]):
                times[n].append(v - u)
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        per_workload = {}
        for cfg in workloads:
            inp = config_inputs(cfg)
            tl, td, tc = [], [], []
            for _ in range(3):
                c0 = time.perf_counter()
                lay = oracle.layout(inp.topk_idx, inp.E, inp.R, inp.C)
                c1 = time.perf_counter()
                rx, _, rtw = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, inp.E, inp.R,
                                             lay)
                c2 = time.perf_counter()
                oracle.combine(rx, lay, rtw)
                c3 = time.perf_counter()
                tl.append(c1 - c0)
                td.append(c2 - c1)
                tc.append(c3 - c2)
            per_workload[inp.name] = {"layout_ms": round(1e3 * sorted(tl)[1], 3),
                                      "dispatch_ms": round(1e3 * sorted(td)[1], 3),
                                      "combine_ms": round(1e3 * sorted(tc)[1], 3)}
    finally:
        if old_aff is not None and pinned is not None:
            os.sched_setaffinity(0, old_aff)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    per_op = {}
    for n in names:
        med = sorted(times[n])[len(times[n]) // 2]
        per_op[n] = {"median_ms": round(med * 1e3, 3)}
        if op_bytes is not None:
            per_op[n]["gbs"] = round(op_bytes[n] / med / 1e9, 3)
    return {"value": round(step_bytes * passes / el / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{passes} whole passes of the benchmark step (same workload, same rows) "
                      f"in {el:.1f} s, single-threaded C oracle"
                      + (f" pinned to CPU {pinned}" if pinned is not None else ""),
            "per_op": per_op, "per_workload": per_workload,
            "host_cpu": model or platform.processor(), "host_nproc": os.cpu_count()}


if __name__ == "__main__":
    main()
