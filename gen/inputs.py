"""Deterministic synthetic workloads shaped like the pages' MoE routing.

Every tensor comes from its own numpy ``PCG64`` stream seeded by
``SeedSequence([seed, stream_tag])`` so that changing one tensor's recipe never
shifts another's.  The recipes:

* ``x``: standard normal fp32, then the low 16 bits dropped (round toward zero)
  to get a bf16 bit pattern.  Truncation is used on purpose: it is not the
  rounding the method itself performs, so the generator shares no arithmetic
  with either implementation.  Rows are returned as ``uint16`` bit patterns.
* uniform routing: ``K`` distinct experts per token, uniformly, in draw order
  (the first ``K`` entries of a random permutation of the experts).
* Zipf routing: expert ``perm[i]`` gets weight ``(i+1)**-s`` over a seeded
  permutation ``perm``; ``K`` distinct experts are drawn without replacement by
  Gumbel-top-K (exact weighted sampling without replacement), in key order.
* redundant replicas: the ``n_rep`` most likely logical experts ``perm[j]`` get
  physical replica ids ``E_logical + j``; each slot routed to a replicated
  expert moves to its replica with probability 1/2.
* masking: each slot independently becomes -1 with probability ``mask``.
* weights: fp32 softmax of per-token standard-normal logits, computed before
  masking (masked slots keep their weight; the method ignores it).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_TAG_X = 1
_TAG_ROUTE = 2
_TAG_WEIGHTS = 3
_TAG_MASK = 4
_TAG_REPLICA = 5
_TAG_PERM = 6


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag)])))


@dataclass
class Inputs:
    """One workload.  Arrays are host numpy arrays, C-contiguous."""

    T: int
    H: int
    E: int
    K: int
    R: int
    C: int
    x: np.ndarray  # uint16 [T, H] bf16 bit patterns
    topk_idx: np.ndarray  # int64 [T, K], -1 = masked slot
    topk_weights: np.ndarray  # float32 [T, K]
    slots: int = 0  # low-latency slots per (local expert, rank); 0 = not an LL workload
    name: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def epr(self) -> int:
        return self.E // self.R


# The five workloads.  Sizes and routing mixes follow the training-scale,
# skewed, decode and large-scale MoE settings the pages describe.
CONFIGS = {
    0: dict(name="tiny", T=128, H=256, E=16, K=4, R=4, C=4, routing="uniform"),
    1: dict(name="training", T=4096, H=7168, E=256, K=8, R=64, C=10, routing="uniform"),
    2: dict(name="skewed", T=4096, H=7168, E=256, K=8, R=32, C=12, routing="zipf",
            zipf_s=1.2, mask=0.10),
    3: dict(name="ll_decode", T=128, H=7168, E=256, K=8, R=32, C=1, routing="uniform",
            slots=128),
    4: dict(name="large", T=8192, H=7168, E=288, K=8, R=144, C=20, routing="zipf",
            zipf_s=1.0, mask=0.05, replicas=32),
}


def _x_bits(T: int, H: int, seed: int) -> np.ndarray:
    f = _rng(seed, _TAG_X).standard_normal((T, H), dtype=np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _route_uniform(T: int, E: int, K: int, seed: int) -> np.ndarray:
    keys = _rng(seed, _TAG_ROUTE).random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int64)


def _zipf_perm(E: int, seed: int) -> np.ndarray:
    return _rng(seed, _TAG_PERM).permutation(E)


def _route_zipf(T: int, E: int, K: int, s: float, perm: np.ndarray, seed: int) -> np.ndarray:
    logp = np.empty(E, dtype=np.float64)
    logp[perm] = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    u = _rng(seed, _TAG_ROUTE).random((T, E))
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    key = logp[None, :] - np.log(-np.log(u))
    return np.argsort(-key, axis=1, kind="stable")[:, :K].astype(np.int64)


def _weights(T: int, K: int, seed: int) -> np.ndarray:
    logits = _rng(seed, _TAG_WEIGHTS).standard_normal((T, K), dtype=np.float32)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def generate(T: int, H: int, E: int, K: int, R: int, C: int, *, routing: str = "uniform",
             zipf_s: float = 1.0, mask: float = 0.0, replicas: int = 0, slots: int = 0,
             seed: int = 0, name: str = "", with_x: bool = True) -> Inputs:
    """Draw one workload.  ``E`` counts physical experts (replicas included)."""
    e_log = E - replicas
    if e_log < K:
        raise ValueError("need at least K logical experts")
    extra = {}
    if routing == "uniform":
        idx = _route_uniform(T, e_log, K, seed)
    elif routing == "zipf":
        perm = _zipf_perm(e_log, seed)
        idx = _route_zipf(T, e_log, K, zipf_s, perm, seed)
        extra["perm"] = perm
    else:
        raise ValueError(f"unknown routing {routing!r}")
    if replicas:
        if routing != "zipf":
            raise ValueError("replicas follow the Zipf popularity order")
        table = np.full(e_log, -1, dtype=np.int64)
        table[extra["perm"][:replicas]] = e_log + np.arange(replicas)
        move = _rng(seed, _TAG_REPLICA).random(idx.shape) < 0.5
        rep = table[idx]
        idx = np.where(move & (rep >= 0), rep, idx)
        extra["redundancy"] = table
    if mask > 0.0:
        m = _rng(seed, _TAG_MASK).random(idx.shape) < mask
        idx = np.where(m, np.int64(-1), idx)
    w = _weights(T, K, seed)
    x = _x_bits(T, H, seed) if with_x else np.zeros((T, 0), dtype=np.uint16)
    return Inputs(T=T, H=H, E=E, K=K, R=R, C=C, x=np.ascontiguousarray(x),
                  topk_idx=np.ascontiguousarray(idx), topk_weights=np.ascontiguousarray(w),
                  slots=slots, name=name, extra=extra)


def random_rows(n: int, h: int, seed: int, tag: int = 7) -> np.ndarray:
    """Standard-normal bf16 rows (uint16 bit patterns, truncated like ``x``),
    used as stand-in expert outputs for combine."""
    f = _rng(seed, 1000 + tag).standard_normal((n, h), dtype=np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def config_inputs(cfg_id: int, seed: int = 0, with_x: bool = True) -> Inputs:
    c = dict(CONFIGS[cfg_id])
    name = c.pop("name")
    return generate(seed=seed, name=name, with_x=with_x, **c)


def random_case(seed: int, T: int, H: int, E: int, K: int, R: int, C: int, *,
                mask: float = 0.0, dup: float = 0.0, slots: int = 0,
                zipf_s: Optional[float] = None) -> Inputs:
    """A small randomized case.  ``dup`` is the per-slot chance that a slot
    repeats the expert of slot 0 of the same token (repeated experts inside a
    token are allowed by the API, and must be handled)."""
    if zipf_s is None:
        inp = generate(T, H, E, K, R, C, seed=seed, mask=0.0, slots=slots)
    else:
        inp = generate(T, H, E, K, R, C, routing="zipf", zipf_s=zipf_s, seed=seed,
                       slots=slots)
    idx = inp.topk_idx.copy()
    r = _rng(seed, 100)
    if dup > 0.0 and K > 1:
        d = r.random((T, K)) < dup
        d[:, 0] = False
        idx = np.where(d, idx[:, :1], idx)
    if mask > 0.0:
        m = r.random((T, K)) < mask
        idx = np.where(m, np.int64(-1), idx)
    inp.topk_idx = np.ascontiguousarray(idx)
    return inp
