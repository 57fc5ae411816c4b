"""Helpers shared by the GPU tests: moving seeded inputs to the device and
comparing the HIP results with the oracle's."""

from __future__ import annotations

import numpy as np
import torch


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of bf16 bit patterns
    (+0 and -0 are the same point)."""
    def ordered(u):
        u = u.astype(np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def assert_bf16_close(got_bits: np.ndarray, exp_bits: np.ndarray, max_ulp: int = 1,
                      exact: bool = True, what: str = "") -> None:
    d = bf16_ulp_diff(got_bits, exp_bits)
    worst = int(d.max()) if d.size else 0
    n_off = int(np.count_nonzero(d))
    assert worst <= max_ulp, f"{what}: max {worst} ulp apart ({n_off} elements differ)"
    if exact:
        assert n_off == 0, f"{what}: {n_off} elements differ by <= {max_ulp} ulp"


LAYOUT_FIELDS = ["num_tokens_per_rank", "num_tokens_per_expert", "rank_prefix_matrix",
                 "channel_prefix_matrix", "recv_channel_prefix_matrix", "send_head",
                 "recv_src_idx"]


def compare_layout(lay, ora) -> None:
    """Every layout output of a handle against the oracle's, bit-exact."""
    for name in LAYOUT_FIELDS:
        np.testing.assert_array_equal(host(getattr(lay, name)), getattr(ora, name), err_msg=name)
    np.testing.assert_array_equal(host(lay.is_token_in_rank).astype(np.uint8),
                                  ora.is_token_in_rank, err_msg="is_token_in_rank")


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
