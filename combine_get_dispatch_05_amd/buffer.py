"""PyTorch-facing façade over libep.so with the call shapes of the pages' Buffer.

"DeepEP Buffer Class API for Expert Parallel Communication" describes a
``Buffer`` with ``get_dispatch_layout``, ``dispatch`` (6 results),
``combine`` (3 results), ``low_latency_dispatch`` (5 results),
``low_latency_combine`` (3 results), the low-latency mask-buffer utilities
and ``destroy``; "Chapter 10, V2: buffers beyond EP" (10.2) adds
``lb_prefetch_weights`` and ``lb_reduce_grads``.  This class keeps those
names and result arities so callers can switch; the slots that carried a CUDA
event or receive hook hold ``None`` (work is ordered on torch's current
stream instead).  The R ranks are logical partitions of this GPU's memory.

Only argument marshalling happens here: every step runs in the HIP kernels
behind the C ABI.  Tensors must live on the current CUDA (HIP) device.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import abi


def _need(t: torch.Tensor, dtype, name: str, ndim: int):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: torch.Tensor, shape, name: str):
    # The C ABI takes bare pointers, so every extent the kernels will index
    # is checked here, before a launch could read or write past a tensor.
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(map(str, devs))}")


@dataclass
class Layout:
    """Device copies of a dispatch layout ("What the Handle Contains")."""

    num_tokens_per_rank: torch.Tensor  # int32 [R]
    num_tokens_per_expert: torch.Tensor  # int32 [E]
    is_token_in_rank: torch.Tensor  # bool [T, R]
    rank_prefix_matrix: torch.Tensor  # int32 [R]
    channel_prefix_matrix: torch.Tensor  # int32 [R, C]
    recv_channel_prefix_matrix: torch.Tensor  # int32 [R, C]
    send_head: torch.Tensor  # int32 [T, R]
    recv_src_idx: torch.Tensor  # int32 [N]


class Handle:
    """Opaque dispatch layout owned by the library (freed on ``free()`` or
    garbage collection, ordered after the work already enqueued)."""

    def __init__(self, raw: int, d: abi.Dims, device: torch.device):
        self._raw = raw
        self.dims = d
        self.device = device

    @property
    def raw(self) -> ctypes.c_void_p:
        if not self._raw:
            raise ValueError("handle already freed")
        return ctypes.c_void_p(self._raw)

    @property
    def num_recv(self) -> int:
        """N, the number of packed rows (reads it back once)."""
        n = ctypes.c_int64(0)
        abi.check(abi.lib().ep_handle_num_recv(self.raw, ctypes.byref(n)), "ep_handle_num_recv")
        return int(n.value)

    @property
    def nbytes(self) -> int:
        return int(abi.lib().ep_handle_nbytes(self.raw))

    def layout(self) -> Layout:
        d = self.dims
        T, R, E, C = d.num_tokens, d.num_ranks, d.num_experts, d.num_channels
        n = self.num_recv
        i32 = dict(dtype=torch.int32, device=self.device)
        lay = Layout(torch.empty(R, **i32), torch.empty(E, **i32),
                     torch.empty((T, R), dtype=torch.uint8, device=self.device),
                     torch.empty(R, **i32), torch.empty((R, C), **i32), torch.empty((R, C), **i32),
                     torch.empty((T, R), **i32), torch.empty(max(n, 1), **i32))
        out = abi.LayoutOut(lay.num_tokens_per_rank.data_ptr(), lay.num_tokens_per_expert.data_ptr(),
                            lay.is_token_in_rank.data_ptr(), lay.rank_prefix_matrix.data_ptr(),
                            lay.channel_prefix_matrix.data_ptr(),
                            lay.recv_channel_prefix_matrix.data_ptr(), lay.send_head.data_ptr(),
                            lay.recv_src_idx.data_ptr(), n)
        abi.check(abi.lib().ep_handle_copy_layout(self.raw, ctypes.byref(out), abi.current_stream()),
                  "ep_handle_copy_layout")
        lay.is_token_in_rank = lay.is_token_in_rank.view(torch.bool)
        lay.recv_src_idx = lay.recv_src_idx[:n]
        return lay

    def free(self) -> None:
        if self._raw:
            abi.lib().ep_handle_free(ctypes.c_void_p(self._raw))
            self._raw = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


@dataclass
class LowLatencyHandle:
    """What low_latency_combine needs to find each (token, slot)'s cell."""

    src_info: torch.Tensor  # int32 [E/R, R, slots]
    topk_slot: torch.Tensor  # int32 [T, K]
    num_slots: int
    num_experts: int
    hidden: int


class Buffer:
    """Expert-parallel layout / dispatch / combine over R logical ranks of one GPU."""

    def __init__(self, num_ranks: int, num_experts: int, num_channels: int = 1):
        if num_experts % num_ranks:
            raise ValueError("num_experts must be a multiple of num_ranks")
        self.num_ranks = int(num_ranks)
        self.num_experts = int(num_experts)
        self.num_channels = int(num_channels)
        self.destroyed = False
        self._mask = None  # device int32 [R], created by the first mask update

    # ------------------------------------------------------- rank masking
    def _mask_ptr(self):
        return abi.ptr(self._mask) if self._mask is not None else None

    def low_latency_update_mask_buffer(self, rank_to_mask: int, mask: bool = False) -> None:
        """Mask (True) or unmask (False) one rank for the low-latency calls."""
        if self._mask is None:
            self._mask = torch.zeros(self.num_ranks, dtype=torch.int32, device="cuda")
        abi.check(abi.lib().ep_mask_update(abi.ptr(self._mask), self.num_ranks, int(rank_to_mask),
                                           1 if mask else 0, abi.current_stream()),
                  "ep_mask_update")

    def low_latency_query_mask_buffer(self, mask_status: torch.Tensor) -> None:
        """Write the mask (0 active, 1 masked) into a CPU int32 tensor [R]."""
        if (mask_status.dtype != torch.int32 or mask_status.numel() != self.num_ranks
                or mask_status.is_cuda or not mask_status.is_contiguous()):
            raise ValueError("mask_status must be a contiguous CPU int32 tensor with one entry "
                             "per rank")
        if self._mask is None:
            mask_status.zero_()
            return
        abi.check(abi.lib().ep_mask_query(abi.ptr(self._mask), self.num_ranks,
                                          ctypes.c_void_p(mask_status.data_ptr()),
                                          abi.current_stream()), "ep_mask_query")

    def low_latency_clean_mask_buffer(self) -> None:
        """Mark every rank active again."""
        if self._mask is not None:
            abi.check(abi.lib().ep_mask_clean(abi.ptr(self._mask), self.num_ranks,
                                              abi.current_stream()), "ep_mask_clean")

    @property
    def num_local_experts(self) -> int:
        return self.num_experts // self.num_ranks

    def _dims(self, T: int, H: int, K: int) -> abi.Dims:
        return abi.dims(T, H, K, self.num_experts, self.num_ranks, self.num_channels)

    # -------------------------------------------------------------- layout
    def get_dispatch_layout(self, topk_idx: torch.Tensor, keep_handle: bool = False):
        """Returns (num_tokens_per_rank [R], num_tokens_per_expert [E],
        is_token_in_rank [T, R] bool, handle or None).  A kept handle can be
        passed to one ``dispatch`` together with the same ``topk_idx``.
        Ranks masked in the mask buffer receive nothing (their slots act as
        masked slots)."""
        _need(topk_idx, torch.int64, "topk_idx", 2)
        T, K = topk_idx.shape
        d = self._dims(T, 8, K)
        dev = topk_idx.device
        ntpr = torch.empty(self.num_ranks, dtype=torch.int32, device=dev)
        ntpe = torch.empty(self.num_experts, dtype=torch.int32, device=dev)
        itr = torch.empty((T, self.num_ranks), dtype=torch.uint8, device=dev)
        out = abi.LayoutOut(ntpr.data_ptr(), ntpe.data_ptr(), itr.data_ptr(), None, None, None,
                            None, None, 0)
        raw = ctypes.c_void_p()
        rc = abi.lib().ep_get_dispatch_layout(ctypes.byref(d), abi.ptr(topk_idx),
                                              abi.ptr(self._mask), ctypes.byref(out),
                                              ctypes.byref(raw) if keep_handle else None,
                                              abi.current_stream())
        h = Handle(raw.value, d, dev) if keep_handle and raw.value else None
        abi.check(rc, "ep_get_dispatch_layout")
        return ntpr, ntpe, itr.view(torch.bool), h

    # ------------------------------------------------------------ dispatch
    def dispatch(self, x: torch.Tensor, topk_idx: Optional[torch.Tensor] = None,
                 topk_weights: Optional[torch.Tensor] = None, handle: Optional[Handle] = None):
        """Returns (recv_x [N, H], recv_topk_idx [N, K] or None,
        recv_topk_weights [N, K] or None, num_recv_tokens_per_expert [R, E/R],
        handle, None).  Without a handle the layout is computed and N is read
        back (one host sync); with a handle from an earlier dispatch only the
        rows are packed and topk arguments are refused.  A fresh dispatch
        leaves out the ranks masked in the mask buffer."""
        _need(x, torch.bfloat16, "x", 2)
        T, H = x.shape
        if handle is None and topk_idx is None:
            raise ValueError("dispatch without a handle needs topk_idx")
        if topk_idx is not None:
            _need(topk_idx, torch.int64, "topk_idx", 2)
            if topk_idx.shape[0] != T:
                raise ValueError("topk_idx and x disagree on the number of tokens")
        if topk_weights is not None:
            if topk_idx is None:
                raise ValueError("topk_weights needs topk_idx")
            _need(topk_weights, torch.float32, "topk_weights", 2)
            _shape(topk_weights, topk_idx.shape, "topk_weights")
        _same_device(x, topk_idx, topk_weights)
        K = topk_idx.shape[1] if topk_idx is not None else handle.dims.num_topk
        d = self._dims(T, H, K)
        dev = x.device
        if handle is not None and handle.device != dev:
            raise ValueError("handle was made on another device")
        raw = ctypes.c_void_p(handle.raw.value if handle is not None else None)
        if handle is not None and handle.dims.num_tokens != T:
            raise ValueError("handle was made for another number of tokens")
        cap = handle.num_recv if handle is not None else int(abi.lib().ep_max_recv_rows(ctypes.byref(d)))
        recv_x = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        rti = torch.empty((cap, K), dtype=torch.int64, device=dev) if topk_idx is not None else None
        rtw = torch.empty((cap, K), dtype=torch.float32, device=dev) if topk_weights is not None else None
        n = ctypes.c_int64(-1)
        mask = abi.ptr(self._mask) if handle is None else None
        rc = abi.lib().ep_dispatch(ctypes.byref(d), abi.ptr(x), abi.ptr(topk_idx),
                                   abi.ptr(topk_weights), mask, ctypes.byref(raw),
                                   abi.ptr(recv_x),
                                   abi.ptr(rti), abi.ptr(rtw), cap, ctypes.byref(n),
                                   abi.current_stream())
        if handle is None and raw.value:
            # owned from here on, so an error below still frees it
            handle = Handle(raw.value, d, dev)
        abi.check(rc, "ep_dispatch")
        N = int(n.value)
        lay_counts = None
        if topk_idx is not None:
            lay_counts = self._expert_counts(handle)
        return (recv_x[:N], rti[:N] if rti is not None else None,
                rtw[:N] if rtw is not None else None, lay_counts, handle, None)

    def _expert_counts(self, handle: Handle) -> torch.Tensor:
        ntpe = torch.empty(self.num_experts, dtype=torch.int32, device=handle.device)
        out = abi.LayoutOut(None, ntpe.data_ptr(), None, None, None, None, None, None, 0)
        abi.check(abi.lib().ep_handle_copy_layout(handle.raw, ctypes.byref(out),
                                                  abi.current_stream()),
                  "ep_handle_copy_layout")
        return ntpe.view(self.num_ranks, self.num_local_experts)

    # ------------------------------------------------------------- combine
    def combine(self, x: torch.Tensor, handle: Handle, topk_weights: Optional[torch.Tensor] = None,
                bias=None):
        """Returns (combined_x [T, H] bf16, combined_topk_weights [T, K] or
        None, None): the ascending-rank fp32 sum of each token's rows, plus
        the optional bias terms (a [T, H] bf16 tensor or a tuple of up to
        two), added before the single rounding.  Ranks masked in the mask
        buffer now are left out of the sums."""
        _need(x, torch.bfloat16, "x", 2)
        d = handle.dims
        if topk_weights is not None:
            _need(topk_weights, torch.float32, "topk_weights", 2)
            _shape(topk_weights, (x.shape[0], d.num_topk), "topk_weights")
        if handle.device != x.device:
            raise ValueError("handle was made on another device")
        T, H = d.num_tokens, x.shape[1]
        biases = [] if bias is None else ([bias] if isinstance(bias, torch.Tensor) else list(bias))
        if len(biases) > 2:
            raise ValueError("at most two bias tensors")
        for b in biases:
            _need(b, torch.bfloat16, "bias", 2)
            if tuple(b.shape) != (T, H):
                raise ValueError("bias must be [num_tokens, hidden]")
        _same_device(x, topk_weights, *biases)
        b0 = biases[0] if len(biases) > 0 else None
        b1 = biases[1] if len(biases) > 1 else None
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
        cw = None
        if topk_weights is not None:
            cw = torch.empty((T, d.num_topk), dtype=torch.float32, device=x.device)
        abi.check(abi.lib().ep_combine(handle.raw, H, abi.ptr(x), x.shape[0], abi.ptr(topk_weights),
                                       abi.ptr(b0), abi.ptr(b1), abi.ptr(self._mask),
                                       abi.ptr(out), abi.ptr(cw),
                                       abi.current_stream()),
                  "ep_combine")
        return out, cw, None

    # --------------------------------------------------------- low latency
    def low_latency_dispatch(self, x: torch.Tensor, topk_idx: torch.Tensor,
                             num_max_dispatch_tokens_per_rank: int,
                             num_experts: Optional[int] = None, use_fp8: bool = False):
        """Returns (packed_x, packed_count [E/R, R], handle, None, None).
        packed_x is [E/R, R, slots, H] bf16, or with use_fp8 the pair
        (codes [E/R, R, slots, H] float8_e4m3fn, scales [E/R, R, slots, H/128]
        fp32).  Unused packed cells are left as allocated.  Ranks masked with
        low_latency_update_mask_buffer receive nothing."""
        if num_experts is not None and num_experts != self.num_experts:
            raise ValueError("num_experts differs from the buffer's")
        _need(x, torch.bfloat16, "x", 2)
        _need(topk_idx, torch.int64, "topk_idx", 2)
        T, H = x.shape
        K = topk_idx.shape[1]
        if topk_idx.shape[0] != T:
            raise ValueError("topk_idx and x disagree on the number of tokens")
        _same_device(x, topk_idx)
        S = int(num_max_dispatch_tokens_per_rank)
        d = self._dims(T, H, K)
        dev = x.device
        epr, R = self.num_local_experts, self.num_ranks
        count = torch.empty((epr, R), dtype=torch.int32, device=dev)
        src = torch.empty((epr, R, S), dtype=torch.int32, device=dev)
        slot = torch.empty((T, K), dtype=torch.int32, device=dev)
        if use_fp8:
            q = torch.empty((epr, R, S, H), dtype=torch.uint8, device=dev)
            sc = torch.empty((epr, R, S, H // 128), dtype=torch.float32, device=dev)
            abi.check(abi.lib().ep_ll_dispatch_fp8(ctypes.byref(d), S, abi.ptr(x), abi.ptr(topk_idx),
                                                   self._mask_ptr(), abi.ptr(q), abi.ptr(sc),
                                                   abi.ptr(count), abi.ptr(src), abi.ptr(slot),
                                                   abi.current_stream()),
                      "ep_ll_dispatch_fp8")
            packed = (q.view(torch.float8_e4m3fn), sc)
        else:
            packed = torch.empty((epr, R, S, H), dtype=torch.bfloat16, device=dev)
            abi.check(abi.lib().ep_ll_dispatch(ctypes.byref(d), S, abi.ptr(x), abi.ptr(topk_idx),
                                               self._mask_ptr(), abi.ptr(packed), abi.ptr(count),
                                               abi.ptr(src), abi.ptr(slot), abi.current_stream()),
                      "ep_ll_dispatch")
        return packed, count, LowLatencyHandle(src, slot, S, self.num_experts, H), None, None

    def low_latency_combine(self, x, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                            handle: LowLatencyHandle):
        """x has packed_x's layout [E/R, R, slots, H] (bf16), or is the FP8 pair
        (codes [E/R, R, slots, H] float8_e4m3fn or uint8, scales [E/R, R,
        slots, H/128] fp32) that low_latency_dispatch(use_fp8=True) returns,
        decoded with its scales in the sum.  Returns (combined_x [T, H] bf16,
        None, None)."""
        _need(topk_idx, torch.int64, "topk_idx", 2)
        _need(topk_weights, torch.float32, "topk_weights", 2)
        T, K = topk_idx.shape
        _shape(topk_weights, (T, K), "topk_weights")
        _shape(handle.topk_slot, (T, K), "the handle's topk_slot")
        if handle.num_experts != self.num_experts:
            raise ValueError("handle was made for another number of experts")
        cells = (self.num_local_experts, self.num_ranks, handle.num_slots)
        if isinstance(x, (tuple, list)):
            q, sc = x
            if q.dtype == torch.float8_e4m3fn:
                q = q.view(torch.uint8)
            _need(q, torch.uint8, "codes", 4)
            _need(sc, torch.float32, "scales", 4)
            H = q.shape[3]
            _shape(q, cells + (H,), "codes")
            if tuple(sc.shape) != tuple(q.shape[:3]) + (H // 128,):
                raise ValueError("scales must be [E/R, R, slots, H/128]")
            _same_device(q, sc, topk_idx, topk_weights, handle.topk_slot)
            d = self._dims(T, H, K)
            out = torch.empty((T, H), dtype=torch.bfloat16, device=q.device)
            abi.check(abi.lib().ep_ll_combine_fp8(ctypes.byref(d), handle.num_slots, abi.ptr(q),
                                                  abi.ptr(sc), abi.ptr(topk_idx),
                                                  abi.ptr(topk_weights), abi.ptr(handle.topk_slot),
                                                  self._mask_ptr(), abi.ptr(out),
                                                  abi.current_stream()),
                      "ep_ll_combine_fp8")
            return out, None, None
        _need(x, torch.bfloat16, "x", 4)
        H = x.shape[3]
        _shape(x, cells + (H,), "x")
        _same_device(x, topk_idx, topk_weights, handle.topk_slot)
        d = self._dims(T, H, K)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
        abi.check(abi.lib().ep_ll_combine(ctypes.byref(d), handle.num_slots, abi.ptr(x),
                                          abi.ptr(topk_idx), abi.ptr(topk_weights),
                                          abi.ptr(handle.topk_slot), self._mask_ptr(),
                                          abi.ptr(out), abi.current_stream()),
                  "ep_ll_combine")
        return out, None, None

    # ------------------------------------------------------ load balancing
    @staticmethod
    def _lb_args(redundant: torch.Tensor, expert: torch.Tensor, mapping: torch.Tensor):
        """Rows per replica / expert; one replica row per mapping entry, and
        replica rows the size of expert rows."""
        for t, n in ((redundant, "redundant tensor"), (expert, "expert tensor")):
            _need(t, torch.bfloat16, n, t.dim())
            if t.dim() < 1:
                raise ValueError(f"{n} needs a leading [rows] dimension")
        _need(mapping, torch.int64, "redundancy_mapping", 1)
        _same_device(redundant, expert, mapping)
        if redundant.shape[0] != mapping.numel():
            raise ValueError("the redundant tensor needs one row per redundancy_mapping entry")
        if tuple(redundant.shape[1:]) != tuple(expert.shape[1:]):
            raise ValueError("replica rows and expert rows must have the same shape")
        return int(torch.Size(expert.shape[1:]).numel())

    def lb_prefetch_weights(self, redundant_expert_weights: torch.Tensor,
                            expert_weights: torch.Tensor, redundancy_mapping: torch.Tensor,
                            num_sms: int = 0, previous_event=None):
        """redundant_expert_weights[j] = expert_weights[redundancy_mapping[j]]
        (bf16, one row per expert / replica).  Returns None."""
        P = self._lb_args(redundant_expert_weights, expert_weights, redundancy_mapping)
        abi.check(abi.lib().ep_lb_prefetch_weights(
            abi.ptr(expert_weights), abi.ptr(redundant_expert_weights), abi.ptr(redundancy_mapping),
            redundancy_mapping.numel(), expert_weights.shape[0], P, abi.current_stream()),
            "ep_lb_prefetch_weights")
        return None

    def lb_reduce_grads(self, redundant_expert_grads: torch.Tensor, expert_grads: torch.Tensor,
                        redundancy_mapping: torch.Tensor, num_sms: int = 0, previous_event=None):
        """Folds each replica's gradient into its expert (in place, fp32
        accumulation, replicas in ascending order, one rounding).  Returns None."""
        P = self._lb_args(redundant_expert_grads, expert_grads, redundancy_mapping)
        abi.check(abi.lib().ep_lb_reduce_grads(
            abi.ptr(redundant_expert_grads), abi.ptr(expert_grads), abi.ptr(redundancy_mapping),
            redundancy_mapping.numel(), expert_grads.shape[0], P, abi.current_stream()),
            "ep_lb_reduce_grads")
        return None

    def destroy(self) -> None:
        """Return pooled device memory of the current device."""
        abi.check(abi.lib().ep_pool_trim(), "ep_pool_trim")
        self.destroyed = True
