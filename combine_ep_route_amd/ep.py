"""Thin Python binding of libep with the C ABI's names.

Argument marshalling only: torch tensors become ep_tensor_t descriptors
(data pointer, dtype, sizes, strides in elements, tag) and the current torch
HIP stream becomes the ep_stream_t.  Every step of the path runs in the HIP
library; this module computes nothing.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _abi as A


class EpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = A.lib().ep_status_string(status).decode()
        hip = A.lib().ep_last_hip_error()
        super().__init__(f"{fn} failed: {name}" + (f" (hipError {hip})" if status == A.EP_ERR_HIP else ""))
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != A.EP_OK:
        raise EpError(fn, status)


_DTYPES = {
    torch.float32: A.EP_DTYPE_F32,
    torch.bfloat16: A.EP_DTYPE_BF16,
    torch.float16: A.EP_DTYPE_F16,
    torch.float8_e4m3fn: A.EP_DTYPE_FP8_E4M3,
    torch.int32: A.EP_DTYPE_I32,
    torch.uint8: A.EP_DTYPE_U8,
}
_TORCH = {v: k for k, v in _DTYPES.items()}


def desc(t: Optional[torch.Tensor], tag: int = A.EP_TAG_NONE):
    """ep_tensor_t describing a torch tensor (None -> NULL).  Every tensor
    the library reads or writes lives in device memory: a host tensor is
    refused here, before its address could reach a kernel."""
    if t is None:
        return None
    if not t.is_cuda and not (tag == A.EP_TAG_RECV_EXPERT_COUNTER_HOST and t.is_pinned()):
        raise ValueError(f"ep tensors must be on the GPU (or, for a host receive counter, pinned), "
                         f"got a {t.device} tensor")
    if t.dim() < 1 or t.dim() > 3:
        raise ValueError("ep tensors have 1 to 3 dimensions")
    d = A.EpTensor()
    d.data = t.data_ptr()
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    # an empty tensor may report any strides (numpy's give 0s): describe it
    # as the contiguous tensor it trivially is
    strides = t.stride() if t.numel() > 0 else torch.empty(t.shape, device="meta").stride()
    for i in range(t.dim()):
        d.sizes[i] = t.shape[i]
        d.strides[i] = strides[i]
    d.tag = tag
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class Group:
    """An ep_group_t plus the configuration it was made with."""

    def __init__(self, ptr: int, config: dict):
        self.ptr = ptr
        self.config = dict(config)

    @property
    def memory_bytes(self) -> int:
        b = ctypes.c_int64()
        _check("ep_group_memory", A.lib().ep_group_memory(self.ptr, ctypes.byref(b)))
        return b.value


def ep_group_stats(group: Group) -> dict:
    st = A.EpStats()
    _check("ep_group_stats", A.lib().ep_group_stats(group.ptr, ctypes.byref(st)))
    return {name: getattr(st, name) for name in A.STAT_FIELDS}


class Handle:
    def __init__(self, ptr: int, group: Group, num_tokens: int):
        self.ptr = ptr
        self.group = group
        self.num_tokens = num_tokens
        self._staged = None   # tensors a staged (send_only) call still reads


def make_config(mode="ht", num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8,
                max_nodes_per_token=4, hidden=7168, max_tokens_per_rank=128,
                num_src_ranks=1, payload="fp8", max_handles=0, num_cus=0, ll_buffers=0, ht_stage2="expert",
                ht_buffers=0, alloc_fn=None, free_fn=None, alloc_ctx=None) -> A.EpConfig:
    c = A.EpConfig()
    c.mode = {"ll": A.EP_MODE_LL, "ht": A.EP_MODE_HT}[mode] if isinstance(mode, str) else mode
    c.num_nodes = num_nodes
    c.ranks_per_node = ranks_per_node
    c.num_experts = num_experts
    c.top_k = top_k
    c.max_nodes_per_token = max_nodes_per_token
    c.hidden = hidden
    c.max_tokens_per_rank = max_tokens_per_rank
    c.num_src_ranks = num_src_ranks
    c.payload = {"fp8": A.EP_DTYPE_FP8_E4M3, "bf16": A.EP_DTYPE_BF16}[payload] \
        if isinstance(payload, str) else payload
    c.max_handles = max_handles
    c.num_cus = num_cus
    c.ll_buffers = ll_buffers
    c.ht_stage2 = {"expert": A.EP_HT_STAGE2_PER_EXPERT, "rank": A.EP_HT_STAGE2_PER_RANK}[ht_stage2] \
        if isinstance(ht_stage2, str) else ht_stage2
    c.ht_buffers = ht_buffers
    c.alloc_fn = alloc_fn if alloc_fn is not None else A.ALLOC_FN()
    c.free_fn = free_fn if free_fn is not None else A.FREE_FN()
    c.alloc_ctx = alloc_ctx
    return c


def ep_create_group(stream=None, **config) -> Group:
    cfg = make_config(**config)
    out = ctypes.c_void_p()
    st = A.lib().ep_create_group(ctypes.byref(cfg), _stream(stream) if torch.cuda.is_available() else None,
                                 ctypes.byref(out))
    _check("ep_create_group", st)
    g = Group(out.value, config)
    g._cfg = cfg  # keep callbacks alive
    return g


def ep_destroy_group(group: Group) -> None:
    _check("ep_destroy_group", A.lib().ep_destroy_group(group.ptr))
    group.ptr = None


def ep_route(group: Group, scores: torch.Tensor, topk_idx: torch.Tensor, stream=None) -> None:
    s = desc(scores, A.EP_TAG_TOKENS)
    t = desc(topk_idx, A.EP_TAG_TOPK_IDX)
    _check("ep_route", A.lib().ep_route(group.ptr, _ref(s), _ref(t), _stream(stream)))


def ep_create_handle(group: Group, topk_idx: torch.Tensor, stream=None) -> Handle:
    out = ctypes.c_void_p()
    t = desc(topk_idx, A.EP_TAG_TOPK_IDX)
    _check("ep_create_handle", A.lib().ep_create_handle(group.ptr, _ref(t), _stream(stream), ctypes.byref(out)))
    return Handle(out.value, group, topk_idx.shape[0])


def ep_route_handle(group: Group, scores: torch.Tensor, topk_idx: torch.Tensor, stream=None) -> Handle:
    out = ctypes.c_void_p()
    sc = desc(scores, A.EP_TAG_TOKENS)
    t = desc(topk_idx, A.EP_TAG_TOPK_IDX)
    _check("ep_route_handle", A.lib().ep_route_handle(group.ptr, _ref(sc), _ref(t), _stream(stream),
                                                      ctypes.byref(out)))
    return Handle(out.value, group, topk_idx.shape[0])


def ep_layout_noalloc(topk_idx: torch.Tensor, maps: dict, device_error: Optional[torch.Tensor] = None,
                      stream=None, **config) -> None:
    """The handle's maps for topk_idx without a group or an allocation:
    maps is {ep_map_t id: int32 device tensor} for the configuration's mode;
    config takes ep_create_group's keyword arguments."""
    cfg = make_config(**config)
    t = desc(topk_idx, A.EP_TAG_TOPK_IDX)
    descs = [desc(maps[m]) if m in maps else None for m in range(8)]
    arr = (ctypes.POINTER(A.EpTensor) * 8)(*[ctypes.pointer(d) if d is not None else None for d in descs])
    err = desc(device_error)
    _check("ep_layout_noalloc", A.lib().ep_layout_noalloc(ctypes.byref(cfg), _ref(t), arr, _ref(err),
                                                          _stream(stream)))


def ep_destroy_handle(handle: Handle) -> None:
    _check("ep_destroy_handle", A.lib().ep_destroy_handle(handle.ptr))


def ep_dispatch(handle: Handle, tokens: torch.Tensor, scales: Optional[torch.Tensor] = None,
                topk_weights: Optional[torch.Tensor] = None,
                recv_counts: Optional[torch.Tensor] = None, send_only: bool = False, stream=None) -> None:
    x = desc(tokens, A.EP_TAG_TOKENS)
    sc = desc(scales, A.EP_TAG_SCALES)
    w = desc(topk_weights, A.EP_TAG_TOPK_WEIGHTS)
    # a pinned host tensor is NCCL-EP's host-side receive counter
    rc = desc(recv_counts, A.EP_TAG_TOKENS_PER_EXPERT if recv_counts is None or recv_counts.is_cuda
              else A.EP_TAG_RECV_EXPERT_COUNTER_HOST)
    _check("ep_dispatch", A.lib().ep_dispatch(handle.ptr, _ref(x), _ref(sc), _ref(w), _ref(rc),
                                              int(bool(send_only)), _stream(stream)))
    if send_only:
        handle._staged = (tokens, scales, topk_weights, recv_counts)   # alive until ep_complete


def ep_quantize(group: Group, tokens: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    x = desc(tokens, A.EP_TAG_TOKENS)
    qd = desc(q, A.EP_TAG_TOKENS)
    sd = desc(scales, A.EP_TAG_SCALES)
    _check("ep_quantize", A.lib().ep_quantize(group.ptr, _ref(x), _ref(qd), _ref(sd), _stream(stream)))


def ep_combine(handle: Handle, expert_out: torch.Tensor, topk_weights: Optional[torch.Tensor],
               out: torch.Tensor, send_only: bool = False, stream=None) -> None:
    y = desc(expert_out, A.EP_TAG_TOKENS)
    w = desc(topk_weights, A.EP_TAG_TOPK_WEIGHTS)
    o = desc(out, A.EP_TAG_TOKENS)
    _check("ep_combine", A.lib().ep_combine(handle.ptr, _ref(y), _ref(w), _ref(o), int(bool(send_only)),
                                            _stream(stream)))
    if send_only:
        handle._staged = (expert_out, topk_weights, out)   # alive until ep_complete


def ep_combine_backward(handle: Handle, grad_out: torch.Tensor, topk_weights: torch.Tensor,
                        grad_expert_out: torch.Tensor, expert_out: Optional[torch.Tensor] = None,
                        grad_weights: Optional[torch.Tensor] = None, stream=None) -> None:
    g = desc(grad_out, A.EP_TAG_TOKENS)
    y = desc(expert_out, A.EP_TAG_TOKENS)
    w = desc(topk_weights, A.EP_TAG_TOPK_WEIGHTS)
    dy = desc(grad_expert_out, A.EP_TAG_TOKENS)
    dw = desc(grad_weights, A.EP_TAG_TOPK_WEIGHTS)
    _check("ep_combine_backward", A.lib().ep_combine_backward(handle.ptr, _ref(g), _ref(y), _ref(w), _ref(dy),
                                                              _ref(dw), _stream(stream)))


def ep_dispatch_backward(handle: Handle, grad_expert_in: torch.Tensor, grad_tokens: torch.Tensor,
                         stream=None) -> None:
    r = desc(grad_expert_in, A.EP_TAG_TOKENS)
    o = desc(grad_tokens, A.EP_TAG_TOKENS)
    _check("ep_dispatch_backward", A.lib().ep_dispatch_backward(handle.ptr, _ref(r), _ref(o), _stream(stream)))


def ep_complete(handle: Handle, stream=None) -> None:
    _check("ep_complete", A.lib().ep_complete(handle.ptr, _stream(stream)))
    handle._staged = None


def ep_dequantize_rows(group: Group, rows: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    r = desc(rows)
    o = desc(y, A.EP_TAG_TOKENS)
    _check("ep_dequantize_rows", A.lib().ep_dequantize_rows(group.ptr, _ref(r), _ref(o), _stream(stream)))


def ep_handle_get_num_recv(handle: Handle, rank: int = -1) -> int:
    n = ctypes.c_int64()
    _check("ep_handle_get_num_recv", A.lib().ep_handle_get_num_recv(handle.ptr, rank, ctypes.byref(n)))
    return n.value


def ep_get_device_error(group: Group) -> int:
    c = ctypes.c_int32()
    _check("ep_get_device_error", A.lib().ep_get_device_error(group.ptr, ctypes.byref(c)))
    return c.value


def ep_status_string(status: int) -> str:
    return A.lib().ep_status_string(status).decode()


def ep_last_hip_error() -> int:
    return A.lib().ep_last_hip_error()


# ---------------------------------------------------------------------------
# Views of library-owned device memory as torch tensors (zero copy)
# ---------------------------------------------------------------------------

class _DeviceArray:
    """Exposes a raw device allocation through __cuda_array_interface__."""

    _TYPESTR = {A.EP_DTYPE_F32: "<f4", A.EP_DTYPE_I32: "<i4", A.EP_DTYPE_U8: "|u1",
                A.EP_DTYPE_BF16: "<u2", A.EP_DTYPE_F16: "<f2", A.EP_DTYPE_FP8_E4M3: "|u1"}

    def __init__(self, d: A.EpTensor):
        shape = tuple(d.sizes[i] for i in range(d.ndim))
        strides = tuple(d.strides[i] * _itemsize(d.dtype) for i in range(d.ndim))
        self.__cuda_array_interface__ = {
            "shape": shape, "typestr": self._TYPESTR[d.dtype], "strides": strides,
            "data": (d.data or 0, False), "version": 3}


def _itemsize(dt: int) -> int:
    return {A.EP_DTYPE_F32: 4, A.EP_DTYPE_I32: 4, A.EP_DTYPE_BF16: 2, A.EP_DTYPE_F16: 2}.get(dt, 1)


def _as_torch(d: A.EpTensor) -> torch.Tensor:
    t = torch.as_tensor(_DeviceArray(d), device="cuda")
    if d.dtype == A.EP_DTYPE_BF16:
        t = t.view(torch.bfloat16)
    return t


def ep_handle_get_map(handle: Handle, which: int) -> torch.Tensor:
    d = A.EpTensor()
    _check("ep_handle_get_map", A.lib().ep_handle_get_map(handle.ptr, which, ctypes.byref(d)))
    return _as_torch(d)


def ep_get_buffer(group: Group, which: int) -> torch.Tensor:
    d = A.EpTensor()
    _check("ep_get_buffer", A.lib().ep_get_buffer(group.ptr, which, ctypes.byref(d)))
    return _as_torch(d)


def ep_handle_get_buffer(handle: Handle, which: int) -> torch.Tensor:
    d = A.EpTensor()
    _check("ep_handle_get_buffer", A.lib().ep_handle_get_buffer(handle.ptr, which, ctypes.byref(d)))
    return _as_torch(d)


def ep_get_partition(handle: Handle, rank: int, which: int) -> torch.Tensor:
    d = A.EpTensor()
    _check("ep_get_partition", A.lib().ep_get_partition(handle.ptr, rank, which, ctypes.byref(d)))
    return _as_torch(d)
