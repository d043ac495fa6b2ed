"""ctypes declarations of the C ABI in include/ep.h and the loader of libep.so.

The library is loaded from this package's directory only; if it is missing
the import of the binding fails loudly -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libep.so")

# ep_status_t
EP_OK = 0
EP_ERR_INVALID_ARGUMENT = 1
EP_ERR_CAPACITY = 2
EP_ERR_OUT_OF_MEMORY = 3
EP_ERR_HIP = 4
EP_ERR_UNSUPPORTED = 5

EP_MODE_LL = 0
EP_MODE_HT = 1
EP_HT_STAGE2_PER_EXPERT = 0
EP_HT_STAGE2_PER_RANK = 1

EP_DTYPE_F32 = 0
EP_DTYPE_BF16 = 1
EP_DTYPE_F16 = 2
EP_DTYPE_FP8_E4M3 = 3
EP_DTYPE_I32 = 4
EP_DTYPE_U8 = 5

EP_TAG_NONE = 0
EP_TAG_TOKENS = 1
EP_TAG_TOPK_IDX = 2
EP_TAG_TOPK_WEIGHTS = 3
EP_TAG_SCALES = 4
EP_TAG_RECV_EXPERT_COUNTER_DEVICE = 5
EP_TAG_RECV_EXPERT_COUNTER_HOST = 6
EP_TAG_TOKENS_PER_EXPERT = 7

EP_DEVERR_BAD_INDEX = 1
EP_DEVERR_DUP_INDEX = 2
EP_DEVERR_ROW_RANGE = 4

EP_MAP_LL_SLOT = 0
EP_MAP_LL_COUNT = 1
EP_MAP_HT_NODE_ROW = 2
EP_MAP_HT_ROW = 3
EP_MAP_HT_RANK_COUNT = 4
EP_MAP_HT_RANK_OFFSET = 5
EP_MAP_HT_EXPERT_COUNT = 6
EP_MAP_HT_EXPERT_OFFSET = 7

EP_NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024

EP_BUF_LL_RECV = 0
EP_BUF_HT_STAGE1 = 1
EP_BUF_HT_STAGE1_TOKEN = 2
EP_BUF_HT_STAGE1_SRC = 3
EP_BUF_HT_STAGE1_TOPK = 4
EP_BUF_HT_STAGE1_WEIGHTS = 5
EP_BUF_HT_STAGE2 = 6
EP_BUF_HT_STAGE2_SRC = 7
EP_BUF_HT_STAGE2_TOKEN = 8
EP_BUF_HT_STAGE2_K = 9
EP_BUF_HT_STAGE2_TOPK = 10
EP_BUF_HT_STAGE2_WEIGHTS = 11


class EpTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("sizes", ctypes.c_int64 * 3),
        ("strides", ctypes.c_int64 * 3),
        ("tag", ctypes.c_int32),
    ]


STAT_FIELDS = ("route_calls", "handles_created", "dispatch_calls", "combine_calls", "complete_calls",
               "combine_backward_calls", "dispatch_backward_calls", "quantize_calls", "tokens_routed",
               "tokens_dispatched", "tokens_combined")


class EpStats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in STAT_FIELDS]


ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
FREE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p)


class EpConfig(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("num_nodes", ctypes.c_int32),
        ("ranks_per_node", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("max_nodes_per_token", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("max_tokens_per_rank", ctypes.c_int32),
        ("num_src_ranks", ctypes.c_int32),
        ("payload", ctypes.c_int32),
        ("max_handles", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("ll_buffers", ctypes.c_int32),
        ("ht_stage2", ctypes.c_int32),
        ("ht_buffers", ctypes.c_int32),
        ("alloc_fn", ALLOC_FN),
        ("free_fn", FREE_FN),
        ("alloc_ctx", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_PT = ctypes.POINTER(EpTensor)
_S = ctypes.c_int

# name -> (restype, argtypes), in the order of include/ep.h
SIGNATURES = {
    "ep_create_group": (_S, [ctypes.POINTER(EpConfig), _P, ctypes.POINTER(_P)]),
    "ep_destroy_group": (_S, [_P]),
    "ep_group_memory": (_S, [_P, ctypes.POINTER(ctypes.c_int64)]),
    "ep_group_stats": (_S, [_P, ctypes.POINTER(EpStats)]),
    "ep_route": (_S, [_P, _PT, _PT, _P]),
    "ep_create_handle": (_S, [_P, _PT, _P, ctypes.POINTER(_P)]),
    "ep_route_handle": (_S, [_P, _PT, _PT, _P, ctypes.POINTER(_P)]),
    "ep_destroy_handle": (_S, [_P]),
    "ep_layout_noalloc": (_S, [ctypes.POINTER(EpConfig), _PT, ctypes.POINTER(_PT), _PT, _P]),
    "ep_handle_get_num_recv": (_S, [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]),
    "ep_handle_get_map": (_S, [_P, ctypes.c_int32, _PT]),
    "ep_dispatch": (_S, [_P, _PT, _PT, _PT, _PT, ctypes.c_int32, _P]),
    "ep_get_buffer": (_S, [_P, ctypes.c_int32, _PT]),
    "ep_handle_get_buffer": (_S, [_P, ctypes.c_int32, _PT]),
    "ep_get_partition": (_S, [_P, ctypes.c_int32, ctypes.c_int32, _PT]),
    "ep_quantize": (_S, [_P, _PT, _PT, _PT, _P]),
    "ep_combine": (_S, [_P, _PT, _PT, _PT, ctypes.c_int32, _P]),
    "ep_complete": (_S, [_P, _P]),
    "ep_combine_backward": (_S, [_P, _PT, _PT, _PT, _PT, _PT, _P]),
    "ep_dispatch_backward": (_S, [_P, _PT, _PT, _P]),
    "ep_dequantize_rows": (_S, [_P, _PT, _PT, _P]),
    "ep_status_string": (ctypes.c_char_p, [_S]),
    "ep_get_device_error": (_S, [_P, ctypes.POINTER(ctypes.c_int32)]),
    "ep_last_hip_error": (ctypes.c_int, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libep.so (built by combine_ep_route_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m combine_ep_route_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib
