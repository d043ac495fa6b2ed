"""MoE expert-parallel dispatch/combine on one MI355X: HIP kernels behind a C ABI.

The library (libep.so, built from csrc/ by ``combine_ep_route_amd.build``)
implements node-limited top-k routing, the handle's counts / prefix sums /
slot and row maps, FP8 E4M3 quantisation with one fp32 scale per 128
elements, the fixed-slot LL pack and the node-deduplicated HT two-stage pack,
and the weighted top-k combine.  This package is its thin Python binding.
"""
from . import _abi  # noqa: F401
from .ep import (  # noqa: F401
    EpError, Group, Handle, desc, ep_combine, ep_combine_backward, ep_complete, ep_create_group,
    ep_create_handle, ep_dispatch_backward, ep_layout_noalloc,
    ep_dequantize_rows, ep_destroy_group, ep_destroy_handle, ep_dispatch,
    ep_get_buffer, ep_get_device_error, ep_get_partition, ep_group_stats, ep_handle_get_buffer, ep_handle_get_map,
    ep_handle_get_num_recv, ep_last_hip_error, ep_quantize, ep_route, ep_route_handle, ep_status_string,
    make_config,
)
