"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import combine_ep_route_amd as ep
import ep_inputs as I
from combine_ep_route_amd import _abi as A


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU: run the CPU suite with -m 'not gpu'")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def group_for(w: I.Workload, **over) -> ep.Group:
    cfg = dict(mode=w.mode, num_nodes=w.num_nodes, ranks_per_node=w.ranks_per_node,
               num_experts=w.num_experts, top_k=w.top_k, max_nodes_per_token=w.max_nodes,
               hidden=w.hidden, max_tokens_per_rank=w.slots, num_src_ranks=w.num_src_ranks,
               payload=w.payload)
    cfg.update(over)
    return ep.ep_create_group(**cfg)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def get_map(h: ep.Handle, which: int) -> np.ndarray:
    return host(ep.ep_handle_get_map(h, which))


def buffer(g: ep.Group, which: int) -> torch.Tensor:
    return ep.ep_get_buffer(g, which)


def route_gpu(g: ep.Group, scores: np.ndarray, k: int) -> np.ndarray:
    s = dev(scores.astype(np.float32))
    out = torch.full((scores.shape[0], k), -7, dtype=torch.int32, device="cuda")
    ep.ep_route(g, s, out)
    return host(out)


__all__ = ["need_gpu", "say", "group_for", "dev", "host", "bits_of", "get_map", "buffer",
           "route_gpu", "A", "I", "ep"]
