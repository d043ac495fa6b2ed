"""NCCL-EP's host-side receive counter ("NCCL EP paper notes", tensor tags:
the receive expert counter exists on the device and on the host): recv_counts
in pinned host memory is written by the receive stage directly, so the
counts are on the host once the stream gets there, with no copy.  Pageable
host memory is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_ht_counts_into_pinned_host_memory():
    S, T, E, K, H = 2, 90, 64, 4, 256
    say("HT recv_counts in pinned host memory")
    topk = I.random_topk(S * T, E, K, seed=71)
    g = ep.ep_create_group(mode="ht", num_nodes=4, ranks_per_node=2, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=T, num_src_ranks=S)
    try:
        h = ep.ep_create_handle(g, dev(topk))
        rc = torch.full((E,), -1, dtype=torch.int32).pin_memory()
        ep.ep_dispatch(h, I.normal_bf16(S * T, H, 72).cuda(), recv_counts=rc)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(rc.numpy(), oracle.layout_ht(topk, S, E, 4, 2)["c2"])
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("per_expert", [False, True])
def test_ll_staged_counts_into_pinned_host_memory(per_expert):
    S, T, E, K, H = 3, 40, 32, 4, 256
    say(f"LL staged recv_counts in pinned host memory ({'[E]' if per_expert else '[E, S]'})")
    topk = I.random_topk(S * T, E, K, seed=73)
    g = ep.ep_create_group(mode="ll", num_nodes=2, ranks_per_node=2, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=T, num_src_ranks=S)
    try:
        h = ep.ep_create_handle(g, dev(topk))
        shape = (E,) if per_expert else (E, S)
        rc = torch.full(shape, -1, dtype=torch.int32).pin_memory()
        ep.ep_dispatch(h, I.normal_bf16(S * T, H, 74).cuda(), recv_counts=rc, send_only=True)
        ep.ep_complete(h)
        torch.cuda.synchronize()
        want, _, _ = oracle.layout_ll(topk, S, E, T)
        np.testing.assert_array_equal(rc.numpy(), want.sum(axis=1) if per_expert else want)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_pageable_host_counter_is_refused_before_anything_runs():
    S, T, E, K, H = 1, 32, 16, 2, 256
    say("LL recv_counts in pageable host memory: refused")
    g = ep.ep_create_group(mode="ll", num_nodes=2, ranks_per_node=2, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=T, num_src_ranks=S)
    try:
        h = ep.ep_create_handle(g, dev(I.random_topk(S * T, E, K, seed=75)))
        host = np.zeros(E, np.int32)                       # pageable
        rc = A.EpTensor()
        rc.data = host.ctypes.data
        rc.dtype = A.EP_DTYPE_I32
        rc.ndim = 1
        rc.sizes[0] = E
        rc.strides[0] = 1
        rc.tag = A.EP_TAG_RECV_EXPERT_COUNTER_HOST
        x = ep.desc(I.normal_bf16(S * T, H, 76).cuda(), A.EP_TAG_TOKENS)
        st = A.lib().ep_dispatch(h.ptr, ctypes.byref(x), None, None, ctypes.byref(rc), 0,
                                 torch.cuda.current_stream().cuda_stream)
        assert st == A.EP_ERR_INVALID_ARGUMENT
        assert ep.ep_group_stats(g)["dispatch_calls"] == 0              # nothing was enqueued
        with pytest.raises(ep.EpError):
            ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)               # no receive buffer taken
        with pytest.raises(ValueError):
            ep.ep_dispatch(h, I.normal_bf16(S * T, H, 76).cuda(), recv_counts=torch.zeros(E, dtype=torch.int32))
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
