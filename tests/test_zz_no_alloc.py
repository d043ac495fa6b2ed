"""ep_layout_noalloc, the handle's maps without a group or an allocation,
against the entry point it varies: ep_create_handle + ep_handle_get_map.

Each case makes two calls in a row on the same GPU (the library's fixed
scratch array keeps the first call's contents), the second with a smaller
batch, and requires every map and count of each call to equal, bit for bit,
what a handle of a group gives for the same topk_idx -- which the parity
tests pin to the oracle (the DeepEP page's fixed LL slots and node-
deduplicated HT rows, NCCL-EP's deterministic order).  Invalid entries set
the same error bits.
"""
import ctypes

import numpy as np
import pytest
import torch

from combine_ep_route_amd import _abi as A
from gpu_util import I, dev, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu

HT_MAPS = (A.EP_MAP_HT_NODE_ROW, A.EP_MAP_HT_ROW, A.EP_MAP_HT_RANK_COUNT, A.EP_MAP_HT_RANK_OFFSET,
           A.EP_MAP_HT_EXPERT_COUNT, A.EP_MAP_HT_EXPERT_OFFSET)
LL_MAPS = (A.EP_MAP_LL_SLOT, A.EP_MAP_LL_COUNT)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _handle_maps(cfg, topk, which):
    g = ep.ep_create_group(**cfg)
    try:
        h = ep.ep_create_handle(g, topk)
        maps = {m: get_map(h, m) for m in which}
        err = ep.ep_get_device_error(g)
        ep.ep_destroy_handle(h)
        return maps, err
    finally:
        ep.ep_destroy_group(g)


def _noalloc_maps(cfg, topk, which, shapes):
    outs = {m: torch.full(shapes[m], -99, dtype=torch.int32, device="cuda") for m in which}
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ep.ep_layout_noalloc(topk, outs, device_error=err, **cfg)
    return {m: host(t) for m, t in outs.items()}, int(host(err)[0])


def _case(cfg, topk_np):
    mode = cfg["mode"]
    n, K = topk_np.shape
    S, E, N = cfg["num_src_ranks"], cfg["num_experts"], cfg["num_nodes"]
    R = N * cfg["ranks_per_node"]
    E2 = R if cfg.get("ht_stage2") == "rank" else E
    which = HT_MAPS if mode == "ht" else LL_MAPS
    shapes = {A.EP_MAP_HT_NODE_ROW: (n, N), A.EP_MAP_HT_ROW: (n, K), A.EP_MAP_HT_RANK_COUNT: (R,),
              A.EP_MAP_HT_RANK_OFFSET: (R,), A.EP_MAP_HT_EXPERT_COUNT: (E2,),
              A.EP_MAP_HT_EXPERT_OFFSET: (E2,), A.EP_MAP_LL_SLOT: (n, K), A.EP_MAP_LL_COUNT: (E, S)}
    topk = dev(topk_np)
    want, want_err = _handle_maps(cfg, topk, which)
    got, got_err = _noalloc_maps(cfg, topk, which, shapes)
    for m in which:
        np.testing.assert_array_equal(got[m].reshape(want[m].shape), want[m], err_msg=f"map {m}")
    assert got_err == want_err


CASES = {
    "ht_prefill": (dict(mode="ht", num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8, max_nodes_per_token=4,
                        hidden=128, max_tokens_per_rank=4096, num_src_ranks=1, payload="fp8"), 4096, 1000),
    "ht_per_rank": (dict(mode="ht", num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8,
                         max_nodes_per_token=4, hidden=128, max_tokens_per_rank=1500, num_src_ranks=3,
                         payload="fp8", ht_stage2="rank"), 3 * 1500, 3 * 333),
    "ll_decode": (dict(mode="ll", num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8, max_nodes_per_token=4,
                       hidden=128, max_tokens_per_rank=128, num_src_ranks=64, payload="fp8"), 64 * 128, 64 * 37),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_layout_equals_the_handle_twice(name):
    cfg, n1, n2 = CASES[name]
    for r, n in enumerate((n1, n2)):
        say(f"no-alloc layout {name}: call {r + 1}, {n} tokens")
        if name == "ll_decode":
            scores = I.page_scores(n, 256, seed=70 + r).astype(np.float32)
            import oracle
            topk = oracle.route(scores, 8, 8, 4)
        else:
            topk = I.random_topk(n, 256, 8, seed=80 + r)
        _case(cfg, topk)


def test_noalloc_invalid_entries_and_empty():
    cfg = dict(mode="ht", num_nodes=4, ranks_per_node=2, num_experts=64, top_k=4, max_nodes_per_token=0,
               hidden=128, max_tokens_per_rank=60, num_src_ranks=3, payload="fp8")
    topk = I.random_topk(3 * 50, 64, 4, seed=77)
    topk[0, 0] = 64
    topk[7, 3] = topk[7, 1]
    say("no-alloc layout with invalid entries, then an empty batch")
    _case(cfg, topk)
    _case(cfg, np.zeros((0, 4), np.int32))


def test_noalloc_rejects_what_exceeds_its_scratch():
    n = 120_000
    topk = torch.zeros((n, 8), dtype=torch.int32, device="cuda")
    outs = {A.EP_MAP_LL_SLOT: torch.empty((n, 8), dtype=torch.int32, device="cuda"),
            A.EP_MAP_LL_COUNT: torch.empty((256, 1), dtype=torch.int32, device="cuda")}
    with pytest.raises(ep.EpError) as e:
        ep.ep_layout_noalloc(topk, outs, mode="ll", num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8,
                             max_nodes_per_token=0, hidden=128, max_tokens_per_rank=n, num_src_ranks=1)
    assert "EP_ERR_CAPACITY" in str(e.value)
