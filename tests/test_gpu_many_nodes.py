"""Topology and routing extremes, GPU vs oracle.

- 64 nodes, the node count's upper limit (one bit per node in a 64-bit
  mask): node-limited routing with few experts per node (the generic routing
  kernel), HT stage-1 rows over 64 destination nodes, the HT layout's maps
  and counts, LL with one expert per node, and the combine.
- top-k equal to the number of experts.
- one token per source and one slot per (expert, source).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, host, need_gpu, say
from test_gpu_parity import _ht_compare, _ht_dispatch, _ll_dispatch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_ht_dispatch_and_combine_on_64_nodes():
    w = I.HT_PREFILL.with_(num_nodes=64, ranks_per_node=2, num_experts=256, top_k=8, max_nodes=4, hidden=512,
                           num_src_ranks=2, tokens_per_rank=100, seed=81)
    say("HT on 64 nodes x 2 ranks, 256 experts, top-8 over at most 4 nodes, H=512")
    x = I.tokens_for(w)
    wts = I.normal_weights(w.num_tokens, 8, 81)
    g, topk, lay = _ht_dispatch(w, x, I.scores_for(w), wts)
    try:
        assert ((topk // 4)[:, :, None] == np.arange(64)).any(axis=1).sum(axis=1).max() <= 4   # <= 4 nodes
        rows2 = int(lay["c2"].sum())
        Y = I.normal_bf16(rows2, 512, 82)
        out = torch.empty((w.num_tokens, 512), dtype=torch.bfloat16, device="cuda")
        h = ep.ep_create_handle(g, dev(topk))
        ep.ep_combine(h, Y.cuda(), dev(wts), out)
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, lay["row2"]))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("S,T,G,K", [(3, 90, 1, 8), (2, 130, 4, 16)])
def test_ht_layout_on_64_nodes(S, T, G, K):
    E = 64 * G * 2
    say(f"HT layout on 64 nodes x {G}: E={E} K={K} S={S} T={T}")
    _ht_compare(I.random_topk(S * T, E, K, seed=83 + G), S, E, 64, G)


def test_ll_dispatch_on_64_nodes():
    say("LL on 64 nodes x 1 rank, one expert per node, top-4 over at most 4 nodes")
    _ll_dispatch(2, 60, 64, 4, 256, "fp8", 64, seed=85, N=64, G=1, M=4)


@pytest.mark.parametrize("mode", ["ht", "ll"])
def test_top_k_equals_the_number_of_experts(mode):
    """K = E = 32: every token goes to every expert (32 rounds of the 32-lane
    maximum in the routing kernel), every slot of every (expert, source) up
    to T is taken."""
    say(f"{mode.upper()}: K = E = 32")
    if mode == "ht":
        w = I.HT_PREFILL.with_(num_nodes=2, ranks_per_node=2, num_experts=32, top_k=32, max_nodes=0, hidden=256,
                               num_src_ranks=2, tokens_per_rank=40, seed=87)
        x = I.tokens_for(w)
        g, topk, lay = _ht_dispatch(w, x, I.scores_for(w), I.normal_weights(w.num_tokens, 32, 87))
        try:
            assert (np.sort(topk, axis=1) == np.arange(32)).all()
            assert (lay["c2"] == 80).all()
        finally:
            ep.ep_destroy_group(g)
    else:
        _ll_dispatch(2, 40, 32, 32, 256, "fp8", 40, seed=88)


def test_one_token_per_source_one_slot():
    """T = T_max = 1: one tile per source holding one token, one slot per
    (expert, source)."""
    say("LL and HT with one token per source and one slot")
    _ll_dispatch(4, 1, 16, 2, 256, "fp8", 1, seed=89)
    topk = I.random_topk(4, 16, 2, seed=90)
    _ht_compare(topk, 4, 16, 2, 2)
