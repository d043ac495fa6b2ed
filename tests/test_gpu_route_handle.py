"""ep_route_handle (routing and the handle in one pass), GPU vs oracle.

The routing rule is the DeepEP page's ("NVSHMEM and DeepEP: GPU-initiated
communication", high-throughput section: node score = sum of the node's best
ceil(K/M) expert scores, M best nodes kept, K best experts among them); the
handle's counts, prefixes and maps follow the same page's LL fixed slots and
HT node-deduplicated two-stage layout with NCCL-EP's deterministic order
("NCCL EP paper notes", tensor layouts).  Every case compares the caller's
topk_idx with oracle.route and every map, count and offset of the handle
with oracle.layout_ll / layout_ht / layout_ht_rank, for the fast routing path
(route and count in one kernel) and for shapes outside it (the routing
kernel, then the count).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, group_for, host, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _check_handle(g, h, topk, mode, S, E, N, G, slots, s2_rank=False):
    if mode == "ll":
        cnt, slot, err = oracle.layout_ll(topk, S, E, slots)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_SLOT), slot)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_COUNT), cnt)
        assert ep.ep_handle_get_num_recv(h, -1) == cnt.sum()
    else:
        lay = oracle.layout_ht(topk, S, E, N, G)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), lay["node_row"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_RANK_COUNT), lay["c1"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_RANK_OFFSET), lay["off1"])
        if s2_rank:
            lay2 = oracle.layout_ht_rank(topk, S, E, N * G)
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay2["row2"])
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_COUNT), lay2["c2"])
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_OFFSET), lay2["off2"])
        else:
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay["row2"])
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_COUNT), lay["c2"])
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_OFFSET), lay["off2"])
        err = lay["err"]
    assert ep.ep_get_device_error(g) == err


def _route_handle(w, scores, **over):
    g = group_for(w, hidden=128, **over)   # the maps do not depend on the hidden size
    try:
        n, K = scores.shape[0], w.top_k
        topk_d = torch.full((n, K), -7, dtype=torch.int32, device="cuda")
        h = ep.ep_route_handle(g, dev(scores), topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, w.num_nodes, K, w.max_nodes))
        mode = over.get("mode", w.mode)
        _check_handle(g, h, topk, mode, w.num_src_ranks, w.num_experts, w.num_nodes, w.ranks_per_node,
                      over.get("max_tokens_per_rank", w.slots), s2_rank=over.get("ht_stage2") == "rank")
        ep.ep_destroy_handle(h)
        return topk
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("wname", ["ht_prefill", "ll_decode", "round_trip", "tiny"])
def test_route_handle_full_workloads(wname):
    w = I.WORKLOADS[wname]
    say(f"route+handle {wname} n={w.num_tokens}")
    topk = _route_handle(w, I.scores_for(w))
    if wname == "ht_prefill":
        lay = oracle.layout_ht(topk, 1, 256, 8, 8)
        # the page's node-dedup figure: 13,758 cross-node rows = 3.36 per token
        assert lay["c1"].sum() - lay["c1"][:8].sum() == 13758


@pytest.mark.parametrize("variant", ["ht_nolimit", "ht_rank", "ll_prefill_mode", "ht_decode_mode"])
def test_route_handle_variants(variant):
    """The no-limit routing, the per-rank stage 2, and each workload in the
    other mode."""
    say(f"route+handle variant {variant}")
    if variant == "ht_nolimit":
        w = I.HT_PREFILL.with_(max_nodes=0)
        _route_handle(w, I.scores_for(w))
    elif variant == "ht_rank":
        w = I.HT_PREFILL
        _route_handle(w, I.scores_for(w), ht_stage2="rank")
    elif variant == "ll_prefill_mode":
        w = I.HT_PREFILL.with_(tokens_per_rank=1000, num_src_ranks=3)
        _route_handle(w, I.scores_for(w), mode="ll")
    else:
        w = I.LL_DECODE
        _route_handle(w, I.scores_for(w), mode="ht")


@pytest.mark.parametrize("E,N,G,K,M,S,T", [
    (64, 4, 2, 4, 2, 3, 333),      # outside the fast path (E % 128 != 0)
    (128, 8, 2, 6, 3, 2, 257),     # fast path, V = 4, a node of 4 lanes
    (512, 8, 8, 8, 4, 1, 300),     # V = 16
    (384, 4, 4, 8, 2, 5, 61),      # V = 12 (K rounds of a maximum)
    (1024, 16, 4, 16, 5, 2, 130),  # outside the fast path (E > 512)
    (256, 8, 8, 8, 0, 4, 17),      # no limit, ragged tiles
    (256, 8, 8, 32, 8, 2, 77),     # K = 32
    (256, 8, 8, 8, 4, 1, 1),       # one token
    (16, 2, 2, 2, 0, 4, 32),       # the tiny topology
])
@pytest.mark.parametrize("mode", ["ht", "ll"])
def test_route_handle_shapes_and_ties(E, N, G, K, M, S, T, mode):
    say(f"route+handle {mode} E={E} N={N} K={K} M={M} S={S} T={T}")
    rng = np.random.default_rng(E + K + S * T)
    n = S * T
    scores = (rng.integers(0, 6, size=(n, E)) * 0.125).astype(np.float32)   # many ties
    scores[::3] = rng.random((len(scores[::3]), E)).astype(np.float32)
    w = I.Workload("case", mode, N, G, E, K, M, 128, S, T, "fp8", "uniform", "softmax_normal", seed=0)
    _route_handle(w, scores)


def test_route_handle_strided_scores_and_empty():
    """Score rows with a stride beyond E take the fast path too when 16-byte
    aligned; n = 0 creates an empty handle."""
    w = I.HT_PREFILL.with_(tokens_per_rank=500)
    scores = I.scores_for(w)
    wide = np.zeros((500, 260), np.float32)
    wide[:, :256] = scores
    g = group_for(w, hidden=128)
    try:
        topk_d = torch.empty((500, 8), dtype=torch.int32, device="cuda")
        h = ep.ep_route_handle(g, dev(wide)[:, :256], topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, 8, 8, 4))
        _check_handle(g, h, topk, "ht", 1, 256, 8, 8, 500)
        ep.ep_destroy_handle(h)
        e_sc = torch.empty((0, 256), dtype=torch.float32, device="cuda")
        e_tk = torch.empty((0, 8), dtype=torch.int32, device="cuda")
        h0 = ep.ep_route_handle(g, e_sc, e_tk)
        assert ep.ep_handle_get_num_recv(h0, -1) == 0
        ep.ep_destroy_handle(h0)
    finally:
        ep.ep_destroy_group(g)


def test_route_handle_repeated_launches_reuse_the_scan_counter():
    """Many handles in a row on one group, alternating the two entry points
    and the token counts: the prefix scan's finish counter is reset by every
    launch, so each handle equals the oracle."""
    w = I.HT_PREFILL
    g = group_for(w, hidden=128, max_handles=4)
    try:
        for r in range(12):
            n = [4096, 100, 1, 3000][r % 4]
            scores = I.page_scores(n, 256, seed=100 + r).astype(np.float32)
            topk_d = torch.empty((n, 8), dtype=torch.int32, device="cuda")
            if r % 2:
                ep.ep_route(g, dev(scores), topk_d)
                h = ep.ep_create_handle(g, topk_d)
            else:
                h = ep.ep_route_handle(g, dev(scores), topk_d)
            topk = host(topk_d)
            np.testing.assert_array_equal(topk, oracle.route(scores, 8, 8, 4))
            _check_handle(g, h, topk, "ht", 1, 256, 8, 8, n)
            ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
