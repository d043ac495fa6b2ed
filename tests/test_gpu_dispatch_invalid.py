"""Dispatch of caller-supplied routings that hold invalid entries, GPU vs
oracle: maps, counts, every row or message, and all metadata.

"NCCL EP paper notes", tensor abstraction: topk_idx [n, K] is the caller's.
An entry out of [0, E) or repeating an earlier entry of its token's row
takes no slot or row; the device error word flags it; the token's other
entries are dispatched as usual, and the stage-1 metadata keeps the token's
row as given.  The dispatch checks a token's entries lane by lane, so the
cases put invalid entries at the first, middle and last positions of a
row, several in one row, and make whole rows invalid.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, buffer, dev, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _corrupted_topk(n, E, K, seed):
    topk = I.random_topk(n, E, K, seed=seed)
    topk[0, 0] = E                      # out of range, first position
    topk[1, K - 1] = topk[1, 0]         # repeat, last position
    topk[2, :] = -1                     # a whole row of -1
    topk[3, 1] = -5
    topk[3, 2] = E + 3                  # two bad entries in one row
    topk[4, K // 2] = topk[4, K // 2 - 1]   # repeat in the middle
    topk[5, :] = topk[5, 0]             # every entry the same expert
    rng = np.random.default_rng(seed + 1)
    for i in rng.choice(np.arange(6, n), size=n // 10, replace=False):
        k = int(rng.integers(K))
        topk[i, k] = int(rng.choice([-1, E, E + 17, topk[i, (k + 1) % K]]))
    return np.ascontiguousarray(topk)


@pytest.mark.parametrize("stage2", ["expert", "rank"])
def test_ht_dispatch_invalid_entries(stage2):
    S, T, E, N, G, K, H = 2, 70, 64, 4, 2, 6, 256
    R = N * G
    n = S * T
    say(f"HT dispatch with invalid entries, stage 2 per {stage2}")
    topk = _corrupted_topk(n, E, K, seed=90)
    x = I.normal_bf16(n, H, 91)
    weights = I.normal_weights(n, K, 92)
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=T, num_src_ranks=S,
                           payload="fp8", ht_stage2=stage2)
    try:
        h = ep.ep_create_handle(g, dev(topk))
        ep.ep_dispatch(h, x.cuda(), topk_weights=dev(weights))
        lay1 = oracle.layout_ht(topk, S, E, N, G)
        lay2 = lay1 if stage2 == "expert" else oracle.layout_ht_rank(topk, S, E, R)
        assert lay1["err"] != 0
        assert ep.ep_get_device_error(g) == lay1["err"]
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), lay1["node_row"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay2["row2"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_RANK_COUNT), lay1["c1"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_RANK_OFFSET), lay1["off1"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_COUNT), lay2["c2"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_OFFSET), lay2["off2"])
        rows1, rows2 = int(lay1["c1"].sum()), int(lay2["c2"].sum())
        pk = oracle.pack_ht(I.bf16_bits(x), topk, weights, T, N, True, lay1["node_row"], lay2["row2"],
                            rows1, rows2)
        np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE1)[:rows1]), pk["stage1"],
                                      err_msg="stage 1")
        np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:rows2]), pk["stage2"],
                                      err_msg="stage 2")
        for name, which in [("meta1_tok", A.EP_BUF_HT_STAGE1_TOKEN), ("meta1_src", A.EP_BUF_HT_STAGE1_SRC),
                            ("meta1_topk", A.EP_BUF_HT_STAGE1_TOPK), ("meta1_w", A.EP_BUF_HT_STAGE1_WEIGHTS)]:
            np.testing.assert_array_equal(host(buffer(g, which)[:rows1]), pk[name], err_msg=name)
        for name, which in [("meta2_src", A.EP_BUF_HT_STAGE2_SRC), ("meta2_tok", A.EP_BUF_HT_STAGE2_TOKEN),
                            ("meta2_k", A.EP_BUF_HT_STAGE2_K)]:
            np.testing.assert_array_equal(host(buffer(g, which)[:rows2]), pk[name], err_msg=name)
        if stage2 == "rank":
            mt, mw = oracle.meta_ht_rank(topk, weights, lay2["row2"], E, R, rows2)
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2_TOPK)[:rows2]), mt)
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2_WEIGHTS)[:rows2]), mw)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ll_dispatch_invalid_entries():
    S, T, E, K, H, slots = 3, 50, 64, 5, 512, 64
    n = S * T
    say("LL dispatch with invalid entries")
    topk = _corrupted_topk(n, E, K, seed=95)
    x = I.normal_bf16(n, H, 96)
    g = ep.ep_create_group(mode="ll", num_nodes=4, ranks_per_node=2, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=slots, num_src_ranks=S,
                           payload="fp8")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        counts = torch.zeros((E, S), dtype=torch.int32, device="cuda")
        ep.ep_dispatch(h, x.cuda(), recv_counts=counts)
        want_cnt, want_slot, err = oracle.layout_ll(topk, S, E, slots)
        assert err != 0
        assert ep.ep_get_device_error(g) == err
        np.testing.assert_array_equal(host(counts), want_cnt)
        slot = get_map(h, A.EP_MAP_LL_SLOT)
        np.testing.assert_array_equal(slot, want_slot)
        used = np.unique(slot[slot >= 0])
        dense = np.where(slot >= 0, np.searchsorted(used, slot), -1).astype(np.int32)
        want = oracle.pack_ll(I.bf16_bits(x), T, K, True, dense, len(used))
        got = host(buffer(g, A.EP_BUF_LL_RECV)[torch.from_numpy(used.astype(np.int64)).cuda()])
        np.testing.assert_array_equal(got, want)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
