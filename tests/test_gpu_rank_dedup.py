"""HT with the per-rank stage 2 (one copy per destination GPU, DeepEP's
received top-k form), GPU vs oracle.

"NVSHMEM and DeepEP: GPU-initiated communication", high-throughput section:
the traffic study compares one copy per expert, per destination GPU and per
destination node (6.70 / 6.26 / 3.36 cross-node copies per token with the
node limit).  With the per-rank stage 2 a rank receives one row per token
that uses it, with the token's entries local to it; the experts' weighted
partial sums come back per rank and the combine sums them.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import page_sim
from gpu_util import A, I, buffer, dev, ep, get_map, group_for, host, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _run(w, weights, fp8=True):
    """Route, handle and dispatch with the per-rank stage 2; compare maps,
    counts, rows and metadata with the oracle.  Returns (group, handle, topk,
    per-rank layout)."""
    S, T, K, H = w.num_src_ranks, w.tokens_per_rank, w.top_k, w.hidden
    E, N, G = w.num_experts, w.num_nodes, w.ranks_per_node
    R = N * G
    scores = I.scores_for(w)
    x = I.tokens_for(w)
    g = group_for(w, ht_stage2="rank", payload="fp8" if fp8 else "bf16")
    try:
        topk_d = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        h = ep.ep_create_handle(g, topk_d)
        counts = torch.zeros(R, dtype=torch.int32, device="cuda")
        ep.ep_dispatch(h, x.cuda(), topk_weights=dev(weights), recv_counts=counts)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, N, K, w.max_nodes))
        lay1 = oracle.layout_ht(topk, S, E, N, G)
        lay = oracle.layout_ht_rank(topk, S, E, R)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), lay1["node_row"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay["row2"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_COUNT), lay["c2"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_OFFSET), lay["off2"])
        np.testing.assert_array_equal(host(counts), lay["c2"])
        for r in (0, R // 2, R - 1):
            assert ep.ep_handle_get_num_recv(h, r) == lay["c2"][r]
        rows1, rows2 = int(lay1["c1"].sum()), int(lay["c2"].sum())
        assert ep.ep_handle_get_num_recv(h, -1) == rows2
        meta = oracle.pack_ht(I.bf16_bits(x[:1]), topk, weights, T, N, True, lay1["node_row"], lay["row2"],
                              rows1, rows2, with_payload=False)
        for name, which in [("meta2_src", A.EP_BUF_HT_STAGE2_SRC), ("meta2_tok", A.EP_BUF_HT_STAGE2_TOKEN),
                            ("meta2_k", A.EP_BUF_HT_STAGE2_K), ("meta1_tok", A.EP_BUF_HT_STAGE1_TOKEN),
                            ("meta1_topk", A.EP_BUF_HT_STAGE1_TOPK)]:
            np.testing.assert_array_equal(host(buffer(g, which)[:rows2 if "2" in name else rows1]),
                                          meta[name], err_msg=name)
        mt, mw = oracle.meta_ht_rank(topk, weights, lay["row2"], E, R, rows2)
        np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2_TOPK)[:rows2]), mt)
        np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2_WEIGHTS)[:rows2]), mw)
        st1, st2 = buffer(g, A.EP_BUF_HT_STAGE1), buffer(g, A.EP_BUF_HT_STAGE2)
        # every row of both stages against the oracle's own pack
        pk = oracle.pack_ht(I.bf16_bits(x), topk, weights, T, N, fp8, lay1["node_row"], lay["row2"],
                            rows1, rows2)
        np.testing.assert_array_equal(host(st1[:rows1]), pk["stage1"], err_msg="stage 1")
        np.testing.assert_array_equal(host(st2[:rows2]), pk["stage2"], err_msg="stage 2")
        return g, h, topk, lay
    except BaseException:
        ep.ep_destroy_group(g)
        raise


def test_per_rank_dispatch_all_rows_and_combine():
    w = I.HT_PREFILL.with_(num_src_ranks=3, tokens_per_rank=700, hidden=1024, seed=31)
    say("HT per-rank stage 2: S=3 T=700 H=1024 (all rows)")
    weights = I.normal_weights(w.num_tokens, 8, 31)
    g, h, topk, lay = _run(w, weights)
    try:
        rows2 = int(lay["c2"].sum())
        # combine: the token's rank rows summed in the order of the entries naming them
        P = I.bf16_bits(I.normal_bf16(rows2, 1024, 32))
        out = torch.empty((w.num_tokens, 1024), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, _bf16(P), None, out)
        np.testing.assert_array_equal(host(out), oracle.combine(P, np.ones((w.num_tokens, 8), np.float32),
                                                                lay["row2"]))
        gx = torch.empty_like(out)
        ep.ep_dispatch_backward(h, _bf16(P), gx)
        np.testing.assert_array_equal(host(gx), oracle.dispatch_backward(P, lay["row2"]))
        with pytest.raises(ep.EpError) as ei:
            ep.ep_combine(h, _bf16(P), dev(weights), out)
        assert ei.value.status == A.EP_ERR_INVALID_ARGUMENT
        with pytest.raises(ep.EpError) as ei:
            ep.ep_combine_backward(h, out, dev(weights), _bf16(P))
        assert ei.value.status == A.EP_ERR_UNSUPPORTED
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_per_rank_bf16_payload():
    """The per-rank stage 2 with BF16 rows (14336 bytes at hidden 7168): every
    row, map and received top-k against the oracle."""
    w = I.HT_PREFILL.with_(num_src_ranks=2, tokens_per_rank=150, seed=35)
    say("HT per-rank stage 2, BF16 payload: S=2 T=150 H=7168 (all rows)")
    g, h, topk, lay = _run(w, I.normal_weights(w.num_tokens, 8, 35), fp8=False)
    try:
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_per_rank_prefill_shape_page_counts():
    """4096 tokens, seed 0: the cross-node per-rank rows are the page's 6.26
    copies per token exactly (the study's total); every row of both stages."""
    w = I.HT_PREFILL
    say("HT per-rank stage 2 at the prefill shape (all rows)")
    g, h, topk, lay = _run(w, I.normal_weights(4096, 8, w.seed))
    try:
        counts = host(ep.ep_handle_get_map(h, A.EP_MAP_HT_EXPERT_COUNT))
        cross = int(counts[8:].sum())                 # ranks outside node 0
        st = page_sim.traffic(topk)
        assert cross == st["per_gpu"] * 4096
        assert round(cross / 4096, 2) == 6.26
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
