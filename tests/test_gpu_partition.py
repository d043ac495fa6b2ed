"""One destination rank's partition of the receive buffers, GPU vs oracle.

"NVSHMEM and DeepEP: GPU-initiated communication", low-latency and
high-throughput sections: every rank owns the receive region of its local
experts (LL: a [local expert][source][slot] block; HT: the rows that reach
it).  With the 64 ranks as partitions of one GPU's memory, ep_get_partition
narrows the group's buffers to one rank: each view must be exactly that
rank's slice of the full buffer, hold the oracle's rows for the entries
routed to that rank, and the partitions together must tile the buffer.
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


def _ht_group(S, T, E, N, G, K, H, stage2="expert"):
    return ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                              max_nodes_per_token=0, hidden=H, max_tokens_per_rank=T, num_src_ranks=S,
                              payload="fp8", ht_stage2=stage2)


def test_ht_partition_bounds_before_any_dispatch():
    """An HT handle that no dispatch has used yet: its partition views take
    their bounds from the rank and expert offsets, which the maps-only pass
    computes when the views are asked for (the rows hold data only once a
    dispatch has run)."""
    S, T, E, N, G, K, H = 2, 90, 64, 4, 2, 4, 256
    R, L = N * G, E // (N * G)
    say(f"HT partition bounds before a dispatch: S={S} T={T} E={E} R={R} K={K}")
    topk = I.random_topk(S * T, E, K, seed=74)
    g = _ht_group(S, T, E, N, G, K, H)
    try:
        h = ep.ep_create_handle(g, dev(topk))
        lay = oracle.layout_ht(topk, S, E, N, G)
        st1, st2 = buffer(g, A.EP_BUF_HT_STAGE1), buffer(g, A.EP_BUF_HT_STAGE2)
        for r in range(R):
            o, c = int(lay["off1"][r]), int(lay["c1"][r])
            p1 = ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE1)
            assert tuple(p1.shape) == (c, st1.shape[1])
            if c:
                assert p1.data_ptr() == st1[o].data_ptr()
            o2, c2 = int(lay["off2"][r * L]), int(lay["c2"][r * L:(r + 1) * L].sum())
            p2 = ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE2)
            assert tuple(p2.shape) == (c2, st2.shape[1])
            if c2:
                assert p2.data_ptr() == st2[o2].data_ptr()
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), lay["node_row"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay["row2"])
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ht_partitions_are_the_ranks_rows():
    S, T, E, N, G, K, H = 3, 200, 64, 4, 2, 4, 256
    R, L = N * G, E // (N * G)
    say(f"HT partitions: S={S} T={T} E={E} R={R} K={K} H={H}")
    x = I.normal_bf16(S * T, H, 71)
    topk = I.random_topk(S * T, E, K, seed=72)
    g = _ht_group(S, T, E, N, G, K, H)
    try:
        h = ep.ep_create_handle(g, dev(topk))
        ep.ep_dispatch(h, x.cuda())
        lay = oracle.layout_ht(topk, S, E, N, G)
        img = oracle.token_rows(I.bf16_bits(x), True)
        st1, st2 = buffer(g, A.EP_BUF_HT_STAGE1), buffer(g, A.EP_BUF_HT_STAGE2)
        tok1_all = host(buffer(g, A.EP_BUF_HT_STAGE1_TOKEN))
        src2_all = host(buffer(g, A.EP_BUF_HT_STAGE2_SRC))
        n1 = n2 = 0
        for r in range(R):
            # stage 1: the rows of destination rank r
            o, c = int(lay["off1"][r]), int(lay["c1"][r])
            p1 = ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE1)
            assert tuple(p1.shape) == (c, st1.shape[1])
            if c:
                assert p1.data_ptr() == st1[o].data_ptr()
            rows = host(p1)
            for i, n in zip(*np.nonzero((lay["node_row"] >= o) & (lay["node_row"] < o + c))):
                np.testing.assert_array_equal(rows[lay["node_row"][i, n] - o], img[i], err_msg=f"rank {r} token {i}")
            np.testing.assert_array_equal(host(ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE1_TOKEN)),
                                          tok1_all[o:o + c])
            assert tuple(ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE1_TOPK).shape) == (c, K)
            # stage 2: the rows of rank r's L experts, expert after expert
            o2, c2 = int(lay["off2"][r * L]), int(lay["c2"][r * L:(r + 1) * L].sum())
            p2 = ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE2)
            assert tuple(p2.shape) == (c2, st2.shape[1])
            if c2:
                assert p2.data_ptr() == st2[o2].data_ptr()
            rows2 = host(p2)
            inside = (lay["row2"] >= o2) & (lay["row2"] < o2 + c2)
            assert int(inside.sum()) == c2
            for i, k in zip(*np.nonzero(inside)):
                assert topk[i, k] // L == r
                np.testing.assert_array_equal(rows2[lay["row2"][i, k] - o2], img[i], err_msg=f"rank {r} entry {i},{k}")
            np.testing.assert_array_equal(host(ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE2_SRC)),
                                          src2_all[o2:o2 + c2])
            n1 += c
            n2 += c2
        assert n1 == int(lay["c1"].sum()) and n2 == S * T * K
        for bad_rank in (-1, R):
            with pytest.raises(ep.EpError) as ei:
                ep.ep_get_partition(h, bad_rank, A.EP_BUF_HT_STAGE1)
            assert ei.value.status == A.EP_ERR_INVALID_ARGUMENT
        with pytest.raises(ep.EpError):
            ep.ep_get_partition(h, 0, A.EP_BUF_LL_RECV)          # an LL buffer id in HT
        with pytest.raises(ep.EpError):
            ep.ep_get_partition(h, 0, A.EP_BUF_HT_STAGE2_TOPK)   # exists only with the per-rank stage 2
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ht_per_rank_stage2_partitions():
    S, T, E, N, G, K, H = 2, 150, 64, 4, 2, 6, 128
    R, L = N * G, E // (N * G)
    say(f"HT per-rank stage-2 partitions: S={S} T={T} E={E} R={R} K={K}")
    x = I.normal_bf16(S * T, H, 73)
    topk = I.random_topk(S * T, E, K, seed=74)
    g = _ht_group(S, T, E, N, G, K, H, stage2="rank")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        ep.ep_dispatch(h, x.cuda())
        lay = oracle.layout_ht_rank(topk, S, E, R)
        total = 0
        for r in range(R):
            o, c = int(lay["off2"][r]), int(lay["c2"][r])
            p = ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE2_TOPK)
            assert tuple(p.shape) == (c, K)
            ids = host(p)
            assert ((ids >= -1) & (ids < L)).all()
            # every row carries at least one entry of the rank (its first one)
            assert (ids >= 0).any(axis=1).all()
            assert tuple(ep.ep_get_partition(h, r, A.EP_BUF_HT_STAGE2).shape)[0] == c
            total += c
        assert total == int(lay["c2"].sum())
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ll_partitions_follow_the_handles_buffer():
    S, T, E, N, G, K, H, slots = 2, 50, 32, 2, 2, 4, 256, 64
    R, L = N * G, E // (N * G)
    per = L * S * slots
    say(f"LL partitions: S={S} T={T} E={E} R={R} K={K} slots={slots}")
    x = I.normal_bf16(S * T, H, 75)
    topk = I.random_topk(S * T, E, K, seed=76)
    g = ep.ep_create_group(mode="ll", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=slots, num_src_ranks=S,
                           payload="fp8", max_handles=3)
    try:
        h = ep.ep_create_handle(g, dev(topk))
        with pytest.raises(ep.EpError):
            ep.ep_get_partition(h, 0, A.EP_BUF_LL_RECV)          # not dispatched yet
        ep.ep_dispatch(h, x.cuda())
        _, slot, _ = oracle.layout_ll(topk, S, E, slots)
        img = oracle.token_rows(I.bf16_bits(x), True)
        rb = img.shape[1]
        full = ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)
        for r in range(R):
            p = ep.ep_get_partition(h, r, A.EP_BUF_LL_RECV)
            assert tuple(p.shape) == (per, full.shape[1])
            assert p.data_ptr() == full[r * per].data_ptr()
            msgs = host(p)
            for i, k in zip(*np.nonzero(topk // L == r)):
                m = slot[i, k] - r * per
                assert 0 <= m < per
                np.testing.assert_array_equal(msgs[m, :rb], img[i], err_msg=f"rank {r} entry {i},{k}")
                assert list(msgs[m, rb:rb + 16].view(np.int32)) == [i % T, i // T, k, 0]
        with pytest.raises(ep.EpError):
            ep.ep_get_partition(h, 0, A.EP_BUF_HT_STAGE1)        # an HT buffer id in LL
        # the next dispatch takes the other receive buffer; each handle's view follows its own
        h2 = ep.ep_create_handle(g, dev(topk))
        ep.ep_dispatch(h2, x.cuda())
        assert ep.ep_get_partition(h2, 1, A.EP_BUF_LL_RECV).data_ptr() != \
            ep.ep_get_partition(h, 1, A.EP_BUF_LL_RECV).data_ptr()
        # a third dispatch takes the first buffer again: the first handle's
        # messages are gone, so its views are refused; the others stay
        h3 = ep.ep_create_handle(g, dev(topk))
        ep.ep_dispatch(h3, x.cuda())
        for fn in (lambda: ep.ep_get_partition(h, 1, A.EP_BUF_LL_RECV),
                   lambda: ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)):
            with pytest.raises(ep.EpError):
                fn()
        assert ep.ep_get_partition(h3, 1, A.EP_BUF_LL_RECV).data_ptr() == full[per].data_ptr()
        assert ep.ep_get_partition(h2, 1, A.EP_BUF_LL_RECV).data_ptr() != full[per].data_ptr()
        torch.cuda.synchronize()
        ep.ep_destroy_handle(h3)
        ep.ep_destroy_handle(h2)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ht_views_of_an_overwritten_handle_are_refused():
    """HT keeps one set of stage rows: after a second handle's dispatch the
    first handle's partitions and buffer views are refused, its maps and
    counts stay, and the second handle's views are served."""
    w = I.HT_PREFILL.with_(tokens_per_rank=200, hidden=256, seed=61)
    g = ep.ep_create_group(mode="ht", num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8,
                           max_nodes_per_token=4, hidden=256, max_tokens_per_rank=200, num_src_ranks=1,
                           payload="fp8", max_handles=2)
    try:
        hs, topks = [], []
        for j in range(2):
            tk = torch.empty((200, 8), dtype=torch.int32, device="cuda")
            hs.append(ep.ep_route_handle(g, dev(I.scores_for(w.with_(seed=61 + j))), tk))
            topks.append(host(tk))
        x = I.normal_bf16(200, 256, 62).cuda()
        ep.ep_dispatch(hs[0], x)
        p0 = host(ep.ep_get_partition(hs[0], 3, A.EP_BUF_HT_STAGE1_TOKEN))
        ep.ep_dispatch(hs[1], x)
        for which in (A.EP_BUF_HT_STAGE1, A.EP_BUF_HT_STAGE2, A.EP_BUF_HT_STAGE2_SRC):
            with pytest.raises(ep.EpError):
                ep.ep_get_partition(hs[0], 3, which)
            with pytest.raises(ep.EpError):
                ep.ep_handle_get_buffer(hs[0], which)
        lay0 = oracle.layout_ht(topks[0], 1, 256, 8, 8)
        np.testing.assert_array_equal(get_map(hs[0], A.EP_MAP_HT_ROW), lay0["row2"])
        lay1 = oracle.layout_ht(topks[1], 1, 256, 8, 8)
        c = int(lay1["c1"][3])
        got = host(ep.ep_get_partition(hs[1], 3, A.EP_BUF_HT_STAGE1_TOKEN))
        assert len(got) == c and len(p0) == int(lay0["c1"][3])
        for h in hs:
            ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ht_double_buffered_stage_rows():
    """With two HT stage-row sets, consecutive dispatches take them in turn:
    two handles' rows stay in place side by side (each equal to the oracle's
    rows for its own routing and tokens), a third dispatch takes the first
    set again and only the first handle's views are refused; every handle's
    combine stays valid."""
    T, H = 300, 256
    w = I.HT_PREFILL.with_(tokens_per_rank=T, hidden=H)
    g = ep.ep_create_group(mode="ht", num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8,
                           max_nodes_per_token=4, hidden=H, max_tokens_per_rank=T, num_src_ranks=1,
                           payload="fp8", max_handles=3, ht_buffers=2)
    try:
        hs, topks, xs = [], [], []
        wts = I.normal_weights(T, 8, 70)
        for j in range(3):
            tk = torch.empty((T, 8), dtype=torch.int32, device="cuda")
            hs.append(ep.ep_route_handle(g, dev(I.scores_for(w.with_(seed=70 + j))), tk))
            topks.append(host(tk))
            xs.append(I.normal_bf16(T, H, 71 + j))

        def want(j):
            lay = oracle.layout_ht(topks[j], 1, 256, 8, 8)
            return lay, oracle.pack_ht(I.bf16_bits(xs[j]), topks[j], wts, T, 8, True, lay["node_row"],
                                       lay["row2"], int(lay["c1"].sum()), int(lay["c2"].sum()))

        def check(j):
            lay, pk = want(j)
            r1, r2 = int(lay["c1"].sum()), int(lay["c2"].sum())
            np.testing.assert_array_equal(host(ep.ep_handle_get_buffer(hs[j], A.EP_BUF_HT_STAGE1)[:r1]), pk["stage1"])
            np.testing.assert_array_equal(host(ep.ep_handle_get_buffer(hs[j], A.EP_BUF_HT_STAGE2)[:r2]), pk["stage2"])
            np.testing.assert_array_equal(host(ep.ep_handle_get_buffer(hs[j], A.EP_BUF_HT_STAGE1_TOPK)[:r1]),
                                          pk["meta1_topk"])
            d = 11
            p1 = host(ep.ep_get_partition(hs[j], d, A.EP_BUF_HT_STAGE1))
            np.testing.assert_array_equal(p1, pk["stage1"][lay["off1"][d]:lay["off1"][d] + lay["c1"][d]])

        ep.ep_dispatch(hs[0], xs[0].cuda(), topk_weights=dev(wts))
        ep.ep_dispatch(hs[1], xs[1].cuda(), topk_weights=dev(wts))
        check(0)
        check(1)
        assert ep.ep_handle_get_buffer(hs[0], A.EP_BUF_HT_STAGE2).data_ptr() != \
            ep.ep_handle_get_buffer(hs[1], A.EP_BUF_HT_STAGE2).data_ptr()
        ep.ep_dispatch(hs[2], xs[2].cuda(), topk_weights=dev(wts))
        with pytest.raises(ep.EpError):
            ep.ep_handle_get_buffer(hs[0], A.EP_BUF_HT_STAGE2)
        with pytest.raises(ep.EpError):
            ep.ep_get_partition(hs[0], 3, A.EP_BUF_HT_STAGE1)
        check(1)
        check(2)
        for j in range(3):
            lay, _ = want(j)
            Y = I.normal_bf16(T * 8, H, 80 + j)
            out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            ep.ep_combine(hs[j], Y.cuda(), dev(wts), out)
            np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, lay["row2"]))
        assert ep.ep_get_device_error(g) == 0
        for h in hs:
            ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
