"""Seeded random configurations through the whole path, GPU vs oracle.

Each case draws a valid topology and batch -- odd node and rank counts,
K not a multiple of M, ragged token counts, both modes and both payloads --
and runs route, handle, dispatch and combine through the C ABI; routing,
maps, counts, every row or message and every output token must equal the
oracle's.  The draws are fixed by the seed, so the cases are the same on
every run.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, buffer, dev, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.choice([1, 2, 3, 4, 5, 8]))
    G = int(rng.choice([1, 2, 3, 4]))
    R = N * G
    L = int(rng.choice([1, 2, 3, 4]))
    E = R * L
    K = int(rng.integers(1, min(E, 12) + 1))
    P = E // N
    Ms = [0] + [m for m in range(1, N) if -(-K // m) <= P and m * P >= K]
    M = int(rng.choice(Ms))
    S = int(rng.integers(1, min(R, 4) + 1))
    T = int(rng.integers(1, 150))
    mode = str(rng.choice(["ll", "ht"]))
    payload = str(rng.choice(["fp8", "bf16"]))
    H = int(rng.choice([128, 256, 384, 640])) if payload == "fp8" else int(rng.choice([16, 48, 256, 528]))
    return dict(N=N, G=G, E=E, K=K, M=M, S=S, T=T, mode=mode, payload=payload, H=H)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("seed", range(64))
def test_random_config_whole_path(seed):
    c = _draw(1000 + seed)
    N, G, E, K, M, S, T, H = c["N"], c["G"], c["E"], c["K"], c["M"], c["S"], c["T"], c["H"]
    fp8, ll = c["payload"] == "fp8", c["mode"] == "ll"
    n = S * T
    say(f"random config {seed}: {c}")
    scores = I.uniform_scores(n, E, seed=2000 + seed).astype(np.float32)
    x = I.normal_bf16(n, H, 3000 + seed)
    wts = I.normal_weights(n, K, 4000 + seed)
    T_max = T + int(seed % 3)
    g = ep.ep_create_group(mode=c["mode"], num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T_max, num_src_ranks=S,
                           payload=c["payload"])
    try:
        topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, N, K, M))
        h = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h, x.cuda(), topk_weights=None if ll else dev(wts))
        xb = I.bf16_bits(x)
        if ll:
            cnt, slot, _ = oracle.layout_ll(topk, S, E, T_max)
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_COUNT), cnt)
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_SLOT), slot)
            used = np.unique(slot[slot >= 0])
            dense = np.where(slot >= 0, np.searchsorted(used, slot), -1).astype(np.int32)
            want = oracle.pack_ll(xb, T, K, fp8, dense, len(used))
            got = host(ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)[torch.from_numpy(used.astype(np.int64)).cuda()])
            np.testing.assert_array_equal(got, want)
            loc, rows = slot, E * S * T_max
        else:
            lay = oracle.layout_ht(topk, S, E, N, G)
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), lay["node_row"])
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay["row2"])
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_RANK_COUNT), lay["c1"])
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_COUNT), lay["c2"])
            r1, r2 = int(lay["c1"].sum()), int(lay["c2"].sum())
            pk = oracle.pack_ht(xb, topk, wts, T, N, fp8, lay["node_row"], lay["row2"], r1, r2)
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE1)[:r1]), pk["stage1"])
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:r2]), pk["stage2"])
            for name, which in [("meta1_tok", A.EP_BUF_HT_STAGE1_TOKEN), ("meta1_src", A.EP_BUF_HT_STAGE1_SRC),
                                ("meta1_topk", A.EP_BUF_HT_STAGE1_TOPK), ("meta1_w", A.EP_BUF_HT_STAGE1_WEIGHTS),
                                ("meta2_src", A.EP_BUF_HT_STAGE2_SRC), ("meta2_tok", A.EP_BUF_HT_STAGE2_TOKEN),
                                ("meta2_k", A.EP_BUF_HT_STAGE2_K)]:
                m = r1 if "1" in name else r2
                np.testing.assert_array_equal(host(buffer(g, which)[:m]), pk[name], err_msg=name)
            loc, rows = lay["row2"], max(r2, 1)
        Y = I.normal_bf16(rows, H, 5000 + seed)
        Yd = Y.cuda().view(E, S * T_max, H) if ll else Y.cuda()
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, Yd, dev(wts), out)
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, loc))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("seed", range(48))
def test_random_config_variants(seed):
    """The same draws with the other features: HT with the per-rank stage 2
    (unit-weight combine of rank rows), LL staged (send_only + ep_complete for
    dispatch and combine), and in both modes the backward adjoints on the
    handle -- row gradients and token gradients bit for bit, weight gradients
    within the fp32 dot-product bound."""
    c = _draw(7000 + seed)
    N, G, E, K, M, S, T, H = c["N"], c["G"], c["E"], c["K"], c["M"], c["S"], c["T"], c["H"]
    fp8, ll = c["payload"] == "fp8", c["mode"] == "ll"
    per_rank = (not ll) and seed % 2 == 0
    R, n = N * G, S * T
    say(f"random variant {seed}: {c} per_rank={per_rank}")
    scores = I.uniform_scores(n, E, seed=8000 + seed).astype(np.float32)
    x = I.normal_bf16(n, H, 9000 + seed)
    wts = I.normal_weights(n, K, 10000 + seed)
    T_max = T + int(seed % 2)
    g = ep.ep_create_group(mode=c["mode"], num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T_max, num_src_ranks=S,
                           payload=c["payload"], ht_stage2="rank" if per_rank else "expert")
    try:
        topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, N, K, M))
        h = ep.ep_create_handle(g, topk_d)
        xb = I.bf16_bits(x)
        if ll:
            counts = torch.zeros((E, S), dtype=torch.int32, device="cuda")
            ep.ep_dispatch(h, x.cuda(), recv_counts=counts, send_only=True)
            ep.ep_complete(h)
            cnt, loc, _ = oracle.layout_ll(topk, S, E, T_max)
            np.testing.assert_array_equal(host(counts), cnt)
            used = np.unique(loc[loc >= 0])
            dense = np.where(loc >= 0, np.searchsorted(used, loc), -1).astype(np.int32)
            got = host(ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)[torch.from_numpy(used.astype(np.int64)).cuda()])
            np.testing.assert_array_equal(got, oracle.pack_ll(xb, T, K, fp8, dense, len(used)))
            rows = E * S * T_max
        else:
            ep.ep_dispatch(h, x.cuda(), topk_weights=dev(wts))
            lay1 = oracle.layout_ht(topk, S, E, N, G)
            lay = oracle.layout_ht_rank(topk, S, E, R) if per_rank else lay1
            loc = lay["row2"]
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), loc)
            r1, r2 = int(lay1["c1"].sum()), int(lay["c2"].sum())
            pk = oracle.pack_ht(xb, topk, wts, T, N, fp8, lay1["node_row"], loc, r1, r2)
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:r2]), pk["stage2"])
            if per_rank:
                mt, mw = oracle.meta_ht_rank(topk, wts, loc, E, R, r2)
                np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2_TOPK)[:r2]), mt)
                np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2_WEIGHTS)[:r2]), mw)
            rows = max(r2, 1)
        Y = I.normal_bf16(rows, H, 11000 + seed)
        Yd = Y.cuda().view(E, S * T_max, H) if ll else Y.cuda()
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        if ll:
            ep.ep_combine(h, Yd, dev(wts), out, send_only=True)
            ep.ep_complete(h)
        else:
            ep.ep_combine(h, Yd, None if per_rank else dev(wts), out)
        cw = np.ones((n, K), np.float32) if per_rank else wts
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), cw, loc))
        if not per_rank:
            gb = I.bf16_bits(I.normal_bf16(n, H, 12000 + seed))
            dY = torch.zeros(Yd.shape, dtype=torch.bfloat16, device="cuda")
            dw = torch.empty((n, K), dtype=torch.float32, device="cuda")
            ep.ep_combine_backward(h, torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16).cuda(),
                                   dev(wts), dY, expert_out=Yd, grad_weights=dw)
            want_dY, want_dw, absum = oracle.combine_backward(gb, wts, loc, rows, I.bf16_bits(Y))
            used = np.unique(loc[loc >= 0])
            np.testing.assert_array_equal(host(dY.view(rows, H))[used], want_dY[used])
            bound = 2.0 * H * 2.0**-24 * absum + 1e-30
            assert np.all(np.abs(host(dw).astype(np.float64) - want_dw) <= bound)
            gx = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
            ep.ep_dispatch_backward(h, Yd, gx)
            np.testing.assert_array_equal(host(gx), oracle.dispatch_backward(I.bf16_bits(Y), loc))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def _draw_large(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.choice([2, 4, 8, 16]))
    G = int(rng.choice([1, 2, 4, 8]))
    R = N * G
    L = int(rng.choice([l for l in (1, 2, 4, 8, 16) if R * l <= 1024]))
    E = R * L
    K = int(rng.integers(1, min(E, 16) + 1))
    P = E // N
    Ms = [0] + [m for m in range(1, N) if -(-K // m) <= P and m * P >= K]
    return dict(N=N, G=G, E=E, K=K, M=int(rng.choice(Ms)), S=int(rng.integers(1, min(R, 6) + 1)),
                T=int(rng.integers(200, 2500)), mode=str(rng.choice(["ll", "ht"])))


@pytest.mark.parametrize("seed", range(24))
def test_random_large_batches_layout_and_rows(seed):
    """Larger random batches (200-2500 tokens per source, up to 6 sources, up
    to 16 nodes, up to 1024 experts): many tiles per key, so the scans'
    chunked paths, in registers and in memory, run.
    Routing, maps, counts and every row or message (FP8, hidden 128) against
    the oracle."""
    c = _draw_large(13000 + seed)
    N, G, E, K, M, S, T = c["N"], c["G"], c["E"], c["K"], c["M"], c["S"], c["T"]
    ll, H, n = c["mode"] == "ll", 128, S * T
    say(f"random large batch {seed}: {c}")
    scores = I.uniform_scores(n, E, seed=14000 + seed).astype(np.float32)
    x = I.normal_bf16(n, H, 15000 + seed)
    wts = I.normal_weights(n, K, 16000 + seed)
    g = ep.ep_create_group(mode=c["mode"], num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T, num_src_ranks=S, payload="fp8")
    try:
        topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, N, K, M))
        h = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h, x.cuda(), topk_weights=None if ll else dev(wts))
        xb = I.bf16_bits(x)
        if ll:
            cnt, slot, _ = oracle.layout_ll(topk, S, E, T)
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_COUNT), cnt)
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_SLOT), slot)
            used = np.unique(slot[slot >= 0])
            dense = np.where(slot >= 0, np.searchsorted(used, slot), -1).astype(np.int32)
            got = host(ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)[torch.from_numpy(used.astype(np.int64)).cuda()])
            np.testing.assert_array_equal(got, oracle.pack_ll(xb, T, K, True, dense, len(used)))
        else:
            lay = oracle.layout_ht(topk, S, E, N, G)
            for which, key in [(A.EP_MAP_HT_NODE_ROW, "node_row"), (A.EP_MAP_HT_ROW, "row2"),
                               (A.EP_MAP_HT_RANK_COUNT, "c1"), (A.EP_MAP_HT_RANK_OFFSET, "off1"),
                               (A.EP_MAP_HT_EXPERT_COUNT, "c2"), (A.EP_MAP_HT_EXPERT_OFFSET, "off2")]:
                np.testing.assert_array_equal(get_map(h, which), lay[key], err_msg=key)
            r1, r2 = int(lay["c1"].sum()), int(lay["c2"].sum())
            pk = oracle.pack_ht(xb, topk, wts, T, N, True, lay["node_row"], lay["row2"], r1, r2)
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE1)[:r1]), pk["stage1"])
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:r2]), pk["stage2"])
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("mode", ["ht", "ll"])
def test_handle_slot_reuse_with_changing_batches(mode):
    """Twelve handles in turn through a two-slot pool on one group, with the
    batch growing and shrinking (1 .. T_max tokens per source, LL across the
    one-launch and two-launch handle paths): every handle's maps, counts,
    rows and combine equal the oracle's, so nothing of an earlier, larger
    handle leaks into a later one."""
    N, G, E, K, M, S, T_max, H = 4, 2, 64, 6, 2, 3, 400, 128
    say(f"handle slot reuse {mode}")
    g = ep.ep_create_group(mode=mode, num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T_max, num_src_ranks=S,
                           payload="fp8", max_handles=2)
    try:
        for j, T in enumerate([400, 3, 257, 64, 1, 399, 130, 5, 256, 2, 300, 65]):
            n = S * T
            scores = I.uniform_scores(n, E, seed=17000 + j).astype(np.float32)
            x = I.normal_bf16(n, H, 17100 + j)
            wts = I.normal_weights(n, K, 17200 + j)
            topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
            ep.ep_route(g, dev(scores), topk_d)
            topk = host(topk_d)
            h = ep.ep_create_handle(g, topk_d)
            ep.ep_dispatch(h, x.cuda(), topk_weights=None if mode == "ll" else dev(wts))
            xb = I.bf16_bits(x)
            if mode == "ll":
                cnt, loc, _ = oracle.layout_ll(topk, S, E, T_max)
                np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_COUNT), cnt, err_msg=f"T={T}")
                np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_SLOT), loc, err_msg=f"T={T}")
                used = np.unique(loc[loc >= 0])
                dense = np.where(loc >= 0, np.searchsorted(used, loc), -1).astype(np.int32)
                got = host(ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)[torch.from_numpy(used.astype(np.int64)).cuda()])
                np.testing.assert_array_equal(got, oracle.pack_ll(xb, T, K, True, dense, len(used)))
                rows = E * S * T_max
            else:
                lay = oracle.layout_ht(topk, S, E, N, G)
                for which, key in [(A.EP_MAP_HT_NODE_ROW, "node_row"), (A.EP_MAP_HT_ROW, "row2"),
                                   (A.EP_MAP_HT_RANK_COUNT, "c1"), (A.EP_MAP_HT_RANK_OFFSET, "off1"),
                                   (A.EP_MAP_HT_EXPERT_COUNT, "c2"), (A.EP_MAP_HT_EXPERT_OFFSET, "off2")]:
                    np.testing.assert_array_equal(get_map(h, which), lay[key], err_msg=f"{key} T={T}")
                r1, r2 = int(lay["c1"].sum()), int(lay["c2"].sum())
                pk = oracle.pack_ht(xb, topk, wts, T, N, True, lay["node_row"], lay["row2"], r1, r2)
                np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:r2]), pk["stage2"])
                loc, rows = lay["row2"], r2
            Y = I.normal_bf16(rows, H, 17300 + j)
            out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
            ep.ep_combine(h, Y.cuda().view(E, S * T_max, H) if mode == "ll" else Y.cuda(), dev(wts), out)
            np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, loc), err_msg=f"T={T}")
            assert ep.ep_get_device_error(g) == 0
            ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("seed", range(32))
def test_random_prequantised_dispatch_and_partitions(seed):
    """Random draws (FP8 groups): ep_quantize then a dispatch of the FP8
    tokens with their scales writes exactly what the dispatch of the BF16
    tokens writes, and ep_get_partition of random ranks is exactly that
    rank's slice of the whole receive buffer."""
    c = _draw(19000 + seed)
    N, G, E, K, M, S, T = c["N"], c["G"], c["E"], c["K"], c["M"], c["S"], c["T"]
    H = int(np.random.default_rng(seed).choice([128, 256, 512]))
    ll, R, n = c["mode"] == "ll", N * G, S * T
    say(f"random pre-quantised dispatch {seed}: {c} H={H}")
    scores = I.uniform_scores(n, E, seed=19100 + seed).astype(np.float32)
    x = I.normal_bf16(n, H, 19200 + seed)
    wts = I.normal_weights(n, K, 19300 + seed)
    images = []
    for form in ("bf16", "fp8"):
        g = ep.ep_create_group(mode=c["mode"], num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                               max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T, num_src_ranks=S,
                               payload="fp8")
        try:
            topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
            ep.ep_route(g, dev(scores), topk_d)
            h = ep.ep_create_handle(g, topk_d)
            w = None if ll else dev(wts)
            if form == "bf16":
                ep.ep_dispatch(h, x.cuda(), topk_weights=w)
            else:
                q = torch.empty((n, H), dtype=torch.float8_e4m3fn, device="cuda")
                sc = torch.empty((n, H // 128), dtype=torch.float32, device="cuda")
                ep.ep_quantize(g, x.cuda(), q, sc)
                ep.ep_dispatch(h, q, scales=sc, topk_weights=w)
            which = A.EP_BUF_LL_RECV if ll else A.EP_BUF_HT_STAGE2
            whole = ep.ep_handle_get_buffer(h, which)
            if ll:
                loc = get_map(h, A.EP_MAP_LL_SLOT)
                used = torch.from_numpy(np.unique(loc[loc >= 0]).astype(np.int64)).cuda()
                images.append(host(whole[used]))
            else:
                r2 = ep.ep_handle_get_num_recv(h, -1)
                images.append(host(whole[:r2]))
            # partitions of a few ranks are slices of the whole buffer
            per = E // R * S * T if ll else None
            for r in sorted({0, R - 1, int(np.random.default_rng(seed + 5).integers(0, R))}):
                part = ep.ep_get_partition(h, r, which)
                if ll:
                    first, count = r * per, per
                else:
                    offs = get_map(h, A.EP_MAP_HT_EXPERT_OFFSET)
                    cnts = get_map(h, A.EP_MAP_HT_EXPERT_COUNT)
                    L = E // R
                    first, count = int(offs[r * L]), int(cnts[r * L:(r + 1) * L].sum())
                assert part.shape[0] == count
                if count:
                    assert part.data_ptr() == whole[first].data_ptr()
                    np.testing.assert_array_equal(host(part), host(whole[first:first + count]))
            assert ep.ep_get_device_error(g) == 0
            ep.ep_destroy_handle(h)
        finally:
            ep.ep_destroy_group(g)
    np.testing.assert_array_equal(images[0], images[1])
