"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact for routing, counts, offsets, slot and row maps, FP8 codes, scales,
headers and metadata; the combine is compared bit for bit as well (the
stated tolerance, 1e-3 relative per element, is checked alongside and is
implied by equality).  Full-size workloads are compared whole: every row,
message and output token of the HT prefill, LL decode, combine and 16384-token
round-trip workloads.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, bits_of, buffer, dev, ep, get_map, group_for, host, need_gpu, route_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# A1 routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wname", ["ht_prefill", "ll_decode", "round_trip", "tiny"])
def test_route_full_workloads(wname):
    w = I.WORKLOADS[wname]
    say(f"route {wname} n={w.num_tokens}")
    scores = I.scores_for(w)
    g = group_for(w, mode="ht", max_tokens_per_rank=w.tokens_per_rank, num_src_ranks=w.num_src_ranks)
    try:
        got = route_gpu(g, scores, w.top_k)
        want = oracle.route(scores, w.num_nodes, w.top_k, w.max_nodes)
        np.testing.assert_array_equal(got, want)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("E,N,G,K,M,n", [
    (64, 4, 2, 4, 2, 1001), (128, 8, 2, 6, 3, 257), (512, 8, 8, 8, 4, 300),
    (1024, 16, 4, 16, 5, 130), (32, 2, 2, 1, 1, 65), (256, 8, 8, 8, 0, 3), (16, 2, 2, 2, 0, 1),
    (256, 8, 8, 32, 8, 77),
])
def test_route_shapes_and_ties(E, N, G, K, M, n):
    say(f"route E={E} N={N} K={K} M={M} n={n}")
    rng = np.random.default_rng(E + K + n)
    scores = (rng.integers(0, 6, size=(n, E)) * 0.125).astype(np.float32)  # many ties
    scores[::3] = rng.random((len(scores[::3]), E)).astype(np.float32)
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=128, max_tokens_per_rank=max(n, 1),
                           num_src_ranks=1, payload="fp8")
    try:
        np.testing.assert_array_equal(route_gpu(g, scores, K), oracle.route(scores, N, K, M))
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("E,N,G,K,M", [(256, 8, 8, 8, 4), (96, 4, 2, 6, 2), (256, 8, 8, 8, 0)])
def test_route_signed_zero_and_negative_ties(E, N, G, K, M):
    """-0 and +0 are equal scores (ties go to the lower index), negative and
    -inf scores order below them, on the fast (E % 128 == 0) and the generic
    routing kernels."""
    say(f"route signed-zero ties E={E} M={M}")
    rng = np.random.default_rng(E + 17)
    n = 300
    scores = rng.choice(np.array([0.0, -0.0, 0.25, -0.25, -np.inf, 1.5], np.float32), size=(n, E))
    scores[::4] = -0.0                              # all-zero rows: pure index order
    scores[1::4, ::2] = 0.0
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=128, max_tokens_per_rank=n,
                           num_src_ranks=1, payload="fp8")
    try:
        got = route_gpu(g, scores, K)
        np.testing.assert_array_equal(got, oracle.route(scores, N, K, M))
        if M == 0:
            np.testing.assert_array_equal(got[0], np.arange(K))
    finally:
        ep.ep_destroy_group(g)


def test_route_empty_and_strided():
    g = ep.ep_create_group(mode="ht", max_tokens_per_rank=64)
    try:
        ep.ep_route(g, torch.empty((0, 256), device="cuda"), torch.empty((0, 8), dtype=torch.int32, device="cuda"))
        wide = dev(I.uniform_scores(33, 300, seed=3).astype(np.float32))
        s = wide[:, 7:263]                      # row stride 300, inner contiguous
        out = torch.empty((33, 8), dtype=torch.int32, device="cuda")
        ep.ep_route(g, s, out)
        want = oracle.route(host(s.contiguous()), 8, 8, 4)
        np.testing.assert_array_equal(host(out), want)
    finally:
        ep.ep_destroy_group(g)


# ---------------------------------------------------------------------------
# A2 layout (handle maps)
# ---------------------------------------------------------------------------

def _ll_case(S, T, E, K, slots, seed, N=8, G=8, corrupt=False):
    topk = I.random_topk(S * T, E, K, seed)
    if corrupt:
        topk[3, 1] = E + 5
        topk[10, 2] = topk[10, 0]
        topk[-1, 0] = -1
    g = ep.ep_create_group(mode="ll", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=128, max_tokens_per_rank=slots,
                           num_src_ranks=S, payload="fp8")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        slot = get_map(h, A.EP_MAP_LL_SLOT)
        cnt = get_map(h, A.EP_MAP_LL_COUNT)
        err = ep.ep_get_device_error(g)
        want_cnt, want_slot, want_err = oracle.layout_ll(topk, S, E, slots)
        np.testing.assert_array_equal(slot, want_slot)
        np.testing.assert_array_equal(cnt, want_cnt)
        assert err == want_err
        n_recv = ep.ep_handle_get_num_recv(h, -1)
        assert n_recv == want_cnt.sum()
        L = E // (N * G)
        assert ep.ep_handle_get_num_recv(h, 1) == want_cnt[L:2 * L].sum()
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("S,T,E,K,slots", [
    (64, 128, 256, 8, 128), (1, 128, 256, 8, 128), (3, 300, 256, 8, 512), (5, 1000, 64, 4, 1000),
    (2, 17, 128, 12, 20), (1, 1, 256, 8, 8), (4, 257, 1024, 32, 300),
])
def test_layout_ll(S, T, E, K, slots):
    say(f"layout LL S={S} T={T} E={E} K={K}")
    _ll_case(S, T, E, K, slots, seed=S * 1000 + T)


def test_layout_ll_invalid_entries():
    _ll_case(2, 40, 64, 4, 64, seed=9, corrupt=True)


def _ht_compare(topk, S, E, N, G, T_max=None):
    T = topk.shape[0] // S
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E,
                           top_k=topk.shape[1], max_nodes_per_token=0, hidden=128,
                           max_tokens_per_rank=T_max or max(T, 1), num_src_ranks=S, payload="fp8")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        want = oracle.layout_ht(topk, S, E, N, G)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), want["node_row"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), want["row2"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_RANK_COUNT), want["c1"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_RANK_OFFSET), want["off1"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_COUNT), want["c2"])
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_EXPERT_OFFSET), want["off2"])
        assert ep.ep_get_device_error(g) == want["err"]
        L = E // (N * G)
        assert ep.ep_handle_get_num_recv(h, 2) == want["c2"][2 * L:3 * L].sum()
        ep.ep_destroy_handle(h)
        return want
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("wname", ["ht_prefill", "round_trip"])
def test_layout_ht_full_workloads(wname):
    w = I.WORKLOADS[wname]
    say(f"layout HT {wname}")
    topk = oracle.route(I.scores_for(w), w.num_nodes, w.top_k, w.max_nodes)
    want = _ht_compare(topk, 1, w.num_experts, w.num_nodes, w.ranks_per_node)
    if wname == "ht_prefill":
        # the page's node-dedup figure: 13,758 cross-node rows = 3.36 per token
        assert round((want["c1"].sum() - want["c1"][:8].sum()) / 4096, 2) == 3.36


@pytest.mark.parametrize("S,T,E,N,G,K", [
    (4, 32, 16, 2, 2, 2), (3, 600, 256, 8, 8, 8), (8, 77, 64, 4, 2, 5), (1, 1, 256, 8, 8, 8),
    (16, 300, 128, 4, 4, 16),
    # chunks longer than a scan thread's registers hold, with ragged last batches:
    # 129 tiles of one source (experts), 400 tiles over rails of two sources
    # (1024 ranks and 1024 experts), experts long while ranks fit registers
    (1, 8229, 256, 8, 8, 8), (40, 600, 1024, 32, 32, 8), (20, 900, 64, 4, 8, 5),
])
def test_layout_ht_shapes(S, T, E, N, G, K):
    say(f"layout HT S={S} T={T} E={E} N={N} G={G} K={K}")
    topk = I.random_topk(S * T, E, K, seed=S + T + E)
    _ht_compare(topk, S, E, N, G)


def test_layout_ht_invalid_entries():
    topk = I.random_topk(3 * 50, 64, 4, seed=77)
    topk[0, 0] = 64
    topk[7, 3] = topk[7, 1]
    _ht_compare(topk, 3, 64, 4, 2)


def test_handle_pool_capacity():
    g = ep.ep_create_group(mode="ll", num_nodes=2, ranks_per_node=2, num_experts=16, top_k=2,
                           max_nodes_per_token=0, hidden=128, max_tokens_per_rank=8,
                           num_src_ranks=1, payload="fp8", max_handles=2)
    try:
        t = dev(I.random_topk(8, 16, 2, seed=1))
        h1 = ep.ep_create_handle(g, t)
        h2 = ep.ep_create_handle(g, t)
        with pytest.raises(ep.EpError) as ei:
            ep.ep_create_handle(g, t)
        assert ei.value.status == A.EP_ERR_CAPACITY
        ep.ep_destroy_handle(h1)
        with pytest.raises(ep.EpError):
            ep.ep_destroy_handle(h1)             # already destroyed
        h3 = ep.ep_create_handle(g, t)
        ep.ep_destroy_handle(h2)
        ep.ep_destroy_handle(h3)
    finally:
        ep.ep_destroy_group(g)


# ---------------------------------------------------------------------------
# A3 + A4: LL dispatch
# ---------------------------------------------------------------------------

def _ll_dispatch(S, T, E, K, H, payload, slots, seed, N=2, G=2, M=0):
    fp8 = payload == "fp8"
    x = I.normal_bf16(S * T, H, seed)
    x[0, :128] = 0.0                              # an all-zero block
    if H >= 256:
        x[1, 128:256] = -0.0
    scores = I.uniform_scores(S * T, E, seed + 1).astype(np.float32)
    g = ep.ep_create_group(mode="ll", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=slots,
                           num_src_ranks=S, payload=payload)
    try:
        topk_d = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        h = ep.ep_create_handle(g, topk_d)
        counts = torch.zeros((E, S), dtype=torch.int32, device="cuda")
        ep.ep_dispatch(h, x.cuda(), recv_counts=counts)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, N, K, M))
        want_cnt, want_slot, _ = oracle.layout_ll(topk, S, E, slots)
        np.testing.assert_array_equal(host(counts), want_cnt)
        slot = get_map(h, A.EP_MAP_LL_SLOT)
        np.testing.assert_array_equal(slot, want_slot)
        buf = buffer(g, A.EP_BUF_LL_RECV)
        # every message (payload, scales, header) against the oracle's pack,
        # the used slots renumbered densely on both sides
        used = np.unique(slot[slot >= 0])
        assert len(used) == int((slot >= 0).sum())
        dense = np.where(slot >= 0, np.searchsorted(used, slot), -1).astype(np.int32)
        want = oracle.pack_ll(I.bf16_bits(x), T, K, fp8, dense, len(used))
        np.testing.assert_array_equal(host(buf[torch.from_numpy(used.astype(np.int64)).cuda()]), want)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("payload", ["fp8", "bf16"])
def test_ll_dispatch_tiny(payload):
    say(f"LL dispatch tiny {payload}")
    _ll_dispatch(4, 32, 16, 2, 256, payload, 32, seed=1)


def test_ll_dispatch_ragged_hidden():
    say("LL dispatch H=1152 (9 blocks, ragged wave), S=3 T=70")
    _ll_dispatch(3, 70, 64, 4, 1152, "fp8", 80, seed=5, N=4, G=2, M=2)


def test_ll_dispatch_full_decode_shape():
    """64 sources x 128 tokens, hidden 7168, 8x8 ranks, node-limited top-8:
    every one of the 65,536 messages (payload, scales, header) against the
    oracle's pack, with the used slots renumbered densely on both sides."""
    w = I.LL_DECODE
    say("LL dispatch full decode shape (all messages)")
    x = I.tokens_for(w)
    scores = I.scores_for(w)
    g = group_for(w)
    try:
        topk_d = torch.empty((w.num_tokens, 8), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        h = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h, x.cuda())
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, 8, 8, 4))
        want_cnt, want_slot, _ = oracle.layout_ll(topk, 64, 256, 128)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_COUNT), want_cnt)
        slot = get_map(h, A.EP_MAP_LL_SLOT)
        np.testing.assert_array_equal(slot, want_slot)
        buf = buffer(g, A.EP_BUF_LL_RECV)
        assert buf.shape == (256 * 64 * 128, 7408)
        used = np.unique(slot[slot >= 0])
        assert len(used) == w.num_tokens * 8
        dense = np.searchsorted(used, slot).astype(np.int32)     # slot -> its rank among the used slots
        want = oracle.pack_ll(I.bf16_bits(x), 128, 8, True, dense, len(used))
        got = host(buf[torch.from_numpy(used.astype(np.int64)).cuda()])
        np.testing.assert_array_equal(got, want)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


# ---------------------------------------------------------------------------
# A3 + A5 + A6: HT dispatch
# ---------------------------------------------------------------------------

def _ht_dispatch(w, x, scores, weights, in_fp8=False):
    S, T, K, H = w.num_src_ranks, w.tokens_per_rank, w.top_k, w.hidden
    fp8 = w.payload == "fp8"
    g = group_for(w)
    try:
        topk_d = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        h = ep.ep_create_handle(g, topk_d)
        counts = torch.zeros(w.num_experts, dtype=torch.int32, device="cuda")
        if in_fp8:
            q, sc = oracle.quantize_rows(I.bf16_bits(x))
            xq = torch.from_numpy(q).cuda().view(torch.float8_e4m3fn)
            ep.ep_dispatch(h, xq, scales=dev(sc), topk_weights=dev(weights), recv_counts=counts)
        else:
            ep.ep_dispatch(h, x.cuda(), topk_weights=dev(weights), recv_counts=counts)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, w.num_nodes, K, w.max_nodes))
        lay = oracle.layout_ht(topk, S, w.num_experts, w.num_nodes, w.ranks_per_node)
        np.testing.assert_array_equal(host(counts), lay["c2"])
        node_row = get_map(h, A.EP_MAP_HT_NODE_ROW)
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        np.testing.assert_array_equal(node_row, lay["node_row"])
        np.testing.assert_array_equal(row2, lay["row2"])
        rows1, rows2 = int(lay["c1"].sum()), int(lay["c2"].sum())
        meta = oracle.pack_ht(I.bf16_bits(x[:1]), topk, weights, T, w.num_nodes, fp8,
                              lay["node_row"], lay["row2"], rows1, rows2, with_payload=False)
        for name, which in [("meta1_tok", A.EP_BUF_HT_STAGE1_TOKEN), ("meta1_src", A.EP_BUF_HT_STAGE1_SRC),
                            ("meta1_topk", A.EP_BUF_HT_STAGE1_TOPK), ("meta1_w", A.EP_BUF_HT_STAGE1_WEIGHTS)]:
            np.testing.assert_array_equal(host(buffer(g, which)[:rows1]), meta[name], err_msg=name)
        for name, which in [("meta2_src", A.EP_BUF_HT_STAGE2_SRC), ("meta2_tok", A.EP_BUF_HT_STAGE2_TOKEN),
                            ("meta2_k", A.EP_BUF_HT_STAGE2_K)]:
            np.testing.assert_array_equal(host(buffer(g, which)[:rows2]), meta[name], err_msg=name)
        st1 = buffer(g, A.EP_BUF_HT_STAGE1)
        st2 = buffer(g, A.EP_BUF_HT_STAGE2)
        # every row of both stages against the oracle's own pack
        pk = oracle.pack_ht(I.bf16_bits(x), topk, weights, T, w.num_nodes, fp8,
                            lay["node_row"], lay["row2"], rows1, rows2)
        np.testing.assert_array_equal(host(st1[:rows1]), pk["stage1"], err_msg="stage 1")
        np.testing.assert_array_equal(host(st2[:rows2]), pk["stage2"], err_msg="stage 2")
        ep.ep_destroy_handle(h)
        return g, topk, lay
    except BaseException:
        ep.ep_destroy_group(g)
        raise


def test_ht_dispatch_midsize_all_rows():
    w = I.HT_PREFILL.with_(tokens_per_rank=700, hidden=1024, seed=31, num_src_ranks=3)
    say("HT dispatch S=3 T=700 H=1024 (all rows)")
    x = I.tokens_for(w)
    g, _, _ = _ht_dispatch(w, x, I.scores_for(w), I.normal_weights(w.num_tokens, 8, 31))
    ep.ep_destroy_group(g)


@pytest.mark.parametrize("payload", ["fp8", "bf16"])
def test_ht_dispatch_tiny(payload):
    w = I.TINY.with_(mode="ht", payload=payload)
    say(f"HT dispatch tiny {payload}")
    scores = I.scores_for(w)
    x = I.tokens_for(w)
    g, _, _ = _ht_dispatch(w, x, scores, I.normal_weights(w.num_tokens, w.top_k, 3))
    ep.ep_destroy_group(g)


def test_bf16_dispatch_full_hidden():
    """BF16 payload at hidden 7168: a token spans four waves of 8-value
    chunks, the last one ragged; HT rows and LL messages (header, zero tail)
    equal the oracle's."""
    w = I.HT_PREFILL.with_(tokens_per_rank=300, payload="bf16", seed=43)
    say("HT dispatch BF16 hidden 7168 (all rows)")
    g, _, _ = _ht_dispatch(w, I.tokens_for(w), I.scores_for(w), I.normal_weights(300, 8, 43))
    ep.ep_destroy_group(g)
    say("LL dispatch BF16 hidden 7168 (all tokens)")
    _ll_dispatch(2, 64, 256, 8, 7168, "bf16", 64, seed=45, N=8, G=8, M=4)


def test_ht_dispatch_prequantised_input():
    w = I.HT_PREFILL.with_(tokens_per_rank=300, hidden=512, seed=41)
    say("HT dispatch with FP8 input + scales")
    x = I.tokens_for(w)
    g, _, _ = _ht_dispatch(w, x, I.scores_for(w), I.normal_weights(300, 8, 41), in_fp8=True)
    ep.ep_destroy_group(g)


def test_ht_dispatch_full_prefill_shape():
    """The page's shape: 4096 tokens, hidden 7168, seed 0 scores: all 16,248
    stage-1 and 32,768 stage-2 rows and their metadata."""
    w = I.HT_PREFILL
    say("HT dispatch full prefill shape (all rows)")
    x = I.tokens_for(w)
    g, topk, lay = _ht_dispatch(w, x, I.scores_for(w), I.normal_weights(4096, 8, w.seed))
    try:
        assert lay["c1"].sum() == 16248 and lay["c2"].sum() == 32768
    finally:
        ep.ep_destroy_group(g)


# ---------------------------------------------------------------------------
# A7 combine
# ---------------------------------------------------------------------------

def test_combine_cfg_geometry_all_tokens():
    """4096 tokens x top-8 over 32768 bf16 rows of hidden 7168 (the combine
    workload); rows placed by the HT handle of the page's routing; every
    output element against the oracle."""
    w = I.COMBINE
    say("combine 4096x8x7168 (all tokens)")
    scores = I.scores_for(w)
    g = group_for(w)
    try:
        topk_d = torch.empty((4096, 8), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        h = ep.ep_create_handle(g, topk_d)
        Yt = I.normal_bf16(32768, 7168, w.seed)
        wts = I.normal_weights(4096, 8, w.seed)
        out = torch.empty((4096, 7168), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, Yt.cuda(), dev(wts), out)
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        want = oracle.combine(I.bf16_bits(Yt), wts, row2)
        np.testing.assert_array_equal(host(out), want)
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("n,K,H", [(1000, 8, 1024), (257, 2, 256), (64, 13, 512), (3, 32, 128)])
def test_combine_all_tokens(n, K, H):
    say(f"combine n={n} K={K} H={H}")
    topk = I.random_topk(n, 4 * K, K, seed=n)
    g = ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=4 * K, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n,
                           num_src_ranks=1, payload="bf16")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        Yt = I.normal_bf16(n * K, H, seed=n + 1)
        wts = I.normal_weights(n, K, seed=n + 2)
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, Yt.cuda(), dev(wts), out)
        want = oracle.combine(I.bf16_bits(Yt), wts, row2)
        got = host(out)
        np.testing.assert_array_equal(got, want)
        # the stated tolerance, for the record (implied by equality)
        g32 = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float()
        r32 = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float()
        assert torch.all((g32 - r32).abs() <= 1e-3 * torch.clamp(r32.abs(), min=1e-3))
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_combine_special_values():
    """Signed zeros, bf16 subnormals (fp32 denormals inside the fma chain: no
    flush to zero on either side), the smallest and largest normals, bf16
    rounding ties and sums that overflow to +inf, against the oracle bit for
    bit.  Large values are positive and weights non-negative, so no inf - inf
    (NaN inputs and results are outside the contract)."""
    n, K, H = 256, 8, 256
    say("combine special values")
    rng = np.random.default_rng(97)
    palette = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080,   # zeros, subnormals,
                        0x7F7F, 0x7F7E, 0x3F80, 0xBF80, 0x3F81, 0xBF81, 0x4000, 0x3F00],   # min normals, max,
                       np.uint16)                                                         # ±1, ±(1 + ulp), 2, 0.5
    Y = palette[rng.integers(0, len(palette), size=(n * K, H))]
    Y[::5] = I.bf16_bits(I.normal_bf16(len(Y[::5]), H, 98))                  # ordinary rows mixed in
    wpal = np.array([0.0, -0.0, 1.0, 0.5, 2.0, 1e-39, 1.5e-45, 0.75, 1.0 + 2.0**-23], np.float32)
    wts = wpal[rng.integers(0, len(wpal), size=(n, K))]
    wts[:, 0] = np.where(rng.random(n) < 0.5, wts[:, 0], 1.0)
    wts[rng.random((n, K)) < 0.02] = 3.0e38      # a few huge weights: overflow to +inf
    # no negative huge products: a huge weight only meets rows without negative values
    topk = I.random_topk(n, 4 * K, K, seed=99)
    g = ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=4 * K, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n,
                           num_src_ranks=1, payload="bf16")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        big = wts > 2.0
        for t, k in zip(*np.nonzero(big)):
            r = Y[row2[t, k]]
            neg = (r & 0x8000) != 0
            r[neg] = 0x8000                      # -0 instead of a negative value
            Y[row2[t, k]] = r
        want = oracle.combine(Y, wts, row2)
        wf = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
        assert not np.isnan(wf).any()
        assert np.isposinf(wf).any() and (want == 0x8000).any() and ((want & 0x7F80) == 0).any()
        Yt = torch.from_numpy(Y.view(np.int16)).view(torch.bfloat16).cuda()
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, Yt, dev(wts), out)
        np.testing.assert_array_equal(host(out), want)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_combine_invalid_and_out_of_range_rows():
    n, K, H = 40, 4, 256
    topk = I.random_topk(n, 16, K, seed=3)
    topk[5, 2] = 99                       # invalid: no row, contributes nothing
    g = ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=16, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n,
                           num_src_ranks=1, payload="bf16")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        assert ep.ep_get_device_error(g) == A.EP_DEVERR_BAD_INDEX
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        assert row2[5, 2] == -1
        rows = n * K - 1
        Yt = I.normal_bf16(rows, H, seed=4)
        wts = I.normal_weights(n, K, seed=5)
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        # give fewer rows than the handle addresses: the last row index is out of range
        short = Yt[: rows - 3].cuda()
        ep.ep_combine(h, short, dev(wts), out)
        assert ep.ep_get_device_error(g) == A.EP_DEVERR_ROW_RANGE
        loc = row2.copy()
        loc[loc >= rows - 3] = -1
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Yt[: rows - 3]), wts, loc))
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


# ---------------------------------------------------------------------------
# Round trips with the identity expert
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["ll", "ht"])
def test_tiny_identity_roundtrip_returns_input(mode):
    """Tiny workload: 128 tokens, hidden 256, 16 experts on 4 ranks, top-2, no
    node limit, BF16 payload, identity experts and softmax-normalised weights
    of the selected scores: the combine returns the input bit for bit."""
    w = I.TINY.with_(mode=mode)
    say(f"tiny identity round trip {mode}")
    scores = I.scores_for(w)
    x = I.tokens_for(w)
    g = group_for(w)
    try:
        topk_d = torch.empty((128, 2), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, 2, 2, 0))
        wts = I.weights_for(w, scores, topk)
        h = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h, x.cuda(), topk_weights=dev(wts))
        if mode == "ll":
            rows = buffer(g, A.EP_BUF_LL_RECV)
        else:
            rows = buffer(g, A.EP_BUF_HT_STAGE2)
        y = torch.empty((rows.shape[0], 256), dtype=torch.bfloat16, device="cuda")
        ep.ep_dequantize_rows(g, rows, y)
        out = torch.empty((128, 256), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, y, dev(wts), out)
        np.testing.assert_array_equal(host(out), I.bf16_bits(x))
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_fp8_roundtrip_large_skewed_all():
    """16384 tokens, Zipf(1.1) popularity, FP8 dispatch (HT), identity expert,
    BF16 combine: routing, maps, every stage-1 and stage-2 row, the identity
    expert's output and every output token equal the oracle's round trip bit
    for bit, and every token stays within the FP8 error bound of its input."""
    w = I.ROUND_TRIP
    say("FP8 round trip 16384 tokens (all rows and tokens)")
    scores = I.scores_for(w)
    x = I.tokens_for(w)
    g = group_for(w)
    try:
        topk_d = torch.empty((w.num_tokens, 8), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, 8, 8, 4))
        wts_all = I.weights_for(w, scores, topk)
        h = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h, x.cuda(), topk_weights=dev(wts_all))
        n_rows = ep.ep_handle_get_num_recv(h, -1)
        assert n_rows == w.num_tokens * 8
        lay = oracle.layout_ht(topk, 1, 256, 8, 8)
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), lay["node_row"])
        np.testing.assert_array_equal(row2, lay["row2"])
        rows1 = int(lay["c1"].sum())
        pk = oracle.pack_ht(I.bf16_bits(x), topk, wts_all, w.num_tokens, 8, True, lay["node_row"],
                            lay["row2"], rows1, n_rows)
        np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE1)[:rows1]), pk["stage1"])
        st2 = buffer(g, A.EP_BUF_HT_STAGE2)[:n_rows]
        np.testing.assert_array_equal(host(st2), pk["stage2"])
        y_or = oracle.dequant_rows(pk["stage2"], 7168, True)
        del pk
        y = torch.empty((n_rows, 7168), dtype=torch.bfloat16, device="cuda")
        ep.ep_dequantize_rows(g, st2, y)
        np.testing.assert_array_equal(host(y), y_or)
        out = torch.empty((w.num_tokens, 7168), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, y, dev(wts_all), out)
        del y
        want = oracle.combine(y_or, wts_all, row2)
        del y_or
        got = host(out)
        np.testing.assert_array_equal(got, want)
        assert ep.ep_get_device_error(g) == 0
        # the round trip returns each token within the FP8 error bound
        xf = x.float().numpy()
        gf = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
        amax = np.abs(xf).reshape(w.num_tokens, -1, 128).max(axis=2).repeat(128, axis=1)
        assert np.all(np.abs(gf - xf) <= 2.0**-4 * np.abs(xf) + 2.0**-8 * np.abs(xf) + amax * 2.0**-9 + 1e-6)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ht_two_live_handles():
    """Two live HT handles on one group: the second dispatch overwrites the
    group's stage rows with its own, and the first handle keeps its maps, so
    each handle's combine equals the oracle's for its own routing."""
    w = I.HT_PREFILL.with_(tokens_per_rank=300, hidden=512, seed=51)
    say("HT two live handles")
    g = group_for(w)
    try:
        xs, tks, hs, lays = [], [], [], []
        for j in range(2):
            scores = I.scores_for(w.with_(seed=51 + j))
            topk_d = torch.empty((300, 8), dtype=torch.int32, device="cuda")
            ep.ep_route(g, dev(scores), topk_d)
            tks.append(host(topk_d))
            hs.append(ep.ep_create_handle(g, topk_d))
            lays.append(oracle.layout_ht(tks[j], 1, 256, 8, 8))
            xs.append(I.normal_bf16(300, 512, 52 + j))
        assert not np.array_equal(tks[0], tks[1])
        wts = I.normal_weights(300, 8, 53)
        for j in range(2):
            ep.ep_dispatch(hs[j], xs[j].cuda(), topk_weights=dev(wts))
        # the group's stage-2 rows are the second dispatch's
        rows2 = int(lays[1]["c2"].sum())
        pk = oracle.pack_ht(I.bf16_bits(xs[1]), tks[1], wts, 300, 8, True, lays[1]["node_row"],
                            lays[1]["row2"], int(lays[1]["c1"].sum()), rows2)
        np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:rows2]), pk["stage2"])
        for j in (0, 1):
            np.testing.assert_array_equal(get_map(hs[j], A.EP_MAP_HT_ROW), lays[j]["row2"])
            Y = I.normal_bf16(300 * 8, 512, 54 + j)
            out = torch.empty((300, 512), dtype=torch.bfloat16, device="cuda")
            ep.ep_combine(hs[j], Y.cuda(), dev(wts), out)
            np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, lays[j]["row2"]))
        assert ep.ep_get_device_error(g) == 0
        for h in hs:
            ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
