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
