"""ep_quantize, the FP8 quantisation as a call of its own, GPU vs oracle.

"NVSHMEM and DeepEP: GPU-initiated communication": FP8 dispatch with one
fp32 scale per 128 elements.  ep_quantize must give exactly the oracle's
codes and scales (scale = amax/448, nearest-even saturating E4M3 of x/scale),
and a dispatch of its output as pre-quantised tokens must write exactly the
rows the dispatch writes when it quantises the BF16 tokens itself.
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


def _group(mode, H, T=300, S=1, E=64, K=4, N=4, G=2):
    return ep.ep_create_group(mode=mode, num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                              max_nodes_per_token=0, hidden=H, max_tokens_per_rank=T, num_src_ranks=S,
                              payload="fp8")


def _tokens(n, H, seed):
    x = I.normal_bf16(n, H, seed)
    x[0, :128] = 0.0                     # an all-zero block
    x[1, 128:256] = -0.0                 # a block of -0
    x[2, :] *= 1e30                      # large magnitudes
    x[3, :] *= 1e-38                     # subnormal scales
    return x


@pytest.mark.parametrize("H", [128, 1152, 7168])
def test_quantize_equals_oracle(H):
    n = 300
    say(f"ep_quantize: n={n} H={H}")
    x = _tokens(n, H, 60 + H)
    g = _group("ht", H)
    try:
        q = torch.empty((n, H), dtype=torch.float8_e4m3fn, device="cuda")
        sc = torch.empty((n, H // 128), dtype=torch.float32, device="cuda")
        ep.ep_quantize(g, x.cuda(), q, sc)
        want_q, want_sc = oracle.quantize_rows(I.bf16_bits(x))
        np.testing.assert_array_equal(host(q.view(torch.uint8)), want_q)
        np.testing.assert_array_equal(host(sc).view(np.uint32), want_sc.view(np.uint32))
    finally:
        ep.ep_destroy_group(g)


def test_quantize_strided_rows():
    n, H = 70, 1024
    say("ep_quantize: strided input and output rows")
    x = _tokens(n, H, 61)
    g = _group("ht", H)
    try:
        xs = torch.zeros((n, H + 256), dtype=torch.bfloat16, device="cuda")
        xs[:, :H] = x.cuda()
        qs = torch.full((n, H + 64), 0x55, dtype=torch.uint8, device="cuda")
        ss = torch.full((n, H // 128 + 3), -1.0, dtype=torch.float32, device="cuda")
        ep.ep_quantize(g, xs[:, :H], qs[:, :H].view(torch.float8_e4m3fn), ss[:, :H // 128])
        want_q, want_sc = oracle.quantize_rows(I.bf16_bits(x))
        qh, sh = host(qs), host(ss)
        np.testing.assert_array_equal(qh[:, :H], want_q)
        np.testing.assert_array_equal(sh[:, :H // 128].view(np.uint32), want_sc.view(np.uint32))
        assert (qh[:, H:] == 0x55).all() and (sh[:, H // 128:] == -1.0).all()   # nothing past the rows
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("mode", ["ht", "ll"])
def test_dispatch_of_quantized_tokens_equals_fused_dispatch(mode):
    S, T, E, K, H = 2, 150, 64, 4, 7168
    n = S * T
    say(f"{mode.upper()} dispatch: ep_quantize + FP8 input vs BF16 input")
    x = _tokens(n, H, 62)
    topk = I.random_topk(n, E, K, seed=63)
    w = I.normal_weights(n, K, 64)
    rows = {}
    for form in ("fused", "split"):
        g = _group(mode, H, T=T, S=S, E=E, K=K)
        try:
            h = ep.ep_create_handle(g, dev(topk))
            if form == "fused":
                ep.ep_dispatch(h, x.cuda(), topk_weights=dev(w) if mode == "ht" else None)
            else:
                q = torch.empty((n, H), dtype=torch.float8_e4m3fn, device="cuda")
                sc = torch.empty((n, H // 128), dtype=torch.float32, device="cuda")
                ep.ep_quantize(g, x.cuda(), q, sc)
                ep.ep_dispatch(h, q, scales=sc, topk_weights=dev(w) if mode == "ht" else None)
            if mode == "ht":
                r2 = get_map(h, A.EP_MAP_HT_ROW)
                nr = get_map(h, A.EP_MAP_HT_NODE_ROW)
                n1, n2 = int((nr >= 0).sum()), int((r2 >= 0).sum())
                rows[form] = (host(buffer(g, A.EP_BUF_HT_STAGE1)[:n1]), host(buffer(g, A.EP_BUF_HT_STAGE2)[:n2]))
            else:
                slot = get_map(h, A.EP_MAP_LL_SLOT)
                used = torch.from_numpy(np.sort(slot[slot >= 0]).astype(np.int64)).cuda()
                rows[form] = (host(buffer(g, A.EP_BUF_LL_RECV)[used]),)
            assert ep.ep_get_device_error(g) == 0
            ep.ep_destroy_handle(h)
        finally:
            ep.ep_destroy_group(g)
    for a, b in zip(rows["fused"], rows["split"]):
        np.testing.assert_array_equal(a, b)
    if mode == "ht":
        # and both equal the oracle's stage-2 rows
        lay = oracle.layout_ht(topk, S, E, 4, 2)
        pk = oracle.pack_ht(I.bf16_bits(x), topk, w, T, 4, True, lay["node_row"], lay["row2"],
                            int(lay["c1"].sum()), int(lay["c2"].sum()))
        np.testing.assert_array_equal(rows["split"][1], pk["stage2"])


def test_quantize_rejects_bf16_payload_groups():
    g = ep.ep_create_group(mode="ht", num_nodes=2, ranks_per_node=2, num_experts=16, top_k=2,
                           max_nodes_per_token=0, hidden=256, max_tokens_per_rank=8, num_src_ranks=1,
                           payload="bf16")
    try:
        x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
        q = torch.empty((8, 256), dtype=torch.float8_e4m3fn, device="cuda")
        sc = torch.empty((8, 2), dtype=torch.float32, device="cuda")
        with pytest.raises(ep.EpError) as ei:
            ep.ep_quantize(g, x, q, sc)
        assert ei.value.status == A.EP_ERR_INVALID_ARGUMENT
    finally:
        ep.ep_destroy_group(g)
