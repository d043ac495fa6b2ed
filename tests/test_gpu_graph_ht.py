"""The HT step captured once in a HIP graph and replayed, GPU vs oracle.

route -> handle -> FP8 dispatch (stage-1 and stage-2 rows, per-expert
receive counts) -> identity expert on the stage-2 rows -> combine, captured
once and replayed on new inputs, with unrelated eager work and
synchronisation between the replays.  Every replay must reproduce the
oracle: routing, maps, counts, both stages' rows and the combined output.
Counts and maps are written by kernels on every replay (nothing is cleared
with a memset), so the captured step is self-contained.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, buffer, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu

S, T, E, N, G, K, H, M = 2, 100, 64, 4, 2, 4, 512, 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _inputs(seed):
    return (I.uniform_scores(S * T, E, seed).astype(np.float32), I.normal_bf16(S * T, H, seed + 1),
            I.normal_weights(S * T, K, seed + 2))


def _want(scores, x, w):
    topk = oracle.route(scores, N, K, M)
    lay = oracle.layout_ht(topk, S, E, N, G)
    rows1, rows2 = int(lay["c1"].sum()), int(lay["c2"].sum())
    pk = oracle.pack_ht(I.bf16_bits(x), topk, w, T, N, True, lay["node_row"], lay["row2"], rows1, rows2)
    y = oracle.dequant_rows(pk["stage2"], H, True)
    return dict(topk=topk, lay=lay, rows1=rows1, rows2=rows2, stage1=pk["stage1"], stage2=pk["stage2"],
                out=oracle.combine(y, w, lay["row2"]))


def test_graph_capture_of_ht_step():
    say(f"graph capture of the HT step: S={S} T={T} E={E} N={N}x{G} K={K} M={M} H={H}")
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T, num_src_ranks=S,
                           payload="fp8")
    try:
        sc_d = torch.empty((S * T, E), dtype=torch.float32, device="cuda")
        x_d = torch.empty((S * T, H), dtype=torch.bfloat16, device="cuda")
        w_d = torch.empty((S * T, K), dtype=torch.float32, device="cuda")
        topk_d = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        y_d = torch.empty((S * T * K, H), dtype=torch.bfloat16, device="cuda")
        out_d = torch.empty((S * T, H), dtype=torch.bfloat16, device="cuda")
        cnt_d = torch.empty(E, dtype=torch.int32, device="cuda")
        st1, st2 = buffer(g, A.EP_BUF_HT_STAGE1), buffer(g, A.EP_BUF_HT_STAGE2)

        def load(seed):
            scores, x, w = _inputs(seed)
            sc_d.copy_(torch.from_numpy(scores))
            x_d.copy_(x)
            w_d.copy_(torch.from_numpy(w))
            torch.cuda.synchronize()
            return scores, x, w

        load(10)
        # one eager step first, so that nothing but library launches runs while capturing
        ep.ep_route(g, sc_d, topk_d)
        h0 = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h0, x_d, topk_weights=w_d)
        ep.ep_destroy_handle(h0)
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            ep.ep_route(g, sc_d, topk_d)
            h = ep.ep_create_handle(g, topk_d)
            ep.ep_dispatch(h, x_d, topk_weights=w_d, recv_counts=cnt_d)
            ep.ep_dequantize_rows(g, st2, y_d)
            ep.ep_combine(h, y_d, w_d, out_d)
        torch.cuda.synchronize()
        for rep, seed in enumerate([10, 20, 30, 20]):
            scores, x, w = load(seed)
            scratch = torch.ones(4096, device="cuda").cumsum(0)   # unrelated eager work
            out_d.zero_()
            cnt_d.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert float(scratch[-1]) == 4096.0
            want = _want(scores, x, w)
            lay = want["lay"]
            np.testing.assert_array_equal(host(topk_d), want["topk"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay["row2"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_NODE_ROW), lay["node_row"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(host(cnt_d), lay["c2"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(host(st1[:want["rows1"]]), want["stage1"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(host(st2[:want["rows2"]]), want["stage2"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(host(out_d), want["out"], err_msg=f"replay {rep}")
            assert ep.ep_get_device_error(g) == 0
            say(f"  replay {rep} ok")
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
