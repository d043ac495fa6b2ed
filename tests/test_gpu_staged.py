"""LL staged execution with double-buffered receive partitions, and HIP-graph
capture of the LL path.

"NCCL EP paper notes" (API section and the send_only / double-buffer pipeline
section): with send_only the dispatch and the combine enqueue their send
stage only and ncclEpComplete runs the receive stage; LL keeps two internal
buffers so that one micro-batch's dispatch overlaps another's combine.  The
tests run the page's two-micro-batch decode pipeline:

    dispatch(0, send_only); dispatch(1, send_only)
    complete(0); expert(0); combine(0, send_only)
    complete(1); expert(1); combine(1, send_only)
    complete(0); complete(1)

with the identity expert, and require the oracle's bytes and outputs, each
micro-batch in its own receive buffer, the un-staged calls' results, and, for
a captured graph of the whole pipeline, the oracle's results on every replay.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, host, need_gpu, say

pytestmark = pytest.mark.gpu

S, T, E, K, N, G, M, H, SLOTS = 4, 48, 32, 4, 4, 2, 2, 1024, 64
CFG = dict(mode="ll", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K, max_nodes_per_token=M,
           hidden=H, max_tokens_per_rank=SLOTS, num_src_ranks=S, max_handles=6)
ROWS = E * S * SLOTS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _mb(seed):
    """Inputs of one micro-batch: router scores, tokens, combine weights."""
    return (I.uniform_scores(S * T, E, seed).astype(np.float32), I.normal_bf16(S * T, H, seed + 1),
            I.normal_weights(S * T, K, seed + 2))


def _want(mb, fp8):
    scores, x, w = mb
    topk = oracle.route(scores, N, K, M)
    counts, slot, err = oracle.layout_ll(topk, S, E, SLOTS)
    assert err == 0
    msgs = oracle.pack_ll(I.bf16_bits(x), T, K, fp8, slot, ROWS)
    y = oracle.dequant_rows(msgs, H, fp8)
    return dict(topk=topk, counts=counts, slot=slot, msgs=msgs, out=oracle.combine(y, w, slot))


def _check_msgs(buf, want):
    used = np.unique(want["slot"][want["slot"] >= 0])
    got = host(buf[torch.from_numpy(used.astype(np.int64)).cuda()])
    np.testing.assert_array_equal(got, want["msgs"][used])


def _tensors():
    topk = [torch.empty((S * T, K), dtype=torch.int32, device="cuda") for _ in range(2)]
    # micro-batch 0 asks for per-(expert, source) counts, 1 for tokens per expert
    cnt = [torch.zeros((E, S), dtype=torch.int32, device="cuda"), torch.zeros(E, dtype=torch.int32, device="cuda")]
    y = [torch.empty((ROWS, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    out = [torch.empty((S * T, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    return topk, cnt, y, out


def _check_counts(cnt, want):
    np.testing.assert_array_equal(host(cnt[0]), want[0]["counts"])
    np.testing.assert_array_equal(host(cnt[1]), want[1]["counts"].sum(axis=1))


@pytest.mark.parametrize("payload", ["fp8", "bf16"])
def test_staged_pipeline_two_micro_batches(payload):
    say(f"LL staged pipeline, two micro-batches, {payload}")
    fp8 = payload == "fp8"
    mbs = [_mb(101), _mb(202)]
    want = [_want(m, fp8) for m in mbs]
    g = ep.ep_create_group(payload=payload, **CFG)
    try:
        topk, cnt, y, out = _tensors()
        x = [mb[1].cuda() for mb in mbs]
        w = [dev(mb[2]) for mb in mbs]
        h = []
        for b in range(2):
            ep.ep_route(g, dev(mbs[b][0]), topk[b])
            h.append(ep.ep_create_handle(g, topk[b]))
            ep.ep_dispatch(h[b], x[b], recv_counts=cnt[b], send_only=True)
        torch.cuda.synchronize()
        assert not host(cnt[0]).any() and not host(cnt[1]).any(), "receive stage ran before ep_complete"
        buf = [ep.ep_handle_get_buffer(h[b], A.EP_BUF_LL_RECV) for b in range(2)]
        assert buf[0].data_ptr() == ep.ep_get_buffer(g, A.EP_BUF_LL_RECV).data_ptr()
        assert buf[1].data_ptr() != buf[0].data_ptr(), "micro-batches share a receive buffer"
        for b in range(2):
            ep.ep_complete(h[b])
            ep.ep_dequantize_rows(g, buf[b], y[b])
            ep.ep_combine(h[b], y[b], w[b], out[b], send_only=True)
        for b in range(2):
            ep.ep_complete(h[b])
        for b in range(2):
            np.testing.assert_array_equal(host(topk[b]), want[b]["topk"])
            _check_msgs(buf[b], want[b])
            np.testing.assert_array_equal(host(out[b]), want[b]["out"], err_msg=f"micro-batch {b}")
        _check_counts(cnt, want)

        # A third dispatch takes the first buffer again and leaves the second alone.
        keep = host(buf[1]).copy()
        h2 = ep.ep_create_handle(g, topk[0])
        ep.ep_dispatch(h2, x[0])
        assert ep.ep_handle_get_buffer(h2, A.EP_BUF_LL_RECV).data_ptr() == buf[0].data_ptr()
        _check_msgs(buf[0], want[0])
        np.testing.assert_array_equal(host(buf[1]), keep)
        for hh in h + [h2]:
            ep.ep_destroy_handle(hh)
        assert ep.ep_get_device_error(g) == 0
    finally:
        ep.ep_destroy_group(g)

    # The same micro-batches through un-staged calls on one receive buffer.
    g1 = ep.ep_create_group(payload=payload, ll_buffers=1, **CFG)
    try:
        topk, cnt, y, out = _tensors()
        for b in range(2):
            ep.ep_route(g1, dev(mbs[b][0]), topk[b])
            hb = ep.ep_create_handle(g1, topk[b])
            ep.ep_dispatch(hb, mbs[b][1].cuda(), recv_counts=cnt[b])
            ep.ep_dequantize_rows(g1, ep.ep_handle_get_buffer(hb, A.EP_BUF_LL_RECV), y[b])
            ep.ep_combine(hb, y[b], dev(mbs[b][2]), out[b])
            np.testing.assert_array_equal(host(out[b]), want[b]["out"], err_msg=f"un-staged {b}")
            ep.ep_destroy_handle(hb)
        _check_counts(cnt, want)
    finally:
        ep.ep_destroy_group(g1)


def test_staged_call_order_errors():
    say("staged-mode call-order errors")
    g = ep.ep_create_group(payload="fp8", **CFG)
    try:
        scores, x, w = _mb(7)
        topk = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk)
        h = ep.ep_create_handle(g, topk)
        y = torch.zeros((ROWS, H), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((S * T, H), dtype=torch.bfloat16, device="cuda")
        codes = {}
        for name, call in [
            ("buffer before dispatch", lambda: ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)),
            ("complete with nothing staged", lambda: ep.ep_complete(h)),
        ]:
            with pytest.raises(ep.EpError) as ei:
                call()
            codes[name] = ei.value.status
        ep.ep_dispatch(h, x.cuda(), send_only=True)
        for name, call in [
            ("dispatch while staged", lambda: ep.ep_dispatch(h, x.cuda())),
            ("combine while dispatch staged", lambda: ep.ep_combine(h, y, dev(w), out)),
        ]:
            with pytest.raises(ep.EpError) as ei:
                call()
            codes[name] = ei.value.status
        ep.ep_complete(h)
        ep.ep_combine(h, y, dev(w), out, send_only=True)
        with pytest.raises(ep.EpError) as ei:
            ep.ep_combine(h, y, dev(w), out, send_only=True)
        codes["combine while combine staged"] = ei.value.status
        ep.ep_complete(h)
        assert set(codes.values()) == {A.EP_ERR_INVALID_ARGUMENT}, codes
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
    # HT has no staged mode
    gh = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                            max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T, num_src_ranks=S)
    try:
        topk = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        ep.ep_route(gh, dev(scores), topk)
        h = ep.ep_create_handle(gh, topk)
        with pytest.raises(ep.EpError) as ei:
            ep.ep_dispatch(h, x.cuda(), send_only=True)
        assert ei.value.status == A.EP_ERR_UNSUPPORTED
        ep.ep_dispatch(h, x.cuda())
        y2 = torch.zeros((S * T * K, H), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(ep.EpError) as ei:
            ep.ep_combine(h, y2, dev(w), out, send_only=True)
        assert ei.value.status == A.EP_ERR_UNSUPPORTED
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(gh)


def test_graph_capture_of_staged_pipeline():
    """route -> handle -> dispatch(send_only) -> complete -> expert ->
    combine(send_only) -> complete for two micro-batches, captured once and
    replayed on new inputs, with eager work and synchronisation between the
    replays; every replay must give the oracle's results."""
    say("graph capture of the staged LL pipeline")
    g = ep.ep_create_group(payload="fp8", **CFG)
    handles = []
    try:
        sc_d = [torch.empty((S * T, E), dtype=torch.float32, device="cuda") for _ in range(2)]
        x_d = [torch.empty((S * T, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        w_d = [torch.empty((S * T, K), dtype=torch.float32, device="cuda") for _ in range(2)]
        topk, cnt, y, out = _tensors()

        def load(seed):
            mbs = [_mb(seed), _mb(seed + 50)]
            for b in range(2):
                sc_d[b].copy_(dev(mbs[b][0]))
                x_d[b].copy_(mbs[b][1].cuda())
                w_d[b].copy_(dev(mbs[b][2]))
            torch.cuda.synchronize()
            return mbs

        load(300)
        # The receive-buffer views, taken from two dispatches before the
        # capture (the buffers alternate, so the captured micro-batches get
        # the same two): nothing but library launches runs while capturing.
        bufs = []
        for b in range(2):
            ep.ep_route(g, sc_d[b], topk[b])
            hb = ep.ep_create_handle(g, topk[b])
            ep.ep_dispatch(hb, x_d[b])
            bufs.append(ep.ep_handle_get_buffer(hb, A.EP_BUF_LL_RECV))
            ep.ep_destroy_handle(hb)
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for b in range(2):
                ep.ep_route(g, sc_d[b], topk[b])
                handles.append(ep.ep_create_handle(g, topk[b]))
                ep.ep_dispatch(handles[b], x_d[b], recv_counts=cnt[b], send_only=True)
            for b in range(2):
                ep.ep_complete(handles[b])
                ep.ep_dequantize_rows(g, bufs[b], y[b])
                ep.ep_combine(handles[b], y[b], w_d[b], out[b], send_only=True)
            for b in range(2):
                ep.ep_complete(handles[b])
        torch.cuda.synchronize()
        for b in range(2):
            assert ep.ep_handle_get_buffer(handles[b], A.EP_BUF_LL_RECV).data_ptr() == bufs[b].data_ptr()
        for rep, seed in enumerate([300, 400, 500, 400]):
            mbs = load(seed)
            scratch = torch.ones(4096, device="cuda").cumsum(0)   # unrelated eager work
            for b in range(2):
                out[b].zero_()
                cnt[b].zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert float(scratch[-1]) == 4096.0
            want = [_want(m, True) for m in mbs]
            for b in range(2):
                np.testing.assert_array_equal(host(topk[b]), want[b]["topk"], err_msg=f"replay {rep}")
                np.testing.assert_array_equal(host(out[b]), want[b]["out"], err_msg=f"replay {rep} mb {b}")
            _check_counts(cnt, want)
            say(f"  replay {rep} ok")
        del graph
        assert ep.ep_get_device_error(g) == 0
    finally:
        torch.cuda.synchronize()
        for hh in handles:
            ep.ep_destroy_handle(hh)
        ep.ep_destroy_group(g)
