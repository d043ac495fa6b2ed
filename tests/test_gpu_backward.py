"""Backward pass with reuse of the forward handle, GPU vs oracle.

"NCCL EP paper notes" (usage, HT training example): the forward pass keeps
one handle per layer; the backward pass walks the layers in reverse, sends
the loss gradient to the experts with the layer's handle, runs the experts'
backward and brings their gradients back, then destroys the handle.
ep_combine_backward and ep_dispatch_backward are the adjoints of the
combine and the dispatch over the handle's row map.  Row gradients and token
gradients are compared bit for bit with the oracle; weight gradients are fp32
dot products of H terms and must lie within the fp32 dot-product error bound
|got - exact| <= 2 * H * 2^-24 * sum |g * y| of the exact (fp64) value.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, group_for, host, need_gpu, say

pytestmark = pytest.mark.gpu

CANARY = 0x7E5A   # a bf16 bit pattern no gradient here produces


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _check_dw(got, want, absum, H, msg=""):
    bound = 2.0 * H * 2.0 ** -24 * absum + 1e-30
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= bound), f"{msg} weight gradient off by {err.max():.3e} (bound {bound.max():.3e})"


def _backward_case(loc, rows, H, fp_seed):
    """Random output gradients, expert outputs, weights and row gradients."""
    n, K = loc.shape
    rng = np.random.default_rng(fp_seed)
    gb = I.bf16_bits(I.normal_bf16(n, H, fp_seed))
    Yb = I.bf16_bits(I.normal_bf16(rows, H, fp_seed + 1))
    w = rng.random((n, K)).astype(np.float32) + 0.05
    dRb = I.bf16_bits(I.normal_bf16(rows, H, fp_seed + 2))
    return gb, Yb, w, dRb


@pytest.mark.parametrize("mode", ["ht", "ll"])
def test_backward_adjoints_match_oracle(mode):
    S, T, H = 2, 300, 1024
    w_ = I.HT_PREFILL.with_(mode=mode, num_src_ranks=S, tokens_per_rank=T, hidden=H, seed=61,
                            max_tokens_per_rank=T + 20)
    say(f"backward adjoints {mode}: S={S} T={T} H={H}")
    g = group_for(w_, max_handles=2)
    try:
        scores = I.scores_for(w_)
        topk_d = torch.empty((S * T, 8), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        h = ep.ep_create_handle(g, topk_d)
        topk = host(topk_d)
        if mode == "ht":
            loc = oracle.layout_ht(topk, S, 256, 8, 8)["row2"]
            rows = S * (T + 20) * 8
            shape = (rows, H)
        else:
            loc = oracle.layout_ll(topk, S, 256, T + 20)[1]
            rows = 256 * S * (T + 20)
            shape = (256, S * (T + 20), H)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW if mode == "ht" else A.EP_MAP_LL_SLOT), loc)
        gb, Yb, w, dRb = _backward_case(loc, rows, H, 70)
        dY = torch.full(shape, 0, dtype=torch.int16, device="cuda").fill_(CANARY).view(torch.bfloat16)
        dw = torch.full((S * T, 8), 7.0, dtype=torch.float32, device="cuda")
        ep.ep_combine_backward(h, _bf16(gb), dev(w), dY, expert_out=_bf16(Yb).view(shape), grad_weights=dw)
        want_dY, want_dw, absum = oracle.combine_backward(gb, w, loc, rows, Yb)
        got_dY = host(dY.view(rows, H))
        used = np.unique(loc[loc >= 0])
        np.testing.assert_array_equal(got_dY[used], want_dY[used])
        untouched = np.setdiff1d(np.arange(rows), used)
        assert np.all(got_dY[untouched] == CANARY), "a row no entry points at was written"
        _check_dw(host(dw), want_dw, absum, H, mode)
        # without expert outputs: row gradients only
        dY2 = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        ep.ep_combine_backward(h, _bf16(gb), dev(w), dY2)
        np.testing.assert_array_equal(host(dY2.view(rows, H))[used], want_dY[used])
        # dispatch adjoint
        gx = torch.empty((S * T, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_dispatch_backward(h, _bf16(dRb).view(shape), gx)
        np.testing.assert_array_equal(host(gx), oracle.dispatch_backward(dRb, loc))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_backward_invalid_entries_and_errors():
    """Caller-supplied top-k with a repeated expert and an out-of-range one:
    those entries write no row and get a zero weight gradient; argument and
    call-order errors are rejected."""
    S, T, H, K = 1, 70, 512, 4
    g = ep.ep_create_group(mode="ht", num_nodes=2, ranks_per_node=2, num_experts=16, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=T, num_src_ranks=S)
    try:
        rng = np.random.default_rng(9)
        topk = np.stack([rng.permutation(16)[:K] for _ in range(T)]).astype(np.int32)
        topk[3, 2] = topk[3, 0]      # repeat
        topk[10, 1] = 99             # out of range
        h = ep.ep_create_handle(g, dev(topk))
        lay = oracle.layout_ht(topk, S, 16, 2, 2)
        loc = lay["row2"]
        assert loc[3, 2] == -1 and loc[10, 1] == -1
        rows = T * K
        gb, Yb, w, dRb = _backward_case(loc, rows, H, 90)
        dY = torch.zeros((rows, H), dtype=torch.bfloat16, device="cuda")
        dw = torch.full((T, K), 5.0, dtype=torch.float32, device="cuda")
        ep.ep_combine_backward(h, _bf16(gb), dev(w), dY, expert_out=_bf16(Yb), grad_weights=dw)
        want_dY, want_dw, absum = oracle.combine_backward(gb, w, loc, rows, Yb)
        used = np.unique(loc[loc >= 0])
        np.testing.assert_array_equal(host(dY)[used], want_dY[used])
        got_dw = host(dw)
        assert got_dw[3, 2] == 0.0 and got_dw[10, 1] == 0.0
        _check_dw(got_dw, want_dw, absum, H)
        gx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_dispatch_backward(h, _bf16(dRb), gx)
        np.testing.assert_array_equal(host(gx), oracle.dispatch_backward(dRb, loc))
        err = ep.ep_get_device_error(g)
        assert err & A.EP_DEVERR_DUP_INDEX and err & A.EP_DEVERR_BAD_INDEX
        # grad_weights without expert outputs, wrong shapes
        for kw in [dict(grad_weights=dw), dict(expert_out=_bf16(Yb)[:, :256], grad_weights=dw)]:
            with pytest.raises(ep.EpError) as ei:
                ep.ep_combine_backward(h, _bf16(gb), dev(w), dY, **kw)
            assert ei.value.status == A.EP_ERR_INVALID_ARGUMENT
        with pytest.raises(ep.EpError):
            ep.ep_dispatch_backward(h, _bf16(dRb), gx[:5])
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_training_reuses_handles_across_layers():
    """The page's training loop with three layers: forward (route, handle,
    FP8 dispatch, identity expert, combine; the output feeds the next
    layer), then backward in reverse with each layer's handle (combine
    adjoint, identity expert backward, dispatch adjoint), destroying the
    handle after its layer.  Every gradient equals the oracle's chain."""
    L, T, H = 3, 256, 1024
    wl = I.HT_PREFILL.with_(tokens_per_rank=T, hidden=H, seed=0)
    say(f"training reuse of handles: {L} layers, {T} tokens, hidden {H}")
    g = group_for(wl, max_handles=L)
    try:
        x0 = I.normal_bf16(T, H, 400)
        xs_b = [I.bf16_bits(x0)]
        handles, weights, Ys, locs = [], [], [], []
        x_d = x0.cuda()
        for l in range(L):
            scores = I.page_scores(T, 256, 500 + l).astype(np.float32)
            topk_d = torch.empty((T, 8), dtype=torch.int32, device="cuda")
            ep.ep_route(g, dev(scores), topk_d)
            h = ep.ep_create_handle(g, topk_d)
            wts = I.normal_weights(T, 8, 600 + l)
            ep.ep_dispatch(h, x_d, topk_weights=dev(wts))
            rows = T * 8
            st2 = ep.ep_get_buffer(g, A.EP_BUF_HT_STAGE2)[:rows]
            Y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
            ep.ep_dequantize_rows(g, st2, Y)
            out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            ep.ep_combine(h, Y, dev(wts), out)
            # oracle forward of this layer
            topk = oracle.route(scores, 8, 8, 4)
            np.testing.assert_array_equal(host(topk_d), topk)
            loc = oracle.layout_ht(topk, 1, 256, 8, 8)["row2"]
            img = oracle.token_rows(xs_b[-1], True)
            Yo = np.zeros((rows, H), np.uint16)
            for t in range(T):
                for k in range(8):
                    Yo[loc[t, k]] = oracle.dequant_rows(img[t:t + 1], H, True)[0]
            np.testing.assert_array_equal(host(Y), Yo, err_msg=f"layer {l} expert rows")
            xs_b.append(oracle.combine(Yo, wts, loc))
            np.testing.assert_array_equal(host(out), xs_b[-1], err_msg=f"layer {l} forward")
            handles.append(h); weights.append(wts); Ys.append(Yo); locs.append(loc)
            x_d = out
        # backward
        grad_b = I.bf16_bits(I.normal_bf16(T, H, 700))
        grad_d = _bf16(grad_b)
        for l in reversed(range(L)):
            rows = T * 8
            dY = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
            dw = torch.empty((T, 8), dtype=torch.float32, device="cuda")
            ep.ep_combine_backward(handles[l], grad_d, dev(weights[l]), dY, expert_out=_bf16(Ys[l]),
                                   grad_weights=dw)
            want_dY, want_dw, absum = oracle.combine_backward(grad_b, weights[l], locs[l], rows, Ys[l])
            np.testing.assert_array_equal(host(dY), want_dY, err_msg=f"layer {l} row gradients")
            _check_dw(host(dw), want_dw, absum, H, f"layer {l}")
            gx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            ep.ep_dispatch_backward(handles[l], dY, gx)      # identity expert: dX rows = dY
            grad_b = oracle.dispatch_backward(want_dY, locs[l])
            np.testing.assert_array_equal(host(gx), grad_b, err_msg=f"layer {l} token gradients")
            grad_d = gx
            ep.ep_destroy_handle(handles[l])
        assert ep.ep_get_device_error(g) == 0
    finally:
        ep.ep_destroy_group(g)
