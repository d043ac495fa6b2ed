"""Group options that change how the path runs but not what it computes,
GPU vs oracle:
  * the CU cap (num_cus): dispatch, combine and the adjoints launch fewer
    workgroups and loop over the work (caps from 1 to 17 CUs);
  * allocator hooks (alloc_fn / free_fn): the group's memory comes from the
    caller, the device is first touched by the first operation, and every
    block is handed back."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, buffer, dev, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("mode", ["ht", "ll"])
@pytest.mark.parametrize("num_cus", [1, 3, 17])
def test_capped_launches_equal_the_oracle(mode, num_cus):
    N, G, E, K, M, S, T, H = 4, 2, 64, 6, 2, 3, 300, 1024
    n, ll = S * T, mode == "ll"
    say(f"CU cap {num_cus} {mode}")
    scores = I.uniform_scores(n, E, seed=21000 + num_cus).astype(np.float32)
    x = I.normal_bf16(n, H, 21100 + num_cus)
    wts = I.normal_weights(n, K, 21200 + num_cus)
    g = ep.ep_create_group(mode=mode, num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T, num_src_ranks=S,
                           payload="fp8", num_cus=num_cus)
    try:
        topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        topk = host(topk_d)
        np.testing.assert_array_equal(topk, oracle.route(scores, N, K, M))
        h = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h, x.cuda(), topk_weights=None if ll else dev(wts))
        xb = I.bf16_bits(x)
        if ll:
            _, loc, _ = oracle.layout_ll(topk, S, E, T)
            used = np.unique(loc[loc >= 0])
            dense = np.where(loc >= 0, np.searchsorted(used, loc), -1).astype(np.int32)
            got = host(ep.ep_handle_get_buffer(h, A.EP_BUF_LL_RECV)[torch.from_numpy(used.astype(np.int64)).cuda()])
            np.testing.assert_array_equal(got, oracle.pack_ll(xb, T, K, True, dense, len(used)))
            rows, shape = E * S * T, (E, S * T, H)
        else:
            lay = oracle.layout_ht(topk, S, E, N, G)
            loc = lay["row2"]
            r1, r2 = int(lay["c1"].sum()), int(lay["c2"].sum())
            pk = oracle.pack_ht(xb, topk, wts, T, N, True, lay["node_row"], loc, r1, r2)
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE1)[:r1]), pk["stage1"])
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:r2]), pk["stage2"])
            rows, shape = r2, (r2, H)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_SLOT if ll else A.EP_MAP_HT_ROW), loc)
        Y = I.normal_bf16(rows, H, 21300 + num_cus)
        Yd = Y.cuda().view(*shape)
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, Yd, dev(wts), out)
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, loc))
        gb = I.bf16_bits(I.normal_bf16(n, H, 21400 + num_cus))
        dY = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        ep.ep_combine_backward(h, torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16).cuda(), dev(wts), dY)
        want_dY, _, _ = oracle.combine_backward(gb, wts, loc, rows)
        np.testing.assert_array_equal(host(dY.view(rows, H))[used if ll else slice(None)],
                                      want_dY[used if ll else slice(None)])
        gx = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_dispatch_backward(h, Yd, gx)
        np.testing.assert_array_equal(host(gx), oracle.dispatch_backward(I.bf16_bits(Y), loc))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


class _TorchPool:
    """alloc_fn / free_fn hooks handing out torch device memory (256-byte
    aligned), counting what comes back."""

    def __init__(self):
        self.live, self.calls, self.freed = {}, 0, 0
        self.alloc_fn = A.ALLOC_FN(self._alloc)
        self.free_fn = A.FREE_FN(self._free)

    def _alloc(self, nbytes, ctx):
        self.calls += 1
        t = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        p = (t.data_ptr() + 255) // 256 * 256
        self.live[p] = t
        return p

    def _free(self, ptr, ctx):
        self.freed += 1
        del self.live[ptr]


@pytest.mark.parametrize("mode", ["ht", "ll"])
def test_allocator_hooks_on_the_device(mode):
    """With allocator hooks group creation makes no HIP call and the first
    operation initialises the device state; the path then works as with
    hipMalloc, and destroying the group hands every block back."""
    N, G, E, K, M, S, T, H = 4, 2, 32, 4, 2, 2, 100, 256
    n, ll = S * T, mode == "ll"
    say(f"allocator hooks {mode}")
    pool = _TorchPool()
    scores = I.uniform_scores(n, E, seed=22000).astype(np.float32)
    x = I.normal_bf16(n, H, 22001)
    wts = I.normal_weights(n, K, 22002)
    g = ep.ep_create_group(mode=mode, num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T, num_src_ranks=S,
                           payload="fp8", alloc_fn=pool.alloc_fn, free_fn=pool.free_fn)
    try:
        assert pool.calls > 0 and len(pool.live) == pool.calls
        topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk_d)
        topk = host(topk_d)
        h = ep.ep_create_handle(g, topk_d)
        ep.ep_dispatch(h, x.cuda(), topk_weights=None if ll else dev(wts))
        if ll:
            _, loc, _ = oracle.layout_ll(topk, S, E, T)
            rows, shape = E * S * T, (E, S * T, H)
        else:
            lay = oracle.layout_ht(topk, S, E, N, G)
            loc = lay["row2"]
            r1, r2 = int(lay["c1"].sum()), int(lay["c2"].sum())
            pk = oracle.pack_ht(I.bf16_bits(x), topk, wts, T, N, True, lay["node_row"], loc, r1, r2)
            np.testing.assert_array_equal(host(buffer(g, A.EP_BUF_HT_STAGE2)[:r2]), pk["stage2"])
            rows, shape = r2, (r2, H)
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_LL_SLOT if ll else A.EP_MAP_HT_ROW), loc)
        Y = I.normal_bf16(rows, H, 22003)
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, Y.cuda().view(*shape), dev(wts), out)
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, loc))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
    assert pool.freed == pool.calls and not pool.live


def test_side_stream_and_blocking_count_queries():
    """The path enqueued on a non-default stream that is still busy with
    earlier work: the blocking receive-count query and the partition query
    wait for the handle's own stream, so they see the counts of this
    routing."""
    N, G, E, K, M, S, T = 8, 8, 256, 8, 4, 1, 4096
    n = S * T
    say("side stream, blocking queries behind earlier work")
    scores = I.scores_for(I.HT_PREFILL)
    want = oracle.layout_ht(oracle.route(scores, N, K, M), S, E, N, G)
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=128, max_tokens_per_rank=T, num_src_ranks=S,
                           payload="fp8")
    try:
        sc = dev(scores)
        topk_d = torch.empty((n, K), dtype=torch.int32, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(30):          # keep the side stream busy for several ms
                big.fill_(7)
            ep.ep_route(g, sc, topk_d)
            h = ep.ep_create_handle(g, topk_d)
            total = ep.ep_handle_get_num_recv(h, -1)
            r5 = ep.ep_handle_get_num_recv(h, 5)
            part = ep.ep_get_partition(h, 9, A.EP_BUF_HT_STAGE1)
        assert total == int(want["c2"].sum())
        assert r5 == int(want["c2"][5 * 4:6 * 4].sum())
        assert part.shape[0] == want["c1"][9]
        side.synchronize()
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
