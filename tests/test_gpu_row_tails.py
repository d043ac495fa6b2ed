"""Receive-buffer row tails: the bytes between a row's end and its pitch.

Rows and LL messages start on 128-byte boundaries (pitch = size rounded up
to 128).  When a row's scale bytes are whole 16-byte groups (hidden % 512 ==
0) the dispatch writes the last line of every row it fills in full, so the
bytes after an HT row, or after an LL message's header, read zero.  For other
hidden sizes that padding is left as it was.  Rows and slots the layout does
not use are never written.  The buffers are filled with a canary byte first;
row contents are compared with the oracle as in the parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu

CANARY = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _pitch_view(g, which):
    """The buffer as [rows - 1, pitch] bytes (the last row is left out so the
    view stays inside the storage the library's view describes)."""
    base = ep.ep_get_buffer(g, which)
    rows, pitch = base.shape[0], base.stride(0)
    return torch.as_strided(base, (rows - 1, pitch), (pitch, 1)), base.shape[1]


@pytest.mark.parametrize("H", [1024, 1152])
def test_ht_row_tails(H):
    S, T, E, N, G, K, M = 2, 300, 64, 4, 2, 6, 2
    say(f"HT row tails H={H}")
    scores = I.uniform_scores(S * T, E, 71).astype(np.float32)
    x = I.normal_bf16(S * T, H, 72)
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=H, max_tokens_per_rank=T + 20,
                           num_src_ranks=S, payload="fp8")   # spare rows after the used ones
    try:
        v1, rb = _pitch_view(g, A.EP_BUF_HT_STAGE1)
        v2, _ = _pitch_view(g, A.EP_BUF_HT_STAGE2)
        v1.fill_(CANARY)
        v2.fill_(CANARY)
        topk = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk)
        h = ep.ep_create_handle(g, topk)
        ep.ep_dispatch(h, x.cuda())
        node_row = get_map(h, A.EP_MAP_HT_NODE_ROW)
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        img = oracle.token_rows(I.bf16_bits(x), True)
        pad = 0 if H % 512 == 0 else CANARY
        for view, rows_of in ((v1, node_row), (v2, row2)):
            used = int((rows_of >= 0).sum())
            assert view.shape[0] >= used + 32
            got = host(view[:used + 32])
            assert got.shape[1] > rb, "no padding to check"
            tok = np.repeat(np.arange(S * T), rows_of.shape[1])
            r = rows_of.reshape(-1)
            keep = r >= 0
            np.testing.assert_array_equal(np.sort(r[keep]), np.arange(used))
            np.testing.assert_array_equal(got[r[keep], :rb], img[tok[keep]])
            assert np.all(got[:used, rb:] == pad), f"row tails not {pad:#x}"
            assert np.all(got[used:] == CANARY), "an unused row was written"
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("H,payload", [(1024, "fp8"), (1152, "fp8"), (512, "bf16"), (576, "bf16")])
def test_ll_message_tails(H, payload):
    S, T, E, K, slots = 3, 40, 32, 4, 48
    say(f"LL message tails H={H} {payload}")
    scores = I.uniform_scores(S * T, E, 81).astype(np.float32)
    x = I.normal_bf16(S * T, H, 82)
    g = ep.ep_create_group(mode="ll", num_nodes=2, ranks_per_node=2, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=slots,
                           num_src_ranks=S, payload=payload)
    try:
        view, rb = _pitch_view(g, A.EP_BUF_LL_RECV)
        view.fill_(CANARY)
        topk = torch.empty((S * T, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(scores), topk)
        h = ep.ep_create_handle(g, topk)
        ep.ep_dispatch(h, x.cuda())
        slot = get_map(h, A.EP_MAP_LL_SLOT)
        got = host(view)
        img = oracle.token_rows(I.bf16_bits(x), payload == "fp8")
        row = img.shape[1]
        assert rb == row + 16 and got.shape[1] > rb
        pad = 0 if H % 512 == 0 else CANARY
        written = np.zeros(got.shape[0], bool)
        for i in range(S * T):
            for k in range(K):
                m = slot[i, k]
                if m >= got.shape[0]:
                    continue                      # the view leaves out the last message
                written[m] = True
                np.testing.assert_array_equal(got[m, :row], img[i], err_msg=f"token {i} k {k}")
                assert list(got[m, row:rb].view(np.int32)) == [i % T, i // T, k, 0]
                assert np.all(got[m, rb:] == pad), f"message tail of token {i} k {k}"
        assert np.all(got[~written] == CANARY), "an unused slot was written"
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
