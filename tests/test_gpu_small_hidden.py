"""Dispatch and combine at the smallest and oddest hidden sizes, GPU vs oracle.

FP8 at H = 128 (one scale block: the wave's scales are stored one by one),
BF16 at H = 16, 48 and 528 (2, 6 and 66 sixteen-byte chunks per row; the
LL header sits outside a whole 128-byte line, so it is written on its own).
HT rows and metadata, LL messages with headers, and the combine of every
token are compared with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, host, need_gpu, say
from test_gpu_parity import _ht_dispatch, _ll_dispatch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("payload,H", [("fp8", 128), ("bf16", 16), ("bf16", 48), ("bf16", 528)])
def test_ht_small_hidden(payload, H):
    w = I.HT_PREFILL.with_(num_src_ranks=2, tokens_per_rank=70, hidden=H, payload=payload, seed=H)
    say(f"HT dispatch + combine, {payload} H={H}")
    x = I.tokens_for(w)
    wts = I.normal_weights(w.num_tokens, 8, H)
    g, topk, lay = _ht_dispatch(w, x, I.scores_for(w), wts)
    try:
        rows2 = int(lay["c2"].sum())
        Y = I.normal_bf16(rows2, H, H + 7)
        out = torch.empty((w.num_tokens, H), dtype=torch.bfloat16, device="cuda")
        h = ep.ep_create_handle(g, dev(topk))
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay["row2"])
        ep.ep_combine(h, Y.cuda(), dev(wts), out)
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, lay["row2"]))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


@pytest.mark.parametrize("payload,H", [("fp8", 128), ("bf16", 16), ("bf16", 48), ("bf16", 528)])
def test_ll_small_hidden(payload, H):
    say(f"LL dispatch, {payload} H={H}")
    _ll_dispatch(2, 70, 64, 4, H, payload, 70, seed=H + 1, N=4, G=2, M=2)
