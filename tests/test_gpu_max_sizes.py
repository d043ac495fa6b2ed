"""Dispatch and combine at the library's maximum sizes, GPU vs oracle.

1024 experts on 1024 ranks (32 nodes x 32), top-32 with at most 8 nodes per
token (node score = sum of each node's 4 best), hidden 16384, two sources of
70 tokens (a ragged second tile).  This runs the K <= 32 kernel variants,
the generic routing kernel (32 scores per lane would exceed the fast path)
and the widest rows (16896-byte FP8 rows, 32768-byte BF16 rows).  Every row,
map and output is compared with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, host, need_gpu, say
from test_gpu_parity import _ht_dispatch, _ll_dispatch

pytestmark = pytest.mark.gpu

MAX = dict(num_nodes=32, ranks_per_node=32, num_experts=1024, top_k=32, max_nodes=8, hidden=16384,
           num_src_ranks=2, tokens_per_rank=70)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("payload", ["fp8", "bf16"])
def test_ht_dispatch_and_combine_at_maximum_sizes(payload):
    w = I.HT_PREFILL.with_(payload=payload, seed=91, **MAX)
    say(f"HT at maximum sizes ({payload}): E=1024 R=1024 K=32 H=16384 S=2 T=70")
    x = I.tokens_for(w)
    wts = I.normal_weights(w.num_tokens, 32, 92)
    g, topk, lay = _ht_dispatch(w, x, I.scores_for(w), wts)
    try:
        rows2 = int(lay["c2"].sum())
        assert rows2 == w.num_tokens * 32
        # combine over random expert outputs at the stage-2 geometry
        Y = I.normal_bf16(rows2, 16384, 93)
        out = torch.empty((w.num_tokens, 16384), dtype=torch.bfloat16, device="cuda")
        h = ep.ep_create_handle(g, dev(topk))
        np.testing.assert_array_equal(get_map(h, A.EP_MAP_HT_ROW), lay["row2"])
        ep.ep_combine(h, Y.cuda(), dev(wts), out)
        np.testing.assert_array_equal(host(out), oracle.combine(I.bf16_bits(Y), wts, lay["row2"]))
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_ll_dispatch_at_maximum_sizes():
    say("LL at maximum sizes (fp8): E=1024 R=1024 K=32 H=16384 S=2 T=70")
    _ll_dispatch(2, 70, 1024, 32, 16384, "fp8", 70, seed=95, N=32, G=32, M=8)
