"""Host-side call counters (ep_group_stats) and the EP_LOG=2 per-call lines."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from gpu_util import I, dev, ep, need_gpu, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_counters_follow_the_calls():
    say("group stats: HT calls, then LL staged calls")
    n, E, K, H = 64, 16, 2, 256
    g = ep.ep_create_group(mode="ht", num_nodes=2, ranks_per_node=2, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n, num_src_ranks=1)
    try:
        topk = torch.empty((n, K), dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(I.uniform_scores(n, E, 3).astype(np.float32)), topk)
        h = ep.ep_create_handle(g, topk)
        x = I.normal_bf16(n, H, 4).cuda()
        ep.ep_dispatch(h, x)
        y = torch.zeros((n * K, H), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        w = dev(I.normal_weights(n, K, 5))
        ep.ep_combine(h, y, w, out)
        ep.ep_combine(h, y, w, out)
        with pytest.raises(ep.EpError):
            ep.ep_combine(h, y, w, out[:1])                # rejected: not counted
        s = ep.ep_group_stats(g)
        assert (s["route_calls"], s["handles_created"], s["dispatch_calls"], s["combine_calls"]) == (1, 1, 1, 2)
        assert (s["tokens_routed"], s["tokens_dispatched"], s["tokens_combined"]) == (n, n, 2 * n)
        assert s["complete_calls"] == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
    g = ep.ep_create_group(mode="ll", num_nodes=2, ranks_per_node=2, num_experts=E, top_k=K,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n, num_src_ranks=1)
    try:
        topk = dev(I.random_topk(n, E, K, seed=6))
        h = ep.ep_create_handle(g, topk)
        ep.ep_dispatch(h, I.normal_bf16(n, H, 7).cuda(), send_only=True)
        ep.ep_complete(h)
        y = torch.zeros((E, n, H), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, y, dev(I.normal_weights(n, K, 8)), out, send_only=True)
        ep.ep_complete(h)
        torch.cuda.synchronize()
        s = ep.ep_group_stats(g)
        assert (s["dispatch_calls"], s["combine_calls"], s["complete_calls"]) == (1, 1, 2)
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_log_level_two_prints_each_call():
    say("EP_LOG=2: one line per call")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import numpy as np, torch, combine_ep_route_amd as ep, ep_inputs as I\n"
            "g = ep.ep_create_group(mode='ht', num_nodes=2, ranks_per_node=2, num_experts=16, top_k=2,"
            " max_nodes_per_token=0, hidden=256, max_tokens_per_rank=32, num_src_ranks=1)\n"
            "t = torch.empty((32, 2), dtype=torch.int32, device='cuda')\n"
            "ep.ep_route(g, torch.from_numpy(I.uniform_scores(32, 16, 1).astype(np.float32)).cuda(), t)\n"
            "h = ep.ep_create_handle(g, t)\n"
            "torch.cuda.synchronize(); ep.ep_destroy_handle(h); ep.ep_destroy_group(g)\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, EP_LOG="2"))
    assert r.returncode == 0, r.stderr
    assert "[ep] route HT tokens=32" in r.stderr
    assert "[ep] create_handle HT tokens=32" in r.stderr
