"""LL combine at the decode geometry, GPU vs oracle, every output token.

"NCCL EP paper notes", tensor layouts: in LL the expert outputs come back as
a 3-D expert-major tensor [E, S*T_max, H] at the dispatch's slot positions;
"NVSHMEM and DeepEP: GPU-initiated communication", low-latency section: 128
tokens per rank, 64 ranks, 256 experts, top-8 with at most 4 nodes, hidden
7168, BF16 combine.  The expert-output tensor is the whole [256, 64*128,
7168] array (30 GB); only the slots the routing uses are filled (N(0,1)
bf16), the rest hold a NaN pattern that the combine must never read.  The
combine runs staged (send_only + ep_complete) as in the decode pipeline and
un-staged, and every one of the 8192 output tokens is compared bit for bit
with oracle.combine over the same slots and weights.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, group_for, host, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_ll_combine_full_decode_geometry():
    w = I.LL_DECODE
    S, T, E, K, H = w.num_src_ranks, w.tokens_per_rank, w.num_experts, w.top_k, w.hidden
    n = S * T
    rows = E * S * T
    say(f"LL combine at [E={E}, S*T={S * T}, H={H}] ({rows * H * 2 / 2**30:.1f} GiB), {n} tokens")
    scores = I.scores_for(w)
    weights = I.normal_weights(n, K, w.seed)
    g = group_for(w, hidden=H)
    try:
        topk = torch.empty((n, K), dtype=torch.int32, device="cuda")
        h = ep.ep_route_handle(g, dev(scores), topk)
        slot = get_map(h, A.EP_MAP_LL_SLOT)
        want_cnt, want_slot, err = oracle.layout_ll(oracle.route(scores, 8, K, 4), S, E, T)
        np.testing.assert_array_equal(slot, want_slot)
        used = np.unique(slot[slot >= 0])
        # expert outputs: N(0,1) bf16 at the used slots, NaN everywhere else
        y_used = I.normal_bf16(len(used), H, 33)
        Y = torch.full((E, S * T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        Y.view(rows, H)[torch.from_numpy(used.astype(np.int64)).cuda()] = y_used.cuda()
        # the oracle sees the used rows only, with the slot map renumbered to them
        compact = np.full(rows, -1, np.int64)
        compact[used] = np.arange(len(used))
        loc = np.where(slot >= 0, compact[np.maximum(slot, 0)], -1).astype(np.int32)
        want = oracle.combine(I.bf16_bits(y_used), weights, loc)
        w_d = dev(weights)
        for staged in (True, False):
            out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
            ep.ep_combine(h, Y, w_d, out, send_only=staged)
            if staged:
                ep.ep_complete(h)
            got = host(out)
            bad = np.nonzero(np.any(got != want, axis=1))[0]
            assert len(bad) == 0, f"staged={staged}: {len(bad)} tokens differ, first {bad[:5]}"
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
        del Y
    finally:
        ep.ep_destroy_group(g)
        torch.cuda.empty_cache()
