"""Special values through the bf16-producing steps, GPU vs oracle, bit for bit.

Each step ends in a bf16 round to nearest even of an fp32 value (FP8
dispatch with fp32 scales and a BF16 combine: "NVSHMEM and DeepEP:
GPU-initiated communication", high-throughput section; the backward pass
reusing the handle: "NCCL EP paper notes", training example).  The inputs
reach the corners of that rounding: signed zeros, fp32 subnormals (no flush
to zero on either side), the largest finite values and overflow to infinity.
NaN inputs are outside the contract, so the inputs are chosen so that no NaN
can arise (no infinite inputs, no inf - inf).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu

# bf16 bit patterns: zeros, subnormals, smallest normals, largest finite,
# +-1 and their neighbours, 2, 0.5
PALETTE = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080,
                    0x7F7F, 0xFF7F, 0x7F7E, 0x3F80, 0xBF80, 0x3F81, 0xBF81, 0x4000, 0x3F00],
                   np.uint16)
# fp32 weights: zeros, subnormals, ordinary values, 1 + ulp, a huge one
WEIGHTS = np.array([0.0, -0.0, 1e-39, 1.5e-45, 0.5, 0.75, 1.0, 1.0 + 2.0**-23, 2.0, -1.5, 3.0e38],
                   np.float32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _group(n, K, H, payload):
    return ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=4 * K, top_k=K,
                              max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n, num_src_ranks=1,
                              payload=payload)


def test_identity_expert_special_scales():
    """decode(q) * scale in fp32, then bf16: every non-NaN code against zero,
    subnormal, tiny, ordinary, huge and overflowing scales."""
    H = 256
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    scales = np.array([0.0, 1.4e-45, 1e-42, 1.2e-38, 2.0**-126, 1.0 / 448.0, 1.0, 1.7, 7.5e35,
                       7.59e35, 1.0e37, 3.0e38], np.float32)
    n = len(scales) * 2
    rng = np.random.default_rng(5)
    rows = np.zeros((n, H + H // 128 * 4), np.uint8)
    for r in range(n):
        # odd rows hold every non-NaN code in order, even rows random ones
        rows[r, :H] = np.resize(codes, H) if r % 2 else rng.choice(codes, size=H)
        blk = np.array([scales[r // 2], scales[(r // 2 + 5) % len(scales)]], np.float32)
        rows[r, H:] = blk.view(np.uint8)
    say(f"identity expert: {n} rows of special codes and scales")
    want = oracle.dequant_rows(rows, H, True)
    wf = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert not np.isnan(wf).any()
    assert np.isinf(wf).any() and (((want & 0x7F80) == 0) & ((want & 0x7F) != 0)).any()
    g = _group(8, 2, H, "fp8")
    try:
        y = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        pitch = (rows.shape[1] + 15) // 16 * 16            # row starts 16-byte aligned
        padded = torch.zeros((n, pitch), dtype=torch.uint8, device="cuda")
        padded[:, :rows.shape[1]] = torch.from_numpy(rows).cuda()
        ep.ep_dequantize_rows(g, padded[:, :rows.shape[1]], y)
        np.testing.assert_array_equal(host(y), want)
    finally:
        ep.ep_destroy_group(g)


def test_backward_special_values():
    """Combine adjoint row gradients bf16(w * g) (one fp32 product each) and
    the dispatch adjoint bf16(sum_k dRows) over special values."""
    n, K, H = 256, 8, 256
    say("backward special values")
    rng = np.random.default_rng(13)
    gb = PALETTE[rng.integers(0, len(PALETTE), size=(n, H))]
    gb[::7] = I.bf16_bits(I.normal_bf16(len(gb[::7]), H, 14))
    w = WEIGHTS[rng.integers(0, len(WEIGHTS), size=(n, K))]
    topk = I.random_topk(n, 4 * K, K, seed=15)
    g = _group(n, K, H, "bf16")
    try:
        h = ep.ep_create_handle(g, dev(topk))
        loc = get_map(h, A.EP_MAP_HT_ROW)
        rows = n * K
        want_dY, _, _ = oracle.combine_backward(gb, w, loc, rows)
        f = torch.from_numpy(want_dY.view(np.int16)).view(torch.bfloat16).float().numpy()
        assert not np.isnan(f).any() and np.isinf(f).any()
        assert (((want_dY & 0x7F80) == 0) & ((want_dY & 0x7F) != 0)).any()
        dY = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine_backward(h, _bf16(gb), dev(w), dY)
        np.testing.assert_array_equal(host(dY), want_dY)
        # dispatch adjoint: finite rows only, so the fp32 chain can reach
        # +-inf but never inf - inf
        dR = PALETTE[rng.integers(0, len(PALETTE), size=(rows, H))]
        want_dx = oracle.dispatch_backward(dR, loc)
        fx = torch.from_numpy(want_dx.view(np.int16)).view(torch.bfloat16).float().numpy()
        assert not np.isnan(fx).any() and np.isinf(fx).any()
        dx = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_dispatch_backward(h, _bf16(dR), dx)
        np.testing.assert_array_equal(host(dx), want_dx)
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def _node_scores_ok(s, N, J):
    """True when no node score (float32 sum of the node's J largest scores,
    largest first) is NaN, i.e. no +inf meets -inf."""
    P = s.shape[1] // N
    top = -np.sort(-s.reshape(len(s), N, P), axis=2)[:, :, :J]
    with np.errstate(invalid="ignore", over="ignore"):
        acc = top[:, :, 0].astype(np.float32)
        for j in range(1, J):
            acc = (acc + top[:, :, j]).astype(np.float32)
    return ~np.isnan(acc).any(axis=1)


@pytest.mark.parametrize("E,N,G,K,M", [(256, 8, 8, 8, 4), (96, 4, 2, 6, 2), (256, 8, 8, 8, 0)])
def test_route_special_scores(E, N, G, K, M):
    """Infinities, the largest finite floats (node scores that overflow to
    +inf and tie), subnormals, signed zeros and negatives, on the fast and
    the generic routing kernels."""
    n = 512
    say(f"route special scores E={E} M={M}")
    pal = np.array([np.inf, 3.4028235e38, 3.0e38, 1.0e38, 1.0, 1e-40, -1e-40, 1.4e-45, 0.0, -0.0,
                    -1.0, -3.0e38, -np.inf], np.float32)
    rng = np.random.default_rng(E + K + M)
    s = pal[rng.integers(0, len(pal), size=(n, E))]
    s[::3] = np.where(rng.random((len(s[::3]), E)) < 0.5, 1e-40, -0.0).astype(np.float32)
    J = (K + M - 1) // M if 0 < M < N else 1
    if 0 < M < N:
        bad = ~_node_scores_ok(s, N, J)
        s[bad] = np.abs(s[bad])                  # no -inf left: no inf - inf in a node score
        assert _node_scores_ok(s, N, J).all()
    g = ep.ep_create_group(mode="ht", num_nodes=N, ranks_per_node=G, num_experts=E, top_k=K,
                           max_nodes_per_token=M, hidden=128, max_tokens_per_rank=n,
                           num_src_ranks=1, payload="fp8")
    try:
        out = torch.full((n, K), -7, dtype=torch.int32, device="cuda")
        ep.ep_route(g, dev(s), out)
        np.testing.assert_array_equal(host(out), oracle.route(s, N, K, M))
    finally:
        ep.ep_destroy_group(g)
