"""FP8 quantisation over its whole bf16 input domain, GPU vs oracle.

Each 128-element block is quantised with scale = amax/448 and
q = E4M3(x/scale) ("NVSHMEM and DeepEP: GPU-initiated communication", FP8
dispatch with one fp32 scale per 128 elements).  Because x and amax are
bf16, a block's codes depend only on the pairs (x, amax).  The blocks below
take every finite non-zero bf16 amax, subnormals included (32,639 values),
and for each amax every bf16 x of either sign from amax down to amax * 2^-24
(24 binades, 3,073 magnitudes; every smaller x has |x/scale| < 2^-15 and so a
zero code), plus +0 and -0.  Element 0 of each block is the amax itself,
with its sign flipped in every other block.  The GPU writes the blocks
through the dispatch (HT stage-2 rows) and through ep_quantize, and both are
compared byte for byte with the oracle's rows: 195 M (x, amax) pairs.

Blocks holding +-inf are outside the dispatch's contract except for their
finite elements, whose codes are +-0 (x / inf) and whose scale is +inf; the
last test checks exactly that.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu

H = 7168
BLOCKS_PER_ROW = H // 128
WINDOW = 24 * 128            # bf16 bit patterns in 24 binades


def _group_of(xs_pos: np.ndarray, width: int) -> np.ndarray:
    """Rows [amaxes, width] of x patterns: magnitudes, their negations, +0, -0
    (the rest +0)."""
    a, npos = xs_pos.shape
    out = np.zeros((a, width), np.uint16)
    out[:, :npos] = xs_pos
    out[:, npos:2 * npos] = xs_pos | 0x8000
    out[:, 2 * npos + 1] = 0x8000
    return out


def _domain_rows() -> np.ndarray:
    """bf16 bit patterns [rows, H]: one group of blocks per finite amax."""
    bodies, heads = [], []
    # amax patterns up to WINDOW: every positive pattern 1..amax
    for a in range(1, WINDOW + 1):
        nblk = (2 * a + 2 + 126) // 127
        bodies.append(_group_of(np.arange(1, a + 1, dtype=np.uint16)[None, :], nblk * 127).reshape(-1, 127))
        heads.append(np.full(nblk, a, np.uint16))
    # the rest: amax - WINDOW .. amax, the same count for each
    big = np.arange(WINDOW + 1, 0x7F80, dtype=np.uint16)
    npos = WINDOW + 1
    nblk = (2 * npos + 2 + 126) // 127
    pos = (big - WINDOW)[:, None] + np.arange(npos, dtype=np.uint16)[None, :]
    bodies.append(_group_of(pos, nblk * 127).reshape(-1, 127))
    heads.append(np.repeat(big, nblk))
    body = np.concatenate(bodies)
    head = np.concatenate(heads)
    head[1::2] |= 0x8000
    blocks = np.concatenate([head[:, None], body], axis=1)
    # two more: an all-zero block and an all -0 block
    blocks = np.concatenate([blocks, np.zeros((1, 128), np.uint16), np.full((1, 128), 0x8000, np.uint16)])
    n_blocks = blocks.shape[0]
    rows = (n_blocks + BLOCKS_PER_ROW - 1) // BLOCKS_PER_ROW
    out = np.zeros((rows * BLOCKS_PER_ROW, 128), np.uint16)
    out[:n_blocks] = blocks
    return out.reshape(rows, H)


def _oracle_rows(bits: np.ndarray) -> np.ndarray:
    """The oracle's row images, rows split over host threads (the oracle's
    C function runs with the interpreter lock released)."""
    n = bits.shape[0]
    workers = max(1, min(16, os.cpu_count() or 1))
    bounds = np.linspace(0, n, workers + 1).astype(int)
    parts = [(bounds[i], bounds[i + 1]) for i in range(workers) if bounds[i + 1] > bounds[i]]
    with ThreadPoolExecutor(len(parts)) as pool:
        outs = list(pool.map(lambda ab: oracle.token_rows(bits[ab[0]:ab[1]], True), parts))
    return np.concatenate(outs)


def _first_diff(got: np.ndarray, want: np.ndarray, what: str):
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    if len(bad):
        r = bad[0]
        col = np.nonzero(got[r] != want[r])[0][0]
        pytest.fail(f"{what}: {len(bad)} rows differ; first row {r} byte {col}: "
                    f"gpu {got[r, col]:#04x} oracle {want[r, col]:#04x}")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(scope="module")
def domain():
    bits = _domain_rows()
    say(f"FP8 domain: {bits.shape[0]} rows x {BLOCKS_PER_ROW} blocks; oracle rows on the host")
    want = _oracle_rows(bits)
    return bits, want


def test_quantisation_domain_dispatch_matches_oracle(domain):
    bits, want = domain
    n = bits.shape[0]
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    # one expert, one rank: every token's single stage-2 row is its own
    g = ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=1, top_k=1,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n,
                           num_src_ranks=1, payload="fp8")
    try:
        topk = torch.zeros((n, 1), dtype=torch.int32, device="cuda")
        h = ep.ep_create_handle(g, topk)
        ep.ep_dispatch(h, x)
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        np.testing.assert_array_equal(row2[:, 0], np.arange(n))
        got = host(ep.ep_get_buffer(g, A.EP_BUF_HT_STAGE2)[:n])
        _first_diff(got, want, "dispatch")
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)


def test_quantisation_domain_quantize_matches_oracle(domain):
    bits, want = domain
    n = bits.shape[0]
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    g = ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=1, top_k=1,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=1,
                           num_src_ranks=1, payload="fp8")
    try:
        q = torch.empty((n, H), dtype=torch.float8_e4m3fn, device="cuda")
        sc = torch.empty((n, BLOCKS_PER_ROW), dtype=torch.float32, device="cuda")
        ep.ep_quantize(g, x, q, sc)
        got = np.concatenate([host(q.view(torch.uint8)), host(sc).view(np.uint8).reshape(n, -1)], axis=1)
        _first_diff(got, want, "ep_quantize")
    finally:
        ep.ep_destroy_group(g)


def test_block_with_infinity_finite_elements():
    """+-inf in a block: scale +inf, finite elements +-0 codes as the oracle's
    x/inf; the infinite element's code is a NaN code (sign unspecified).  The
    row's other blocks are quantised as usual."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, H)).astype(np.float32)
    x[0, 5] = np.inf
    x[1, 128 * 7 + 100] = -np.inf
    x[2, 0] = np.inf
    x[2, 1] = -np.inf
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    want = oracle.token_rows(bits, True)
    g = ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=1, top_k=1,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=4,
                           num_src_ranks=1, payload="fp8")
    try:
        h = ep.ep_create_handle(g, torch.zeros((4, 1), dtype=torch.int32, device="cuda"))
        ep.ep_dispatch(h, xb.cuda())
        got = host(ep.ep_get_buffer(g, A.EP_BUF_HT_STAGE2)[:4])
        inf_pos = np.isinf(x)
        for r in range(4):
            codes_ok = ~inf_pos[r]
            np.testing.assert_array_equal(got[r, :H][codes_ok], want[r, :H][codes_ok])
            assert np.all((got[r, :H][inf_pos[r]] & 0x7F) == 0x7F)
            np.testing.assert_array_equal(got[r, H:], want[r, H:])   # scales, inf included
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
