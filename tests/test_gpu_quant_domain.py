"""FP8 quantisation over (nearly) its whole bf16 input domain, GPU vs oracle.

Each 128-element block is quantised with scale = amax/448 and
q = E4M3(x/scale) ("NVSHMEM and DeepEP: GPU-initiated communication", FP8
dispatch with one fp32 scale per 128 elements).  Because x and amax are
bf16, the quotient x/scale depends only on the pair (x, amax), and scaling
both by a power of two leaves it unchanged unless the scale leaves the
normal fp32 range.  So the blocks below cover: every bf16 mantissa of amax
at exponents -120, -64, 0, 64 and 120, plus every subnormal bf16 amax; and
for each amax, every bf16 x of either sign within 24 binades below it (any
smaller x encodes to a zero code).  Element 0 of each block is amax itself.
The rows the GPU writes are compared byte for byte with the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import A, I, dev, ep, get_map, host, need_gpu, say

pytestmark = pytest.mark.gpu

H = 7168
BLOCKS_PER_ROW = H // 128


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _domain_rows() -> np.ndarray:
    """bf16 bit patterns [rows, H] covering the (x, amax) domain."""
    amaxes = []
    for e in (-120, -64, 0, 64, 120):
        exp_field = e + 127
        amaxes += [(exp_field << 7) | m for m in range(128)]
    amaxes += list(range(1, 128))                                   # subnormal bf16
    all_bits = np.arange(1 << 15, dtype=np.uint32)                  # non-negative patterns
    all_vals = _bf16_value(all_bits)
    finite = np.isfinite(all_vals)
    blocks = []
    for a in amaxes:
        av = _bf16_value(np.array([a], np.uint32))[0]
        sel = finite & (all_vals <= av) & (all_vals >= av * 2.0**-24)
        xs = all_bits[sel]
        xs = np.concatenate([xs, xs | 0x8000, [0, 0x8000]]).astype(np.uint16)
        for start in range(0, len(xs), 127):
            chunk = xs[start:start + 127]
            blk = np.zeros(128, np.uint16)
            blk[0] = a
            blk[1:1 + len(chunk)] = chunk
            blocks.append(blk)
    # also blocks of all-zero and of negative amax (the largest |x| negative)
    z = np.zeros(128, np.uint16)
    blocks.append(z)
    neg = np.array(blocks[7], np.uint16).copy()
    neg[0] |= 0x8000
    blocks.append(neg)
    n_blocks = len(blocks)
    rows = (n_blocks + BLOCKS_PER_ROW - 1) // BLOCKS_PER_ROW
    flat = np.zeros(rows * BLOCKS_PER_ROW * 128, np.uint16)
    flat[:n_blocks * 128] = np.concatenate(blocks)
    return flat.reshape(rows, H)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_quantisation_domain_matches_oracle():
    bits = _domain_rows()
    n = bits.shape[0]
    say(f"FP8 domain check: {n} rows x {BLOCKS_PER_ROW} blocks")
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    # one expert, one rank: every token's single stage-2 row is its own
    g = ep.ep_create_group(mode="ht", num_nodes=1, ranks_per_node=1, num_experts=1, top_k=1,
                           max_nodes_per_token=0, hidden=H, max_tokens_per_rank=n,
                           num_src_ranks=1, payload="fp8")
    try:
        topk = torch.zeros((n, 1), dtype=torch.int32, device="cuda")
        h = ep.ep_create_handle(g, topk)
        ep.ep_dispatch(h, x.cuda())
        row2 = get_map(h, A.EP_MAP_HT_ROW)
        np.testing.assert_array_equal(row2[:, 0], np.arange(n))
        got = host(ep.ep_get_buffer(g, A.EP_BUF_HT_STAGE2)[:n])
        want = oracle.token_rows(bits, True)
        bad = np.nonzero(np.any(got != want, axis=1))[0]
        if len(bad):
            r = bad[0]
            col = np.nonzero(got[r] != want[r])[0][0]
            pytest.fail(f"{len(bad)} rows differ; first row {r} byte {col}: "
                        f"gpu {got[r, col]:#04x} oracle {want[r, col]:#04x}")
        assert ep.ep_get_device_error(g) == 0
        ep.ep_destroy_handle(h)
    finally:
        ep.ep_destroy_group(g)
