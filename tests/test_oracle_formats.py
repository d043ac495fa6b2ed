"""Pins for the oracle's number formats, quantisation and combine (CPU only).

FP8 payload with one fp32 scale per 128 elements and a BF16 combine:
"NVSHMEM and DeepEP: GPU-initiated communication", high-throughput mode
section (FP8 dispatch, BF16 combine).  Library routines used as pins: torch's
CPU casts to bfloat16 and float8_e4m3fn (both round to nearest even).
"""
import numpy as np
import pytest
import torch

import ep_inputs as I
import oracle


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(oracle.f32_to_bf16_array(x), _torch_bf16_bits(x))


def test_bf16_rounding_at_overflow_matches_torch():
    """Every fp32 of the top binade of either sign, and the infinities: from
    the largest finite bf16 plus half its spacing (0x7F7F8000) upwards the
    value rounds to infinity, below it to the largest finite bf16."""
    top = np.arange(0x7F000000, 0x7F800000 + 1, dtype=np.uint64).astype(np.uint32)
    top = np.concatenate([top, top | np.uint32(0x80000000)])
    x = top.view(np.float32)
    got = oracle.f32_to_bf16_array(x)
    np.testing.assert_array_equal(got, _torch_bf16_bits(x))
    f = lambda b: oracle.f32_to_bf16(np.array([b], np.uint32).view(np.float32)[0])
    assert f(0x7F7F7FFF) == 0x7F7F and f(0x7F7F8000) == 0x7F80 and f(0x7F7FFFFF) == 0x7F80
    assert f(0xFF7F8000) == 0xFF80 and f(0x7F800000) == 0x7F80
    assert oracle.f32_to_bf16(float("nan")) == 0x7FC0


def test_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to 1.0 (even)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2**-8 + 2**-16], np.float32)
    got = oracle.f32_to_bf16_array(x)
    np.testing.assert_array_equal(got, _torch_bf16_bits(x))
    assert got[0] == 0x3F80 and got[1] == 0x3F82


def test_e4m3_code_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert np.isnan(ref[c])
            continue
        assert oracle.e4m3_decode(c) == ref[c]
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0**-6 and oracle.e4m3_value(0x01) == 2.0**-9


def _boundary_values():
    """Every code value and every midpoint between neighbours, +-3 ulps."""
    vals = np.array([oracle.e4m3_value(c) for c in range(127)], np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    out, up, dn = [pts], pts, pts
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    out.append(np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30], np.float32))
    allv = np.concatenate(out)
    allv = allv[allv >= 0]
    return np.concatenate([allv, -allv]).astype(np.float32)


def test_e4m3_encode_boundaries_match_torch():
    x = _boundary_values()
    np.testing.assert_array_equal(oracle.e4m3_encode_array(x), _torch_e4m3(x))


def test_e4m3_encode_strided_sweep_matches_torch():
    # every 61st bit pattern of [0, 480) plus its negation, subnormals included
    hi = np.float32(480.0).view(np.uint32)
    bits = np.arange(0, int(hi), 61, dtype=np.uint32)
    x = bits.view(np.float32)
    x = np.concatenate([x, -x])
    np.testing.assert_array_equal(oracle.e4m3_encode_array(x), _torch_e4m3(x))


def test_e4m3_signed_zero_and_saturation():
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-9) == 0x80
    assert oracle.e4m3_encode(1e-9) == 0x00
    assert oracle.e4m3_encode(448.0 * 1.0001) == 0x7E
    assert oracle.e4m3_encode(-1e6) == 0xFE


def test_e4m3_nan_is_the_format_nan():
    """A NaN encodes to S.1111.111, which torch's float8_e4m3fn reads as NaN
    (the format has no infinities and one NaN pattern per sign)."""
    pos = np.array([np.nan], np.float32)
    neg = -pos
    for v in (pos, neg):
        c = int(oracle.e4m3_encode_array(v)[0])
        assert c & 0x7F == 0x7F
        assert c & 0x80 == (0x80 if np.signbit(v[0]) else 0)
        assert np.isnan(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item())


def test_block_with_infinity():
    """A block holding +-inf: amax is inf, so scale = inf/448 = inf and every
    finite x gives x/inf = +-0 (IEEE 754 division), codes 0x00 / 0x80; the
    infinite element's quotient inf/inf is NaN, a NaN code.  The other block
    of the row is unaffected."""
    x = np.zeros((1, 256), np.float32)
    x[0, :128] = np.linspace(-3.0, 3.0, 128, dtype=np.float32)
    x[0, 17] = np.inf
    x[0, 128:] = np.linspace(-1.0, 1.0, 128, dtype=np.float32)
    bits = I.bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    q, sc = oracle.quantize_rows(bits)
    assert np.isinf(sc[0, 0]) and sc[0, 0] > 0
    finite = np.ones(128, bool)
    finite[17] = False
    want = np.where(bits[0, :128] & 0x8000, 0x80, 0x00).astype(np.uint8)
    np.testing.assert_array_equal(q[0, :128][finite], want[finite])
    assert q[0, 17] & 0x7F == 0x7F
    q2, sc2 = oracle.quantize_rows(bits[:, 128:].copy())
    np.testing.assert_array_equal(q[0, 128:], q2[0])
    assert sc[0, 1] == sc2[0, 0] == np.float32(1.0) / np.float32(448.0)


# ---------------------------------------------------------------------------
# Quantisation of rows: amax/448 scale, one per 128 elements
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def xq():
    x = I.normal_bf16(64, 1024, seed=9)
    x[3, 128:256] = 0.0                                   # an all-zero block
    x[5, :128] = -0.0
    x[7, 300] = 1e-30                                     # tiny value
    bits = I.bf16_bits(x)
    q, sc = oracle.quantize_rows(bits)
    return x, bits, q, sc


def test_quantize_matches_torch_blockwise(xq):
    """Same per-block recipe with torch's fp32 ops and its e4m3 cast."""
    x, _, q, sc = xq
    xf = x.to(torch.float32).view(x.shape[0], -1, 128)
    amax = xf.abs().amax(dim=-1)
    scale = amax / torch.tensor(448.0)
    safe = torch.where(scale == 0, torch.ones_like(scale), scale)
    v = torch.where(scale[..., None] == 0, torch.zeros_like(xf), xf / safe[..., None])
    codes = v.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).view(x.shape[0], -1)
    np.testing.assert_array_equal(sc, scale.numpy())
    # zero blocks: torch keeps -0 -> 0x80 from xf/1 = -0; the oracle stores 0x00
    z = (scale == 0).repeat_interleave(128, dim=1).numpy()
    ref = codes.numpy().copy()
    ref[z] = 0
    np.testing.assert_array_equal(q, ref)


def test_quantize_invariants(xq):
    x, bits, q, sc = xq
    n, H = q.shape
    for i in range(n):
        for b in range(H // 128):
            blk = q[i, b * 128:(b + 1) * 128]
            if sc[i, b] == 0:
                assert np.all(blk == 0)
                continue
            # amax/scale = 448 (1 +- 2^-23) rounds to 448: some code is +-448
            assert np.any((blk & 0x7F) == 0x7E)


def test_quantize_error_bound(xq):
    x, bits, q, sc = xq
    xf = x.to(torch.float32).numpy().astype(np.float64)
    dec = np.vectorize(oracle.e4m3_decode)(q).astype(np.float64)
    s = np.repeat(sc.astype(np.float64), 128, axis=1)
    err = np.abs(dec * s - xf)
    # normal codes: half an ulp of a 3-bit mantissa, 2^-4 relative;
    # subnormal codes: half the subnormal spacing 2^-10 times the scale
    bound = np.maximum(2.0**-4 * np.abs(xf), 2.0**-10 * s) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_row_image_layout(xq):
    _, bits, q, sc = xq
    rows = oracle.token_rows(bits, fp8=True)
    assert rows.shape[1] == 1024 + 8 * 4
    np.testing.assert_array_equal(rows[:, :1024], q)
    np.testing.assert_array_equal(rows[:, 1024:].copy().view(np.float32), sc)
    rows16 = oracle.token_rows(bits, fp8=False)
    np.testing.assert_array_equal(rows16.view(np.uint16), bits)


def test_dequant_matches_torch(xq):
    _, bits, q, sc = xq
    rows = oracle.token_rows(bits, fp8=True)
    y = oracle.dequant_rows(rows, 1024, fp8=True)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    ref = (dec * torch.from_numpy(sc).repeat_interleave(128, dim=1)).to(torch.bfloat16)
    np.testing.assert_array_equal(y, ref.view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------------------
# Combine: fp32 fused multiply-add chain in k order, then bf16
# ---------------------------------------------------------------------------

def test_combine_identity_returns_input():
    """Identity experts + normalised weights return the input bit for bit."""
    n, K, H = 96, 8, 256
    x = I.bf16_bits(I.normal_bf16(n, H, seed=21))
    w = I.normal_weights(n, K, seed=22)
    loc = np.arange(n * K, dtype=np.int32).reshape(n, K)
    Y = np.repeat(x, K, axis=0)                    # row i*K+k holds token i
    np.testing.assert_array_equal(oracle.combine(Y, w, loc), x)


def test_combine_one_hot_is_gather():
    n, K, H = 50, 4, 128
    rng = np.random.default_rng(5)
    Y = I.bf16_bits(I.normal_bf16(300, H, seed=23))
    loc = rng.integers(0, 300, size=(n, K)).astype(np.int32)
    w = np.zeros((n, K), np.float32)
    pick = rng.integers(0, K, size=n)
    w[np.arange(n), pick] = 1.0
    np.testing.assert_array_equal(oracle.combine(Y, w, loc), Y[loc[np.arange(n), pick]])


def test_combine_skips_invalid_and_k1_copy():
    H = 64
    Y = I.bf16_bits(I.normal_bf16(10, H, seed=24))
    loc = np.array([[3], [-1]], np.int32)
    w = np.ones((2, 1), np.float32)
    out = oracle.combine(Y, w, loc)
    np.testing.assert_array_equal(out[0], Y[3])
    assert np.all(out[1] == 0)


def test_combine_within_fp64_error_bound():
    n, K, H = 64, 8, 512
    rng = np.random.default_rng(6)
    Yt = I.normal_bf16(400, H, seed=25)
    Y = I.bf16_bits(Yt)
    loc = rng.integers(0, 400, size=(n, K)).astype(np.int32)
    w = I.normal_weights(n, K, seed=26)
    out = torch.from_numpy(oracle.combine(Y, w, loc).view(np.int16)).view(torch.bfloat16)
    out = out.to(torch.float64).numpy()
    Yf = Yt.to(torch.float64).numpy()
    exact = np.einsum("nk,nkh->nh", w.astype(np.float64), Yf[loc])
    mag = np.einsum("nk,nkh->nh", np.abs(w.astype(np.float64)), np.abs(Yf[loc]))
    bound = K * 2.0**-24 * mag + 2.0**-8 * np.abs(exact) + 1e-40
    assert np.all(np.abs(out - exact) <= bound)


def _bf16_exact(values):
    """bf16 bit patterns of values bf16 holds exactly."""
    u = np.array(values, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def test_combine_is_a_fused_multiply_add_chain():
    """Worked by hand.  Weights -(1+2^-23) and 1+2^-23 on two rows of
    1+2^-7: the first step rounds -(1+2^-7+2^-23+2^-30) to -(1+2^-7+2^-23);
    a fused second step then leaves exactly 2^-30 (bf16 0x3080), whereas a
    product rounded before the add would cancel to 0."""
    Y = np.tile(_bf16_exact([1 + 2.0**-7]), (2, 4))
    w = np.array([[-(1 + 2.0**-23), 1 + 2.0**-23]], np.float32)
    out = oracle.combine(Y, w, np.array([[0, 1]], np.int32))
    assert np.all(out == 0x3080) and _bf16_exact([2.0**-30])[0] == 0x3080


def test_combine_accumulates_in_k_order():
    """Worked by hand.  Rows 2^24, 1, -2^24 with unit weights: in k order
    2^24 + 1 is a tie that rounds to 2^24 (even) and the sum ends at +0; in
    the reverse order -2^24 + 1 is exact and the sum ends at 1."""
    rows = _bf16_exact([2.0**24, 1.0, -2.0**24])
    Y = np.repeat(rows[:, None], 4, axis=1)
    w = np.ones((2, 3), np.float32)
    out = oracle.combine(Y, w, np.array([[0, 1, 2], [2, 1, 0]], np.int32))
    assert np.all(out[0] == 0x0000) and np.all(out[1] == 0x3F80)


def test_combine_starts_from_plus_zero():
    """Every product is -0 (1 * -0, and -0 * +0): the chain from +0 ends at
    +0, where starting from -0 or from the first product would give -0."""
    Y = np.array([[0x8000] * 4, [0x0000] * 4], np.uint16)
    w = np.array([[1.0, -0.0]], np.float32)
    out = oracle.combine(Y, w, np.array([[0, 1]], np.int32))
    assert np.all(out == 0x0000)
