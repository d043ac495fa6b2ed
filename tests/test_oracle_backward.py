"""Pins of the oracle's backward pass (reuse of the forward handle in training,
"NCCL EP paper notes", usage section): combine_backward is the adjoint of the
combine and dispatch_backward the adjoint of the dispatch.  Checked against
the forward map itself in exact arithmetic, central differences, torch's
CPU fp32 multiply + bf16 cast, and special cases -- not against a retyped
formula."""
import numpy as np
import pytest
import torch

import oracle


def _bits(vals: np.ndarray) -> np.ndarray:
    """float values exactly representable in bf16 -> bf16 bits."""
    f = np.ascontiguousarray(vals, np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), f), "not a bf16 value"
    return b


def _vals(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _case(seed, n=6, K=3, H=16, rows=24, drop=True, exact=True):
    rng = np.random.default_rng(seed)
    loc = np.full((n, K), -1, np.int32)
    perm = rng.permutation(rows)[: n * K].reshape(n, K).astype(np.int32)
    loc[:] = perm
    if drop:
        loc[1, 2] = -1
        loc[4, 0] = -1
    if exact:
        g = rng.integers(-8, 9, (n, H)).astype(np.float32)
        Y = rng.integers(-8, 9, (rows, H)).astype(np.float32)
        w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0, -1.0], np.float32), (n, K))
    else:
        g = _vals(_bits_round(rng.standard_normal((n, H))))
        Y = _vals(_bits_round(rng.standard_normal((rows, H))))
        w = rng.random((n, K)).astype(np.float32)
    return g, Y, w.astype(np.float32), loc


def _bits_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _forward64(Y, w, loc):
    """The combine's linear map in fp64 (no rounding)."""
    n, K = loc.shape
    out = np.zeros((n, Y.shape[1]), np.float64)
    for t in range(n):
        for k in range(K):
            if loc[t, k] >= 0:
                out[t] += np.float64(w[t, k]) * Y[loc[t, k]].astype(np.float64)
    return out


def test_adjoint_identity_exact():
    """<g, C(Y; w)> = sum_tk w_tk dw_tk = sum_r <dY_r, Y_r>, all exact: small
    integers and power-of-two weights make every product and sum exact."""
    g, Y, w, loc = _case(1)
    dY, dw, da = oracle.combine_backward(_bits(g), w, loc, Y.shape[0], _bits(Y))
    lhs = float(np.sum(g.astype(np.float64) * _forward64(Y, w, loc)))
    mid = float(np.sum(w.astype(np.float64) * dw))
    rhs = float(np.sum(_vals(dY).astype(np.float64) * Y.astype(np.float64)))
    assert lhs == mid == rhs
    # the row a (t, k) entry points at holds exactly w * g
    for t in range(loc.shape[0]):
        for k in range(loc.shape[1]):
            r = loc[t, k]
            if r >= 0:
                np.testing.assert_array_equal(_vals(dY[r]), w[t, k] * g[t])
                assert dw[t, k] == float(np.dot(g[t].astype(np.float64), Y[r].astype(np.float64)))
            else:
                assert dw[t, k] == 0.0 and da[t, k] == 0.0
    # rows no entry points at are not written
    untouched = np.setdiff1d(np.arange(Y.shape[0]), loc[loc >= 0])
    assert not dY[untouched].any()


def test_weight_gradient_is_the_derivative():
    """dw equals the central difference of F(w) = <g, C(Y; w)> (linear in w,
    so the difference quotient is exact up to fp64 rounding)."""
    g, Y, w, loc = _case(2, n=5, K=4, H=64, rows=40, exact=False)
    _, dw, da = oracle.combine_backward(_bits(g), w, loc, Y.shape[0], _bits(Y))
    F = lambda ww: float(np.sum(g.astype(np.float64) * _forward64(Y, ww, loc)))
    d = 0.5
    for t in range(loc.shape[0]):
        for k in range(loc.shape[1]):
            wp = w.astype(np.float64).copy(); wp[t, k] += d
            wm = w.astype(np.float64).copy(); wm[t, k] -= d
            fd = (F(wp) - F(wm)) / (2 * d)
            assert abs(fd - dw[t, k]) <= 1e-9 * (1 + da[t, k])
            if loc[t, k] >= 0:
                assert da[t, k] == pytest.approx(float(np.sum(np.abs(g[t].astype(np.float64) * Y[loc[t, k]]))))


def test_row_gradient_rounding_matches_torch():
    """dY = bf16(w * g) with one fp32 multiply: torch's CPU fp32 multiply
    followed by its nearest-even bf16 cast (a library routine) agrees on every
    element, including products that need rounding."""
    rng = np.random.default_rng(3)
    n, K, H, rows = 16, 4, 256, 64
    g = _bits_round(rng.standard_normal((n, H)) * 3)
    w = (rng.random((n, K)) * 1.7 + 0.01).astype(np.float32)
    loc = rng.permutation(rows)[: n * K].reshape(n, K).astype(np.int32)
    dY, _, _ = oracle.combine_backward(g, w, loc, rows)
    gt = torch.from_numpy(_vals(g))
    for t in range(n):
        for k in range(K):
            want = (torch.tensor(w[t, k]) * gt[t]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            np.testing.assert_array_equal(dY[loc[t, k]], want)


def test_dispatch_backward_special_cases():
    rng = np.random.default_rng(4)
    rows, H = 12, 32
    R = _bits_round(rng.standard_normal((rows, H)))
    # K = 1: a row gather (copy)
    loc1 = rng.permutation(rows)[:5].reshape(5, 1).astype(np.int32)
    np.testing.assert_array_equal(oracle.dispatch_backward(R, loc1), R[loc1[:, 0]])
    # exact data: the fp32 sum equals the fp64 sum, rounded once to bf16
    Ri = rng.integers(-20, 21, (rows, H)).astype(np.float32)
    loc = rng.permutation(rows)[:9].reshape(3, 3).astype(np.int32)
    loc[2, 1] = -1
    got = _vals(oracle.dispatch_backward(_bits(Ri), loc))
    for t in range(3):
        want = sum(Ri[r].astype(np.float64) for r in loc[t] if r >= 0)
        np.testing.assert_array_equal(got[t], want.astype(np.float32))
    # adjointness with the dispatch's copy: <dx, x> = sum_r <dRows_r, rows_r>
    x = rng.integers(-4, 5, (3, H)).astype(np.float32)
    rows_img = np.zeros((rows, H), np.float64)
    for t in range(3):
        for r in loc[t]:
            if r >= 0:
                rows_img[r] = x[t]
    assert float(np.sum(got.astype(np.float64) * x)) == float(np.sum(Ri.astype(np.float64) * rows_img))
