"""Pins of the per-rank HT stage-2 layout (one copy per destination GPU, the
alternative the DeepEP page's high-throughput traffic study compares).

- The page's printed per-GPU copy counts: 6.26 cross-node copies per token
  with the 4-node limit, 6.50 without (tests/golden/deepep_routing_study.txt),
  reproduced through the numpy restatement of the study; the oracle's row
  counts must equal that restatement's exact totals.
- Brute force: every row recounted from its definition on small inputs.
- The rows form a bijection onto [0, total); each valid entry lands in
  exactly one row's received top-k, with its local id and weight.
- The per-rank combine (sum of per-rank partial rows) equals the per-expert
  combine when the partial rows hold the exact weighted sums.
"""
import os

import numpy as np
import pytest

import ep_inputs as I
import oracle
from oracle import page_sim

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deepep_routing_study.txt")


def _golden_per_gpu(key):
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, *vals = line.split()
            if name == key:
                return float(vals[2])          # the per_gpu column
    raise KeyError(key)


def _rank_rows_per_token(topk, L):
    return np.array([len(np.unique(r // L)) for r in topk])


@pytest.mark.parametrize("limit", ["4nodes", "none"])
def test_page_per_gpu_copy_counts(limit):
    scores = I.page_scores(page_sim.TOKENS, page_sim.EXPERTS, 0).astype(np.float32)
    M = 4 if limit == "4nodes" else 0
    topk = oracle.route(scores, 8, 8, M)
    st = page_sim.traffic(topk)
    assert round(st["per_gpu"], 2) == _golden_per_gpu(limit)
    lay = oracle.layout_ht_rank(topk, 1, 256, 64)
    assert lay["err"] == 0
    rank_of_row = np.repeat(np.arange(64), lay["c2"])
    # source rank 0 sits on node 0 (ranks 0..7); cross-node rows go to ranks 8..63
    cross = int((rank_of_row >= 8).sum())
    assert cross == st["per_gpu"] * page_sim.TOKENS       # the study's exact total
    assert int(lay["c2"].sum()) == int(_rank_rows_per_token(topk, 4).sum())


def test_brute_force_rows():
    rng = np.random.default_rng(5)
    S, T, K, E, R = 3, 23, 5, 24, 6
    L = E // R
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(S * T)]).astype(np.int32)
    topk[4, 3] = topk[4, 1]                   # a repeat: no row
    topk[9, 0] = -2                           # out of range: no row
    lay = oracle.layout_ht_rank(topk, S, E, R)
    assert lay["err"] == 3
    row2 = lay["row2"]
    total = int(lay["c2"].sum())
    used = row2[row2 >= 0]
    np.testing.assert_array_equal(np.sort(used), np.arange(total))
    valid = lambda i, k: 0 <= topk[i, k] < E and topk[i, k] not in topk[i, :k]
    ranks_of = [sorted({topk[i, k] // L for k in range(K) if valid(i, k)}) for i in range(S * T)]
    for r in range(R):
        assert lay["c2"][r] == sum(r in rs for rs in ranks_of)
        assert lay["off2"][r] == sum(lay["c2"][:r])
    for i in range(S * T):
        seen = set()
        for k in range(K):
            if not valid(i, k):
                assert row2[i, k] == -1
                continue
            r = topk[i, k] // L
            if r in seen:
                assert row2[i, k] == -1
                continue
            seen.add(r)
            earlier = sum(r in ranks_of[j] for j in range(i))
            assert row2[i, k] == lay["off2"][r] + earlier


def test_received_topk_metadata():
    rng = np.random.default_rng(6)
    n, K, E, R = 40, 6, 32, 8
    L = E // R
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(n)]).astype(np.int32)
    w = rng.random((n, K)).astype(np.float32)
    lay = oracle.layout_ht_rank(topk, 1, E, R)
    rows = int(lay["c2"].sum())
    mt, mw = oracle.meta_ht_rank(topk, w, lay["row2"], E, R, rows)
    seen = 0
    for i in range(n):
        for k in range(K):
            row = lay["row2"][i, k]
            if row < 0:
                continue
            r = topk[i, k] // L
            for kk in range(K):
                if topk[i, kk] // L == r:
                    assert mt[row, kk] == topk[i, kk] - r * L and mw[row, kk] == w[i, kk]
                    seen += 1
                else:
                    assert mt[row, kk] == -1 and mw[row, kk] == 0.0
    assert seen == n * K                      # every entry lands in exactly one row


def test_per_rank_combine_equals_per_expert_combine_on_exact_data():
    rng = np.random.default_rng(7)
    n, K, E, R, H = 12, 4, 16, 4, 8
    L = E // R
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(n)]).astype(np.int32)
    w = rng.choice(np.array([0.25, 0.5, 1.0], np.float32), (n, K))
    # per-expert outputs, small integers: every weighted sum is exact
    lay_e = oracle.layout_ht(topk, 1, E, 2, 2)
    rows_e = n * K
    Ye = rng.integers(-6, 7, (rows_e, H)).astype(np.float32)
    Ye_b = (Ye.view(np.uint32) >> 16).astype(np.uint16)
    want = oracle.combine(Ye_b, w, lay_e["row2"])
    # per-rank partial rows: the rank's weighted sum of its experts' outputs
    lay_r = oracle.layout_ht_rank(topk, 1, E, R)
    rows_r = int(lay_r["c2"].sum())
    P = np.zeros((rows_r, H), np.float32)
    for i in range(n):
        for k in range(K):
            row = lay_r["row2"][i, k]
            if row < 0:
                continue
            r = topk[i, k] // L
            for kk in range(K):
                if topk[i, kk] // L == r:
                    P[row] += w[i, kk] * Ye[lay_e["row2"][i, kk]]
    P_b = (P.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((P_b.astype(np.uint32) << 16).view(np.float32), P)
    got = oracle.combine(P_b, np.ones((n, K), np.float32), lay_r["row2"])
    np.testing.assert_array_equal(got, want)
