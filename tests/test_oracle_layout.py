"""Pins for the oracle's counts, prefix sums and slot/row maps (CPU only).

Fixed slots per (local expert, source rank) for the low-latency mode and the
node-deduplicated, same-position two-hop layout for the high-throughput mode:
"NVSHMEM and DeepEP: GPU-initiated communication" (low-latency and high-
throughput sections); HT output rows grouped by expert with per-expert counts
in a deterministic order: "NCCL EP paper notes" (tensor layouts).
"""
import os

import numpy as np
import pytest

import ep_inputs as I
import oracle
from oracle import page_sim

SIZES = os.path.join(os.path.dirname(__file__), "golden", "ll_buffer_sizing.txt")


def _sizes():
    d = {}
    for line in open(SIZES):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()
        d[k] = float(v)
    return d


def test_message_sizes_closed_form():
    g = _sizes()
    H = 7168
    assert oracle.row_bytes(H, True) + 16 == g["ll_msg_fp8_bytes"]
    assert oracle.row_bytes(H, False) + 16 == g["ll_msg_bf16_bytes"]
    assert oracle.row_bytes(H, False) == g["combine_msg_bf16_bytes"]
    assert oracle.row_bytes(H, True) == g["ht_token_fp8_bytes"]
    msg = oracle.row_bytes(H, True) + 16
    assert round(4 * 64 * 128 * msg / 2**20) == g["ll_recv_mib_rounded"]
    assert round(8 * 32 * 64 * msg / 1e6) == g["exercise_mb_batch64"]
    assert round(8 * 32 * 256 * msg / 1e6) == g["exercise_mb_batch256"]


def test_ll_occupancy_matches_page():
    """One source's 128 tokens x top-8 fill K/E of a rank's reserved slots."""
    g = _sizes()
    w = I.LL_DECODE
    topk = oracle.route(I.scores_for(w, 128), 8, 8, 4)
    counts, slot_map, err = oracle.layout_ll(topk, 1, 256, 128)
    assert err == 0 and counts.sum() == 128 * 8
    msg = oracle.row_bytes(7168, True) + 16
    used_per_rank_mib = counts.sum() * 64 / 64 * msg / 2**20     # 64 sources, spread evenly
    assert round(used_per_rank_mib, 1) == g["ll_used_mib_1dp"]
    assert counts.sum() / (256 * 128) == 8 / 256


def _brute_ll(topk, S, E, slots):
    n, K = topk.shape
    T = n // S
    want = np.full((n, K), -1, np.int32)
    for i in range(n):
        s = i // T
        for k in range(K):
            e = topk[i, k]
            if e < 0 or e >= E or e in topk[i, :k]:
                continue
            earlier = 0
            for i2 in range(s * T, i + 1):
                for k2 in range(K if i2 < i else k):
                    e2 = topk[i2, k2]
                    if e2 == e and not (e2 in topk[i2, :k2]):
                        earlier += 1
            want[i, k] = (e * S + s) * slots + earlier
    return want


def test_ll_brute_force_tiny():
    S, T, K, E, slots = 3, 20, 3, 8, 24
    topk = I.random_topk(S * T, E, K, seed=31)
    topk[5, 1] = -1
    topk[7, 2] = topk[7, 0]           # duplicate
    topk[9, 0] = E                    # out of range
    counts, slot_map, err = oracle.layout_ll(topk, S, E, slots)
    np.testing.assert_array_equal(slot_map, _brute_ll(topk, S, E, slots))
    assert err == oracle.ERR_BAD_INDEX | oracle.ERR_DUP_INDEX
    valid = slot_map >= 0
    assert counts.sum() == valid.sum() == S * T * K - 3
    # bijection onto the first counts[e, s] slots of every (e, s)
    used = np.sort(slot_map[valid])
    assert len(np.unique(used)) == len(used)
    expect = np.concatenate([(e * S + s) * slots + np.arange(counts[e, s])
                             for e in range(E) for s in range(S)])
    np.testing.assert_array_equal(used, np.sort(expect))


def test_ll_capacity_error():
    topk = np.zeros((5, 1), np.int32)          # 5 tokens of one source, same expert
    with pytest.raises(ValueError):
        oracle.layout_ll(topk, 1, 4, 4)


def _brute_ht(topk, S, E, N, G):
    n, K = topk.shape
    T = n // S
    per_node = E // N
    R = N * G

    def valid(i, k):
        e = topk[i, k]
        return 0 <= e < E and e not in topk[i, :k]

    def nodes_of(i):
        return sorted({topk[i, k] // per_node for k in range(K) if valid(i, k)})

    c1 = np.zeros(R, np.int64)
    for i in range(n):
        for nd in nodes_of(i):
            c1[nd * G + (i // T) % G] += 1
    node_row = np.full((n, N), -1, np.int64)
    for i in range(n):
        s = i // T
        for nd in nodes_of(i):
            d = nd * G + s % G
            before = sum(c1[:d])
            earlier = sum(1 for i2 in range(i) if (i2 // T) % G == s % G and nd in nodes_of(i2))
            node_row[i, nd] = before + earlier
    c2 = np.zeros(E, np.int64)
    for i in range(n):
        for k in range(K):
            if valid(i, k):
                c2[topk[i, k]] += 1
    row2 = np.full((n, K), -1, np.int64)
    for i in range(n):
        for k in range(K):
            if not valid(i, k):
                continue
            e = topk[i, k]
            earlier = sum(1 for i2 in range(i) for k2 in range(K)
                          if valid(i2, k2) and topk[i2, k2] == e)
            row2[i, k] = sum(c2[:e]) + earlier
    return c1, node_row, c2, row2


@pytest.mark.parametrize("S", [1, 3])
def test_ht_brute_force_tiny(S):
    E, N, G, K, T = 16, 4, 2, 3, 15
    topk = I.random_topk(S * T, E, K, seed=40 + S)
    topk[2, 2] = -3
    d = oracle.layout_ht(topk, S, E, N, G)
    c1, node_row, c2, row2 = _brute_ht(topk, S, E, N, G)
    np.testing.assert_array_equal(d["c1"], c1)
    np.testing.assert_array_equal(d["node_row"], node_row)
    np.testing.assert_array_equal(d["c2"], c2)
    np.testing.assert_array_equal(d["row2"], row2)
    assert d["err"] == oracle.ERR_BAD_INDEX
    np.testing.assert_array_equal(d["off1"], np.concatenate([[0], np.cumsum(c1)[:-1]]))
    np.testing.assert_array_equal(d["off2"], np.concatenate([[0], np.cumsum(c2)[:-1]]))


def test_ht_page_shape_counts():
    """Page-3 shape: cross-node stage-1 rows per token round to 3.36 (and 3.97
    including the own node); stage-2 rows = tokens x top-8."""
    s = I.page_scores(4096, 256, 0).astype(np.float32)
    topk = oracle.route(s, 8, 8, 4)
    d = oracle.layout_ht(topk, 1, 256, 8, 8)
    c1 = d["c1"]
    own_node = c1[:8].sum()
    assert round((c1.sum() - own_node) / 4096, 2) == 3.36
    assert round(c1.sum() / 4096, 2) == 3.97
    assert d["c2"].sum() == 4096 * 8
    # only same-position ranks (rail 0) receive stage-1 rows from source rank 0
    assert np.all(c1.reshape(8, 8)[:, 1:] == 0)
    st = page_sim.traffic(topk)
    assert (c1.sum() - own_node) == st["cross_node_rows"]
    # stage-2 rows grouped by expert; a rank's rows are its 4 experts' rows
    for r in range(64):
        assert d["c2"][4 * r:4 * r + 4].sum() == (topk // 4 == r).sum()


def test_ht_rows_are_bijections():
    w = I.ROUND_TRIP
    topk = oracle.route(I.scores_for(w, 2048), 8, 8, 4)
    d = oracle.layout_ht(topk, 1, 256, 8, 8)
    nr = d["node_row"][d["node_row"] >= 0]
    assert np.array_equal(np.sort(nr), np.arange(d["c1"].sum()))
    r2 = d["row2"][d["row2"] >= 0]
    assert np.array_equal(np.sort(r2), np.arange(2048 * 8))
    # deterministic order inside each expert: rows ascend with the token index
    for e in range(256):
        tok, k = np.nonzero(topk == e)
        rows = d["row2"][tok, k]
        assert np.all(np.diff(rows) == 1) and np.all(np.diff(tok) > 0)


def test_pack_roundtrip_headers():
    S, T, K, E, H, slots = 2, 6, 2, 8, 256, 8
    topk = I.random_topk(S * T, E, K, seed=50)
    x = I.bf16_bits(I.normal_bf16(S * T, H, seed=51))
    counts, slot_map, _ = oracle.layout_ll(topk, S, E, slots)
    buf = oracle.pack_ll(x, T, K, True, slot_map, E * S * slots)
    rows = oracle.token_rows(x, True)
    rb = rows.shape[1]
    for i in range(S * T):
        for k in range(K):
            m = buf[slot_map[i, k]]
            np.testing.assert_array_equal(m[:rb], rows[i])
            assert list(m[rb:].view(np.int32)) == [i % T, i // T, k, 0]


@pytest.mark.parametrize("S", [1, 3])
def test_ht_pack_rows_and_metadata_roundtrip(S):
    """Every HT row holds the image of the token its map entry names, and its
    metadata names that entry back: stage 1 (token, source, the token's
    top-k and weights) at node_row(i, n); stage 2 (source, token, k) at
    row2(i, k).  Rows no entry names do not exist (the counts are exact)."""
    T, K, E, N, G, H = 40, 4, 32, 4, 2, 256
    topk = I.random_topk(S * T, E, K, seed=60 + S)
    topk[5, 1] = topk[5, 0]                       # a repeated entry: no row
    w = np.random.default_rng(61).random((S * T, K)).astype(np.float32)
    x = I.bf16_bits(I.normal_bf16(S * T, H, seed=62))
    lay = oracle.layout_ht(topk, S, E, N, G)
    rows1, rows2 = int(lay["c1"].sum()), int(lay["c2"].sum())
    pk = oracle.pack_ht(x, topk, w, T, N, True, lay["node_row"], lay["row2"], rows1, rows2)
    img = oracle.token_rows(x, True)
    seen1, seen2 = set(), set()
    for i in range(S * T):
        s, t = divmod(i, T)
        for n in range(N):
            r = lay["node_row"][i, n]
            if r < 0:
                continue
            seen1.add(int(r))
            np.testing.assert_array_equal(pk["stage1"][r], img[i])
            assert pk["meta1_tok"][r] == t and pk["meta1_src"][r] == s
            np.testing.assert_array_equal(pk["meta1_topk"][r], topk[i])
            np.testing.assert_array_equal(pk["meta1_w"][r], w[i])
        for k in range(K):
            r = lay["row2"][i, k]
            if r < 0:
                continue
            seen2.add(int(r))
            np.testing.assert_array_equal(pk["stage2"][r], img[i])
            assert (pk["meta2_src"][r], pk["meta2_tok"][r], pk["meta2_k"][r]) == (s, t, k)
    assert seen1 == set(range(rows1)) and seen2 == set(range(rows2))
    assert lay["row2"][5, 1] == -1
