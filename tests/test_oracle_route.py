"""Pins for the oracle's node-limited top-k routing (CPU only).

Routing rule: "NVSHMEM and DeepEP: GPU-initiated communication", high-
throughput mode section -- score each node by the sum of its 2 best expert
scores, keep the 4 best nodes, choose the top-8 experts inside them.
"""
import itertools
import os

import numpy as np
import pytest

import ep_inputs as I
import oracle
from oracle import page_sim

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deepep_routing_study.txt")


def _golden_rows():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, *vals = line.split()
        rows[name] = [float(v) for v in vals]
    return rows


@pytest.fixture(scope="module")
def page_scores64():
    return I.page_scores(page_sim.TOKENS, page_sim.EXPERTS, 0)


@pytest.mark.parametrize("limit,key", [(0, "none"), (4, "4nodes")])
def test_page_study_numbers(page_scores64, limit, key):
    """The numpy restatement reproduces every number the page prints."""
    want = _golden_rows()[key]
    tk = page_sim.route_numpy(page_scores64, page_sim.NODES, page_sim.TOP_K, limit)
    st = page_sim.traffic(tk)
    got = [st["nodes_per_token"], st["per_expert"], st["per_gpu"], st["per_node"],
           st["ms_expert"], st["ms_gpu"], st["ms_node"]]
    assert [round(g, 2) for g in got] == want


@pytest.mark.parametrize("limit", [0, 4])
def test_c_oracle_matches_page_study(page_scores64, limit):
    """The C oracle on float32 scores picks exactly the numpy fp64 experts."""
    ref = page_sim.route_numpy(page_scores64, 8, 8, limit)
    got = oracle.route(page_scores64.astype(np.float32), 8, 8, limit)
    np.testing.assert_array_equal(got, ref)
    st = page_sim.traffic(got)
    want = _golden_rows()["4nodes" if limit else "none"]
    assert round(st["per_node"], 2) == want[3]
    assert round(st["nodes_per_token"], 2) == want[0]


def test_no_limit_is_stable_topk():
    """M = 0 reduces to a textbook top-k: numpy's stable descending argsort."""
    s = I.uniform_scores(500, 64, seed=11).astype(np.float32)
    s[::7, 3] = s[::7, 5]                       # inject ties
    got = oracle.route(s, 4, 6, 0)
    ref = np.argsort(-s, axis=1, kind="stable")[:, :6]
    np.testing.assert_array_equal(got, ref)


def _brute_route(s, nodes, k, m):
    """Enumerate node subsets and expert subsets (float64 sums, no ties)."""
    E = s.shape[0]
    per = E // nodes
    j = -(-k // m)
    node_score = []
    for n in range(nodes):
        grp = s[n * per:(n + 1) * per].astype(np.float64)
        node_score.append(max(sum(c) for c in itertools.combinations(grp, j)))
    best_nodes = max(itertools.combinations(range(nodes), m),
                     key=lambda sub: sum(node_score[n] for n in sub))
    cand = [e for e in range(E) if e // per in best_nodes]
    best_set = max(itertools.combinations(cand, k), key=lambda sub: sum(float(s[e]) for e in sub))
    return sorted(best_set, key=lambda e: -float(s[e]))


@pytest.mark.parametrize("seed,E,N,K,M", [(0, 16, 4, 4, 2), (1, 16, 4, 4, 2), (2, 16, 4, 4, 2),
                                         (3, 16, 4, 4, 2),
                                         # K not a multiple of M: ceil(K/M) terms per node score
                                         (4, 16, 4, 3, 2), (5, 24, 4, 5, 3), (6, 20, 5, 7, 3)])
def test_brute_force_tiny(seed, E, N, K, M):
    s = I.uniform_scores(40, E, seed=100 + seed).astype(np.float32)
    got = oracle.route(s, N, K, M)
    for t in range(s.shape[0]):
        assert list(got[t]) == _brute_route(s[t], N, K, M)


def test_forced_ties_follow_lower_index():
    """Scores snapped to a coarse grid: ties go to the lower node / expert index."""
    E, N, K, M = 32, 4, 4, 2
    rng = np.random.default_rng(7)
    s = (rng.integers(0, 4, size=(300, E)) * 0.25).astype(np.float32)
    got = oracle.route(s, N, K, M)
    per = E // N
    for t in range(s.shape[0]):
        row = s[t]
        ns = [sum(sorted(row[n * per:(n + 1) * per], reverse=True)[:2]) for n in range(N)]
        kept = sorted(range(N), key=lambda n: (-ns[n], n))[:M]
        cand = [e for e in range(E) if e // per in kept]
        want = sorted(cand, key=lambda e: (-row[e], e))[:K]
        assert list(got[t]) == want


def test_invariants_page_shape(page_scores64):
    s = page_scores64[:1024].astype(np.float32)
    tk = oracle.route(s, 8, 8, 4)
    for t in range(tk.shape[0]):
        row = tk[t]
        assert len(set(row.tolist())) == 8
        assert len(set((row // 32).tolist())) <= 4
        vals = s[t, row]
        assert np.all(vals[:-1] >= vals[1:])


def test_rejects_bad_config():
    s = np.zeros((2, 10), np.float32)
    with pytest.raises(ValueError):
        oracle.route(s, 3, 2, 0)          # 10 experts not divisible by 3 nodes
