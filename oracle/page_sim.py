"""The DeepEP page's routing-traffic study, restated in numpy -- TEST INFRASTRUCTURE.

Source: "NVSHMEM and DeepEP: GPU-initiated communication", section on the
high-throughput mode (node-deduplicated two-hop dispatch).  The page routes
4096 tokens held by one GPU of node 0 over 8 nodes x 8 GPUs and 256 experts
(4 per GPU), top-8, with and without the DeepSeek-V3 node limit (score each
node by the sum of its 2 best expert scores, keep 4 nodes), and reports per
token: nodes touched (own node included), and cross-node copies when sending
one copy per expert, per destination GPU, and per destination node, plus the
time those copies take on a 50 GB/s NIC at 7168 + 7168/128*4 bytes per token.

This is an independent second implementation of the routing rule (sorting
with numpy rather than the C oracle's repeated arg-max); the tests require
both to agree and to reproduce the numbers the page prints.
"""
from __future__ import annotations

import numpy as np

NODES, GPUS_PER_NODE, EXPERTS, TOP_K, MAX_NODES = 8, 8, 256, 8, 4
TOKENS, HIDDEN = 4096, 7168
TOKEN_BYTES = HIDDEN + HIDDEN // 128 * 4       # FP8 payload + one fp32 scale per 128
NIC_BYTES_PER_S = 50e9


def route_numpy(scores: np.ndarray, nodes: int, top_k: int, max_nodes: int) -> np.ndarray:
    """Node-limited top-k with stable sorts (ties to the lower index)."""
    n_tok, n_exp = scores.shape
    per_node = n_exp // nodes
    grouped = scores.reshape(n_tok, nodes, per_node)
    if 0 < max_nodes < nodes:
        take = -(-top_k // max_nodes)                       # ceil(K / M)
        best = -np.sort(-grouped, axis=2)[:, :, :take]      # largest first
        node_score = best[:, :, 0]
        for j in range(1, take):
            node_score = node_score + best[:, :, j]
        order = np.argsort(-node_score, axis=1, kind="stable")
        keep = np.zeros((n_tok, nodes), dtype=bool)
        np.put_along_axis(keep, order[:, :max_nodes], True, axis=1)
        cand = np.where(keep[:, :, None], grouped, -np.inf).reshape(n_tok, n_exp)
    else:
        cand = scores
    return np.argsort(-cand, axis=1, kind="stable")[:, :top_k].astype(np.int32)


def traffic(topk: np.ndarray, src_node: int = 0, experts_per_gpu: int = EXPERTS // (NODES * GPUS_PER_NODE),
            gpus_per_node: int = GPUS_PER_NODE) -> dict:
    """Per-token traffic statistics of one routing decision."""
    gpu = topk // experts_per_gpu
    node = gpu // gpus_per_node
    remote = node != src_node
    nodes_touched = np.array([len(np.unique(r)) for r in node])
    per_expert = remote.sum(axis=1)
    per_gpu = np.array([len(np.unique(g[m])) for g, m in zip(gpu, remote)])
    per_node = np.array([len(np.unique(n[m])) for n, m in zip(node, remote)])
    n_tok = topk.shape[0]

    def ms(copies):
        return n_tok * copies * TOKEN_BYTES / NIC_BYTES_PER_S * 1e3

    return dict(
        nodes_per_token=nodes_touched.mean(),
        per_expert=per_expert.mean(), per_gpu=per_gpu.mean(), per_node=per_node.mean(),
        ms_expert=ms(per_expert.mean()), ms_gpu=ms(per_gpu.mean()), ms_node=ms(per_node.mean()),
        cross_node_rows=int(per_node.sum()), node_rows_incl_own=int(nodes_touched.sum()))
