"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and shapes them into the workloads; it holds
none of the dispatch/combine arithmetic (no routing, counting, quantisation,
packing or reduction).  Both the CPU oracle and the GPU path are fed from the
arrays returned here, so neither side ever generates inputs for the other.

Workloads follow the pages:
  * "NVSHMEM and DeepEP: GPU-initiated communication" (high-throughput mode,
    routing simulation): 8 nodes x 8 GPUs, 256 experts (4 per GPU), top-8,
    at most 4 nodes per token, 4096 tokens on one GPU of node 0, router scores
    drawn as U[0,1) per (token, expert) plus 0.5*U[0,1) per expert, seed 0.
  * "NCCL EP paper notes" (LL buffer sizing / message sizes): hidden 7168,
    128 tokens per rank, DeepSeek-V3 shapes.

Returned token tensors are bfloat16 with values ~N(0,1) rounded to nearest
even by torch's CPU cast (a library routine, not method arithmetic).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# ---------------------------------------------------------------------------
# Topologies and workload configurations
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mode: str                  # "ll" or "ht"
    num_nodes: int
    ranks_per_node: int
    num_experts: int
    top_k: int
    max_nodes: int             # 0 = no node limit
    hidden: int
    num_src_ranks: int
    tokens_per_rank: int
    payload: str               # "fp8" or "bf16"
    scores: str                # "page", "uniform", "zipf"
    weights: str               # "softmax_selected" or "softmax_normal"
    seed: int
    max_tokens_per_rank: Optional[int] = None

    @property
    def num_ranks(self) -> int:
        return self.num_nodes * self.ranks_per_node

    @property
    def num_tokens(self) -> int:
        return self.num_src_ranks * self.tokens_per_rank

    @property
    def slots(self) -> int:
        return self.max_tokens_per_rank or self.tokens_per_rank

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny dispatch+combine: 128 tokens as 4 sources x 32, hidden 256, 16 experts on
# 4 virtual ranks (2 nodes x 2), top-2, no node limit, U[0,1) scores.
TINY = Workload("tiny", "ll", 2, 2, 16, 2, 0, 256, 4, 32, "bf16", "uniform",
                "softmax_selected", seed=1)
# LL decode dispatch: 64 virtual sources x 128 tokens, 256 experts on 64 ranks.
LL_DECODE = Workload("ll_decode", "ll", 8, 8, 256, 8, 4, 7168, 64, 128, "fp8",
                     "page", "softmax_normal", seed=2)
# HT prefill dispatch: the page's routing simulation shape, seed 0.
HT_PREFILL = Workload("ht_prefill", "ht", 8, 8, 256, 8, 4, 7168, 1, 4096, "fp8",
                      "page", "softmax_normal", seed=0)
# Combine at the HT prefill geometry (32768 expert-output rows).
COMBINE = Workload("combine", "ht", 8, 8, 256, 8, 4, 7168, 1, 4096, "fp8",
                   "page", "softmax_normal", seed=4)
# Large skewed round trip: 16384 tokens, Zipf(1.1) expert popularity.
ROUND_TRIP = Workload("round_trip", "ht", 8, 8, 256, 8, 4, 7168, 1, 16384, "fp8",
                      "zipf", "softmax_normal", seed=5)

WORKLOADS = {w.name: w for w in (TINY, LL_DECODE, HT_PREFILL, COMBINE, ROUND_TRIP)}


# ---------------------------------------------------------------------------
# Router scores
# ---------------------------------------------------------------------------


def page_scores(num_tokens: int, num_experts: int, seed: int) -> np.ndarray:
    """U[0,1) per (token, expert) plus 0.5*U[0,1) per expert, float64.

    Drawn in the order the DeepEP page's simulation draws them (the token
    matrix first, then the per-expert bias) so that seed 0 at 4096 x 256 is
    the page's own input.
    """
    rng = np.random.default_rng(seed)
    base = rng.random((num_tokens, num_experts))
    bias = rng.random(num_experts) * 0.5
    return base + bias


def uniform_scores(num_tokens: int, num_experts: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.random((num_tokens, num_experts))


def zipf_bias(num_experts: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Normalised Zipf popularity r^-s / sum(r^-s) with ranks from a seeded permutation."""
    ranks = rng.permutation(num_experts) + 1
    w = ranks.astype(np.float64) ** (-s)
    return w / np.sum(np.arange(1, num_experts + 1, dtype=np.float64) ** (-s))


def zipf_scores(num_tokens: int, num_experts: int, seed: int, s: float = 1.1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    base = rng.random((num_tokens, num_experts))
    return base + zipf_bias(num_experts, s, rng)


def scores_for(w: Workload, num_tokens: Optional[int] = None) -> np.ndarray:
    """Router scores as float32 [num_tokens, num_experts] (the routed dtype)."""
    n = w.num_tokens if num_tokens is None else num_tokens
    if w.scores == "page":
        s = page_scores(n, w.num_experts, w.seed)
    elif w.scores == "uniform":
        s = uniform_scores(n, w.num_experts, w.seed)
    elif w.scores == "zipf":
        s = zipf_scores(n, w.num_experts, w.seed)
    else:
        raise ValueError(w.scores)
    return np.ascontiguousarray(s.astype(np.float32))


# ---------------------------------------------------------------------------
# Tokens, expert outputs and weights
# ---------------------------------------------------------------------------


def normal_bf16(rows: int, cols: int, seed: int) -> torch.Tensor:
    """~N(0,1) values cast to bfloat16 (torch CPU cast, round to nearest even)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def tokens_for(w: Workload, num_tokens: Optional[int] = None) -> torch.Tensor:
    n = w.num_tokens if num_tokens is None else num_tokens
    return normal_bf16(n, w.hidden, w.seed + 1000)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw uint16 bit patterns of a CPU bfloat16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def softmax_fp32(logits: np.ndarray) -> np.ndarray:
    """Row softmax in float64, then cast to float32 (used to draw weights)."""
    z = logits.astype(np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def normal_weights(num_tokens: int, top_k: int, seed: int) -> np.ndarray:
    """Softmax over top-k logits drawn ~N(0,1)."""
    rng = np.random.default_rng(seed + 2000)
    return np.ascontiguousarray(softmax_fp32(rng.standard_normal((num_tokens, top_k))))


def selected_score_weights(scores: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """Softmax over each token's selected router scores (the tiny workload)."""
    picked = np.take_along_axis(scores.astype(np.float64), topk_idx.astype(np.int64), axis=1)
    return np.ascontiguousarray(softmax_fp32(picked))


def weights_for(w: Workload, scores: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    if w.weights == "softmax_selected":
        return selected_score_weights(scores, topk_idx)
    return normal_weights(topk_idx.shape[0], w.top_k, w.seed)


def random_topk(num_tokens: int, num_experts: int, top_k: int, seed: int) -> np.ndarray:
    """Distinct random experts per token (for layout tests independent of routing)."""
    rng = np.random.default_rng(seed)
    keys = rng.random((num_tokens, num_experts))
    return np.ascontiguousarray(np.argsort(keys, axis=1)[:, :top_k].astype(np.int32))
