"""Indexer scores and top-k selection over c4a entries (oracle; test infrastructure only).

[vLLM-V4] section 2 (DeepSeek Sparse Attention): even after c4a compression
a 1M-token sequence has about 250K compressed entries, so each query attends
only to the top-k of them.  [vLLM-V4] appendix, exact k values: k = 512 by
default for c4a (2048 in DeepSeek V3.2, 8192 for c128a).  [vLLM-V4]
appendix, causality: a query at position t may only use entries with
anchor 4j + 3 <= t.  [SGLang-pools] section 4: one indexer key per entry,
128 fp8 values plus one float32 scale (132 bytes).

Reading of the score (the pages cite DSA but print no formula): for query
position t, indexer heads h with weights w_h and queries q_h,
    s_j = sum_h w_h * max(0, q_h . k_j)
where k_j is the dequantized key row; no extra scale.

Reading of the selection: candidates are the causal entries J; the first
k' = min(k, |J|) entries in the order (score descending, entry index
ascending) are selected; the output is padded with -1 to k.
"""

from __future__ import annotations

import numpy as np

from . import geometry
from .paged import PagedCache


def scores(q_idx: np.ndarray, head_w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """s_j = sum_h w_h relu(q_h . k_j) for keys [n, d] and queries [H, d]; float64 [n]."""
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    dots = k @ q.T                                   # [n, H]
    return np.maximum(dots, 0.0) @ np.asarray(head_w, dtype=np.float64)


def query_scores(idx_cache: PagedCache, b: int, t: int, q_idx, head_w) -> np.ndarray:
    """Scores of every causal c4a entry j < n(t + 1) of sequence b for a query at t."""
    n = geometry.visible_entries(t, 4)
    if n == 0:
        return np.zeros(0)
    return scores(q_idx, head_w, idx_cache.read(b, np.arange(n)))


def topk(s: np.ndarray, k: int) -> np.ndarray:
    """Entry ids of the k' = min(k, n) best scores, ties to the lower id, padded with -1 to k."""
    n = len(s)
    order = np.lexsort((np.arange(n), -np.asarray(s, dtype=np.float64)))
    out = np.full(k, -1, dtype=np.int64)
    kk = min(k, n)
    out[:kk] = order[:kk]
    return out
