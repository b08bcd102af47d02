"""Sparse MQA with K = V over top-k entries plus a sliding window, then inverse RoPE.

Oracle; test infrastructure only.

[vLLM-V4] section 2: keys and values are shared (one row serves both), the
query attends only to the top-k compressed tokens, and a window of 128
uncompressed tokens keeps local detail.  [vLLM-V4] appendix, why the short
window: a query at m sees the uncompressed tokens [m - 127, m].  [vLLM-V4]
appendix, why inverse RoPE: with v_n = k_n = R_n k the output carries R_n,
so it is multiplied by R_m^{-1}: out = sum softmax(q_m . k_n) R_{n-m} k.
[vLLM-V4] appendix, exact k values: c128a attends to all of its (at most
8192) entries, framed as top-k with k = 8192.

Readings:
* the row set is {c_j : j in the top-k list} union {v_p : t-W+1 <= p <= t,
  p >= 0}; no entry is dropped for overlapping the window;
* list entries outside [0, n(t + 1)) are padding and are skipped;
* logits are softmax_scale * q_h . row over the whole stored row, and the
  output is the full row width (latent and RoPE dimensions alike);
* the inverse rotation is applied at the query position t;
* lse = log(sum exp(logits)) in natural log (minus infinity for no rows).
"""

from __future__ import annotations

import numpy as np

from . import formats, geometry
from .paged import PagedCache
from .rope import inverse_rope


def attend(q: np.ndarray, rows: np.ndarray, softmax_scale: float):
    """Softmax attention with the same rows as keys and values.

    q: [H, d]; rows: [N, d].  Returns (o [H, d], lse [H]).
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    if len(rows) == 0:
        return np.zeros((H, d)), np.full(H, -np.inf)
    z = softmax_scale * (q @ rows.T)                       # [H, N]
    m = np.max(z, axis=1, keepdims=True)
    p = np.exp(z - m)
    l = np.sum(p, axis=1, keepdims=True)
    o = (p / l) @ rows
    return o, (m + np.log(l))[:, 0]


def gather_rows(kv: PagedCache, swa: PagedCache, b: int, t: int, ratio: int,
                topk_ids, window: int) -> np.ndarray:
    """Rows a query at position t of sequence b attends to, in list order."""
    n_vis = geometry.visible_entries(t, ratio)
    if topk_ids is None:
        ent = np.arange(n_vis)
    else:
        ids = np.asarray(topk_ids, dtype=np.int64)
        ent = ids[(ids >= 0) & (ids < n_vis)]
    parts = []
    if len(ent):
        parts.append(kv.read(b, ent))
    p0 = max(0, t - window + 1)
    if t >= p0 and window > 0:
        parts.append(swa.read(b, np.arange(p0, t + 1)))
    return np.concatenate(parts) if parts else np.zeros((0, kv.dim))


def sparse_attn_decode(cu_q, q_pos, q: np.ndarray, kv: PagedCache, ratio: int, topk_ids,
                       swa: PagedCache, window: int, softmax_scale: float,
                       rope_base: float, rope_dims: int):
    """out [total_q, H, d] = R_t^{-1} attention(q, rows, rows) per query; also lse [total_q, H]."""
    total_q, H, d = q.shape
    out = np.zeros((total_q, H, d))
    lse = np.zeros((total_q, H))
    for b in range(len(cu_q) - 1):
        for i in range(int(cu_q[b]), int(cu_q[b + 1])):
            t = int(q_pos[i])
            rows = gather_rows(kv, swa, b, t, ratio, None if topk_ids is None else topk_ids[i], window)
            o, l = attend(q[i], rows, softmax_scale)
            out[i] = inverse_rope(o, t, rope_base, rope_dims)
            lse[i] = l
    return out, lse


def output_fp8(out: np.ndarray):
    """The output rows as fp8 for the output projection ([vLLM-V4] section 3 part 2, second
    fusion: inverse RoPE, then fp8 quantisation).  Reading (the pages give no layout): each
    (query, head) row is quantised like an fp8 cache row (formats.fp8_quantize_row: one float32
    scale amax/448 per row, nearest-even saturating E4M3 codes of row / scale).

    out [..., d] float64 -> (codes [..., d] uint8, scales [...] float32).
    """
    out = np.asarray(out, dtype=np.float64)
    flat = out.reshape(-1, out.shape[-1])
    codes = np.zeros(flat.shape, dtype=np.uint8)
    scales = np.zeros(flat.shape[0], dtype=np.float32)
    for r in range(flat.shape[0]):
        codes[r], scales[r] = formats.fp8_quantize_row(flat[r])
    return codes.reshape(out.shape), scales.reshape(out.shape[:-1])
