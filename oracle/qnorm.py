"""Query normalisation + RoPE, and the window-key RoPE + insert (oracle; test infrastructure only).

[vLLM-V4] section 3 part 2, third fusion: before the main attention, what is left after the
compressor is elementwise work on the queries and on the uncompressed sliding-window keys;
one kernel does it, each warp taking one query head or one key head on its own.  The pages
name the operations (query normalisation, KV RoPE, K insert) and nothing more.

Readings (parity unpinned where the pages are silent):
* query normalisation: RMSNorm of each query head over its d dimensions, with eps and a
  gain gamma[d] shared by the heads as inputs (gamma defaults to 1) -- the same RMSNorm the
  compressor applies to an entry (oracle.compress.rms_norm);
* then RoPE at the query's own position t on the last rope_dims dimensions (consecutive
  pairs): the rotation every key stored for position t carries (oracle.rope);
* the query leaves in the dtype it came in (bf16 in the workloads: the attention's input);
* the window keys are RoPE_p(x_p) of the new raw rows, stored into the window cache at their
  positions; no norm (the raw rows come normalised from the projection).  These are the rows
  the compressor's optional window output writes; here they are produced beside the queries.
"""

from __future__ import annotations

import numpy as np

from . import formats
from .compress import rms_norm
from .paged import PagedCache
from .rope import rope


def q_norm_rope(q: np.ndarray, gamma, eps: float, pos: int, rope_base: float,
                rope_dims: int) -> np.ndarray:
    """One query's heads [H, d]: each head RMS-normalised (times gamma), then RoPE at pos."""
    q = np.asarray(q, dtype=np.float64)
    n = np.stack([rms_norm(q[h], gamma, eps) for h in range(q.shape[0])])
    return rope(n, pos, rope_base, rope_dims)


def window_keys(ctx_lens, cu_new, new_raw: np.ndarray, raw_dtype: str, rope_base: float,
                rope_dims: int, swa: PagedCache) -> dict:
    """Store RoPE_p(x_p) for every new raw row of every sequence into the window cache.

    Sequence b held ctx_lens[b] raw tokens and receives new_raw[cu_new[b]:cu_new[b+1]] at
    positions ctx_lens[b], ctx_lens[b] + 1, ...  Returns the float64 rows keyed by (b, p).
    """
    vals = formats.decode_stored(new_raw, raw_dtype) if len(new_raw) else np.zeros((0, swa.dim))
    rows = {}
    for b in range(len(ctx_lens)):
        for r in range(int(cu_new[b]), int(cu_new[b + 1])):
            p = int(ctx_lens[b]) + (r - int(cu_new[b]))
            v = rope(vals[r], p, rope_base, rope_dims)
            rows[(b, p)] = v
            swa.write(b, p, v)
    return rows


def q_norm_rope_swa(q_pos, q: np.ndarray, q_dtype: str, gamma, eps: float, rope_base: float,
                    rope_dims: int, ctx_lens=None, cu_new=None, new_raw=None,
                    raw_dtype: str = "bf16", swa: PagedCache | None = None):
    """The fused call: every query's heads normalised and rotated, and (when a window cache is
    given) every new raw row's window key stored.

    q: stored values [total_q, H, d] of q_dtype; returns (q_out float64 [total_q, H, d] before
    rounding to q_dtype, window rows dict).
    """
    qv = formats.decode_stored(q, q_dtype) if q.size else np.zeros(q.shape)
    out = np.zeros(qv.shape)
    for i in range(qv.shape[0]):
        out[i] = q_norm_rope(qv[i], gamma, eps, int(q_pos[i]), rope_base, rope_dims)
    rows = {}
    if swa is not None:
        rows = window_keys(ctx_lens, cu_new, new_raw, raw_dtype, rope_base, rope_dims, swa)
    return out, rows
