"""KV compressor: weighted sum -> RMSNorm -> RoPE -> paged insert (oracle; test infrastructure only).

[vLLM-V4] section 2: a c4a entry is a weighted sum of 8 raw tokens with
stride 4, a c128a entry a weighted sum of 128 raw tokens with stride 128.
[vLLM-V4] appendix, exact position ranges: combine the fixed raw group first,
then apply RoPE once at the entry's anchor position, then store.
[vLLM-V4] section 3 part 2, first fusion: the compressed K goes through
RMSNorm, then RoPE, then is inserted into the cache of the main attention or
of the indexer (separate instances per head dimension).
[vLLM-V4] section 3 part 1: each compressor keeps a rolling residual of the
last coff * ratio raw tokens per request (8 for c4a, 128 for c128a),
registered as sliding-window KV.

Readings:
* weights: one scalar per (entry, window slot), shared by all channels, equal
  to a softmax over the entry's own coff * ratio logits (logits are inputs,
  indexed by entry);
* a slot at a negative position holds the value 0 and keeps its logit;
* RMSNorm spans the whole row with epsilon an input (1e-6 in the workloads)
  and gamma an input defaulting to 1 -- parity unpinned;
* a call emits every entry whose anchor position it inserts;
* the state cache receives the new raw rows among the last coff * ratio
  positions after the call;
* when a window cache is given, every new raw row x_p is also stored there
  as RoPE_p(x_p) (the uncompressed sliding-window key/value row).
"""

from __future__ import annotations

import numpy as np

from . import formats, geometry
from .paged import PagedCache
from .rope import rope


def softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def rms_norm(y: np.ndarray, gamma: np.ndarray | None, eps: float) -> np.ndarray:
    """y / sqrt(mean(y**2) + eps) * gamma over the whole row (parity unpinned: eps and span)."""
    y = np.asarray(y, dtype=np.float64)
    n = y / np.sqrt(np.mean(y * y) + eps)
    if gamma is not None:
        n = n * np.asarray(gamma, dtype=np.float64)
    return n


def compress_entry(window_rows: np.ndarray, logits: np.ndarray, gamma, eps: float,
                   anchor: int, rope_base: float, rope_dims: int) -> np.ndarray:
    """One compressed entry from its raw window [W, d] (zeros at negative positions).

    w = softmax(logits); y = sum_r w_r x_r; n = RMSNorm(y); c = RoPE_anchor(n).
    """
    w = softmax(logits)
    y = w @ np.asarray(window_rows, dtype=np.float64)
    return rope(rms_norm(y, gamma, eps), anchor, rope_base, rope_dims)


def compress_insert(ratio: int, ctx_lens, cu_new, new_raw: np.ndarray, raw_dtype: str,
                    cu_entries, gate_logits: np.ndarray, gamma, eps: float,
                    rope_base: float, rope_dims: int,
                    state: PagedCache, out: PagedCache, swa: PagedCache | None = None):
    """Apply one compressor call to the paged caches (in place).

    Sequence b held ctx_lens[b] raw tokens before the call and receives the
    rows new_raw[cu_new[b]:cu_new[b+1]] (stored values of ``raw_dtype``) at
    positions ctx_lens[b], ctx_lens[b] + 1, ...  Its completed entries
    j = n(L_old) .. n(L_new) - 1 take the logits rows
    gate_logits[cu_entries[b] + (j - n(L_old))].

    Returns (entries, window_rows): dicts keyed by (b, j) and (b, p) holding
    the float64 values before they were rounded to the cache dtype.
    """
    W = geometry.window_len(ratio)
    raw_vals = formats.decode_stored(new_raw, raw_dtype) if len(new_raw) else np.zeros((0, out.dim))
    entries, window_rows = {}, {}
    for b in range(len(ctx_lens)):
        L_old = int(ctx_lens[b])
        rows_b = raw_vals[int(cu_new[b]):int(cu_new[b + 1])]
        L_new = L_old + len(rows_b)
        d = rows_b.shape[1] if len(rows_b) else out.dim

        def raw(p: int) -> np.ndarray:
            if p < 0:
                return np.zeros(d)
            if p >= L_old:
                return rows_b[p - L_old]
            return state.read(b, p)

        j_first = geometry.num_entries(L_old, ratio)
        j_end = geometry.num_entries(L_new, ratio)
        assert int(cu_entries[b + 1]) - int(cu_entries[b]) == j_end - j_first
        for e, j in enumerate(range(j_first, j_end)):
            s = geometry.entry_start(j, ratio)
            win = np.stack([raw(p) for p in range(s, s + W)])
            c = compress_entry(win, gate_logits[int(cu_entries[b]) + e], gamma, eps,
                               geometry.entry_anchor(j, ratio), rope_base, rope_dims)
            entries[(b, j)] = c
            out.write(b, j, c)
        # rolling residual: keep the new rows among the last W positions
        for p in range(max(L_old, L_new - W), L_new):
            state.write(b, p, rows_b[p - L_old])
        if swa is not None:
            for p in range(L_old, L_new):
                v = rope(rows_b[p - L_old], p, rope_base, rope_dims)
                window_rows[(b, p)] = v
                swa.write(b, p, v)
    return entries, window_rows
