"""Run the CPU oracle on one step's generator inputs, and compare GPU results with it.

Test infrastructure: imports only ``oracle`` and the generator's CPU tensors.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import attention, compress, formats, geometry, indexer
from oracle.paged import PagedCache
from oracle.rope import inverse_rope

DT = {torch.float32: "f32", torch.bfloat16: "bf16", torch.uint8: "fp8"}


def np_rows(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def cache_fmt(rows: torch.Tensor, scales) -> str:
    """Stored format of a cache's rows: uint8 rows with uint8 (E8M0) scales are fp4."""
    if rows.dtype == torch.uint8 and scales is not None and scales.dtype == torch.uint8:
        return "fp4"
    return DT[rows.dtype]


def oracle_cache(triple) -> PagedCache:
    rows, scales, bt = triple
    return PagedCache(np_rows(rows), cache_fmt(rows, scales), bt.numpy().copy(),
                      None if scales is None else scales.numpy().copy())


def raw_values(t: torch.Tensor) -> tuple[np.ndarray, str]:
    return np_rows(t), DT[t.dtype]


def prepare(d: dict) -> dict:
    """Oracle copies of the step's caches (input preparation, not part of the step)."""
    c = {name: oracle_cache(d[name]) for name in ("kv", "swa", "state", "idx", "idx_state") if name in d}
    return c


def run_oracle(cfg, d: dict, queries=None, topk_override=None, caches: dict | None = None) -> dict:
    """The step on the oracle.  ``queries``: indices of the queries to evaluate (default all).
    ``caches``: the result of prepare(d) (made here when not given); they are updated in place."""
    res: dict = {}
    caches = prepare(d) if caches is None else caches
    kv, swa, state = caches["kv"], caches["swa"], caches["state"]
    idx = caches.get("idx")
    gamma = None if d.get("gamma") is None else d["gamma"].numpy().astype(np.float64)
    if "compress" in cfg.stages:
        raw, rdt = raw_values(d["new_raw"])
        ent, win = compress.compress_insert(
            cfg.ratio, d["ctx_lens"].tolist(), d["cu_new"].tolist(), raw, rdt, d["cu_entries"].tolist(),
            d["logits"].numpy(), gamma, cfg.eps, cfg.rope_base, 64, state, kv, swa)
        res["entries"], res["window_rows"] = ent, win
    if "compress_idx" in cfg.stages:
        raw, rdt = raw_values(d["new_idx_raw"])
        idx_state = caches["idx_state"]
        ent, _ = compress.compress_insert(
            4, d["ctx_lens"].tolist(), d["cu_new"].tolist(), raw, rdt, d["cu_entries"].tolist(),
            d["idx_logits"].numpy(), None, cfg.eps, cfg.rope_base, 64, idx_state, idx, None)
        res["idx_entries"] = ent
        res["idx_state"] = idx_state
    res["kv"], res["swa"], res["state"], res["idx"] = kv, swa, state, idx

    cu_q = d["cu_q"].tolist()
    q_pos = d["q_pos"].tolist()
    total_q = len(q_pos)
    qsel = list(range(total_q)) if queries is None else list(queries)
    seq = np.searchsorted(np.array(cu_q), np.arange(total_q), side="right") - 1
    q = formats.decode_stored(np_rows(d["q"]), DT[d["q"].dtype])
    res["queries"] = qsel
    res["topk"], res["scores"], res["out"], res["lse"] = {}, {}, {}, {}
    if "index" in cfg.stages:
        q_idx = formats.decode_stored(np_rows(d["q_idx"]), DT[d["q_idx"].dtype])
        w = d["head_w"].numpy().astype(np.float64)
        for i in qsel:
            s = indexer.query_scores(idx, int(seq[i]), q_pos[i], q_idx[i], w[i])
            res["scores"][i] = s
            res["topk"][i] = indexer.topk(s, cfg.k)
    for i in qsel:
        if "attn" not in cfg.stages:
            break
        if topk_override is not None:
            ids = topk_override[i]
        elif "index" in cfg.stages:
            ids = res["topk"][i]
        else:
            ids = None if "topk" not in d else d["topk"][i].numpy()
        res["out"][i], res["lse"][i] = _attend(cfg, d, kv, swa, int(seq[i]), q_pos[i], q[i], ids)
    return res


def _attend(cfg, d, kv, swa, b, t, q_i, ids):
    rows = attention.gather_rows(kv, swa, b, t, cfg.ratio, ids, cfg.window)
    o, l = attention.attend(q_i, rows, cfg.softmax_scale)
    return inverse_rope(o, t, cfg.rope_base, 64), l


def attend_query(cfg, d: dict, res: dict, i: int, ids):
    """Oracle attention of query i over the entry list ``ids`` (caches as left by run_oracle)."""
    cu_q = d["cu_q"].tolist()
    b = int(np.searchsorted(np.array(cu_q), i, side="right") - 1)
    q = formats.decode_stored(np_rows(d["q"][i]), DT[d["q"].dtype])
    return _attend(cfg, d, res["kv"], res["swa"], b, int(d["q_pos"][i]), q, ids)


# ------------------------------------------------------------------ comparisons

def half_ulp_bf16(c: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(c), 2.0 ** -126)
    e = np.floor(np.log2(a))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def half_ulp_fp8(c: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(c), 2.0 ** -6)
    e = np.floor(np.log2(a))
    return np.ldexp(1.0, (e - 4).astype(np.int64))


def check_rounded_row(gpu_vals: np.ndarray, exact: np.ndarray, fmt: str, gpu_scale=None, ref_scale=None):
    """A stored row is acceptable if every element is a rounding of a value within delta of the
    exact one: |stored - exact| <= half an ulp of exact + delta, where
    delta = 1e-5 |exact| + 1e-6 max|row| is the float32 accuracy of the fused kernel (errors of
    float32 arithmetic scale with the row's magnitude, not with an element that cancels to
    nearly zero).  fp8 rows are compared in code units; their scales must agree to 1e-6."""
    if fmt == "fp8":
        assert gpu_scale is not None and ref_scale is not None
        ok_s = abs(float(gpu_scale) - float(ref_scale)) <= 1e-6 * abs(float(ref_scale))
        vals = gpu_vals / float(gpu_scale)
        c = exact / float(ref_scale)
        half = half_ulp_fp8(c)
    else:
        ok_s = True
        vals, c = gpu_vals, exact
        half = half_ulp_bf16(c) if fmt == "bf16" else np.zeros_like(c)
    delta = 1e-5 * np.abs(c) + 1e-6 * float(np.max(np.abs(c)))
    err = np.abs(vals - c)
    tol = half + delta + 1e-30
    return bool(ok_s and np.all(err <= tol)), float(np.max(err / tol))


def check_fp4_row(packed: np.ndarray, sbytes: np.ndarray, exact: np.ndarray):
    """A stored fp4 row (packed bytes [d/2], E8M0 bytes [d/16]) against the exact row [d].

    Per block of 16 values, with the float32 accuracy of the kernel
    delta = 1e-5 |exact| + 1e-6 max|row| (as in check_rounded_row):
    * the scale 2^k is the smallest power of two with amax / 2^k <= 6, up to delta on amax
      (an all-zero block has k = 0);
    * every code is a rounding, at scale 2^k, of a value within delta of the exact one: within
      half the E2M1 spacing at that magnitude (0.25 below 2, 0.5 below 4, 1 up to 6).
    Returns (ok, worst err/tol)."""
    exact = np.asarray(exact, dtype=np.float64)
    d = exact.size
    blocks = exact.reshape(d // 16, 16)
    k = np.asarray(sbytes, dtype=np.int64) - 127
    amax = np.max(np.abs(blocks), axis=1)
    row_max = float(np.max(amax)) if amax.size else 0.0
    tiny = 1e-5 * amax + 1e-6 * row_max
    top = 6.0 * np.ldexp(1.0, k)
    ok_s = np.where(amax > 0, (amax - tiny <= top) & (amax + tiny > top / 2), k == 0)
    sc = np.ldexp(1.0, k)[:, None]
    vals = formats.fp4_unpack(packed, sbytes).reshape(d // 16, 16) / sc
    c = blocks / sc
    a = np.abs(c)
    half = np.where(a < 2.0, 0.25, np.where(a < 4.0, 0.5, 1.0))
    delta = (1e-5 * np.abs(blocks) + 1e-6 * row_max) / sc
    ratio = np.abs(vals - c) / (half + delta)
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return bool(np.all(ok_s) and np.all(ratio <= 1.0)), (worst if np.all(ok_s) else 1e9)


def topk_acceptable(gpu_ids: np.ndarray, scores: np.ndarray, k: int, rel: float = 1e-5):
    """R11: |G| = k', every id scoring above tau(1+rel) is in G, every id in G scores >= tau(1-rel).
    Also checks the output form: ascending ids, no duplicates, -1 padding."""
    n = len(scores)
    kk = min(k, n)
    g = gpu_ids[gpu_ids >= 0]
    if len(g) != kk or np.any(gpu_ids[kk:] != -1) or np.any(gpu_ids[:kk] < 0):
        return False, "size/padding"
    if len(np.unique(g)) != kk or np.any(np.diff(g) <= 0):
        return False, "not strictly ascending"
    if np.any(g >= n):
        return False, "non-causal id"
    if kk == 0:
        return True, "empty"
    tau = np.sort(scores)[::-1][kk - 1]
    band = rel * max(abs(float(tau)), 1e-30)
    must = np.nonzero(scores > tau + band)[0]
    if not np.all(np.isin(must, g)):
        return False, "missing a clear winner"
    if np.any(scores[g] < tau - band):
        return False, "contains a clear loser"
    return True, "ok"


def allclose_out(gpu: np.ndarray, ref: np.ndarray, atol: float = 1e-5, rtol: float = 2e-3):
    """|gpu - ref| <= atol + rtol |ref| elementwise; equal values (e.g. both -inf for the lse of a
    query without rows) pass, an infinity on one side only fails."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    same = gpu == ref
    with np.errstate(invalid="ignore"):
        err = np.where(same, 0.0, np.abs(gpu - ref))
        tol = atol + rtol * np.where(np.isfinite(ref), np.abs(ref), 0.0)
    ratio = np.where(np.isnan(err), np.inf, err / tol)
    return bool(np.all(ratio <= 1.0)), float(np.max(ratio)) if ratio.size else 0.0


def decode_gpu_rows(rows: torch.Tensor, scales, blocks_slots):
    """Stored values of the given (block, slot) rows of a GPU cache copied to CPU."""
    r = rows.cpu()
    dt = cache_fmt(r, scales)
    blk, slot = blocks_slots
    vals = np_rows(r[blk, slot])
    sc = None if scales is None else scales.cpu().numpy()[blk, slot]
    return formats.decode_stored(vals, dt, sc if dt in ("fp8", "fp4") else None), sc


__all__ = ["run_oracle", "check_rounded_row", "check_fp4_row", "cache_fmt", "topk_acceptable", "allclose_out", "geometry"]
