"""End-to-end parity of one step: the HIP library against the CPU oracle on the same inputs.

Used by the GPU tests and by the smoke check.  Every comparison follows the acceptance rules
of the method's definition:
* stored cache rows (compressed entries, window rows) must round a value within
  delta = 1e-5 |exact| + 1e-6 max|row| of the oracle's exact value (the float32 accuracy of
  the fused kernel); fp8 scales must agree to 1e-6; state rows are bit-exact copies;
* top-k sets must match except where scores are within 1e-5 relative of the k-th score;
  the GPU's reported scores must agree with the oracle's to 1e-5 relative;
* attention outputs must satisfy |gpu - oracle| <= 1e-5 + 2e-3 |oracle| elementwise; a
  query whose GPU top-k set differs from the oracle's (a near tie) is only checked for
  its top-k, since its row set differs.
"""

from __future__ import annotations

import copy

import numpy as np
import torch

from tests import oracle_step as O
from workloads import configs, inputs

SMALL_DECODE = configs.scaled(configs.C4A_1M_B4_FP8, (9220, 4099, 2562, 2049), k=256, n_heads=128,
                              name_suffix="smoke")


def _rows_at(cache_cpu, bt: torch.Tensor, b: int, r: int):
    rows, scales = cache_cpu
    rpb = rows.shape[1]
    blk, slot = int(bt[b, r // rpb]), r % rpb
    v = O.np_rows(rows[blk, slot])
    dt = O.DT[rows.dtype]
    sc = None if scales is None else float(scales[blk, slot])
    return O.formats.decode_stored(v, dt, None if sc is None else np.float32(sc)), sc


def _oracle_scale(ocache, b, r):
    blk, slot = ocache.locate(b, r)
    return None if ocache.scales is None else float(ocache.scales[blk, slot])


def _with_gpu_rows(ocache, gpu_cache, slots):
    """A copy of an oracle cache that holds the GPU's stored rows at the (block, slot) pairs
    ``slots`` (rows the step wrote and that passed their rounding check)."""
    rows, scales = gpu_cache
    c = copy.copy(ocache)
    c.rows = ocache.rows.copy()
    c.scales = None if ocache.scales is None else ocache.scales.copy()
    for blk, slot in slots:
        c.rows[blk, slot] = O.np_rows(rows[blk, slot])
        if c.scales is not None:
            c.scales[blk, slot] = scales[blk, slot].numpy()
    return c


def compare(cfg, d: dict, step, ores: dict) -> dict:
    """Check every output of the step.  Stored rows are checked against the oracle's exact
    values with the rounding allowance of tests/oracle_step.check_rounded_row; attention is then
    checked against the oracle run on the rows the GPU stored (each stage on the GPU's own
    inputs), because a value within float32 accuracy of a rounding midpoint may be rounded
    either way and one code of a dominant window row moves the output by more than the
    attention tolerance."""
    rep = {"fail": [], "checked": {}, "worst": {}}
    stored = {"kv": [], "swa": []}  # (block, slot) of the written rows that passed

    def note(kind, ok, ratio, where):
        rep["checked"][kind] = rep["checked"].get(kind, 0) + 1
        rep["worst"][kind] = max(rep["worst"].get(kind, 0.0), ratio)
        if not ok:
            rep["fail"].append(f"{kind} {where} (err/tol {ratio:.3g})")

    g = step.g

    def cpu_cache(name):
        c = g[name]
        return c.rows.cpu(), None if c.scales is None else c.scales.cpu()

    if "compress" in cfg.stages:
        kv = cpu_cache("kv")
        fmt = cfg.kv_dtype
        for (b, j), c in ores["entries"].items():
            gv, gs = _rows_at(kv, d["kv"][2], b, j)
            ok, r = O.check_rounded_row(gv, c, fmt, gs, _oracle_scale(ores["kv"], b, j))
            note("entry", ok, r, (b, j))
            if ok:
                stored["kv"].append(tuple(int(x) for x in ores["kv"].locate(b, j)))
        swa = cpu_cache("swa")
        for (b, p), v in ores["window_rows"].items():
            gv, gs = _rows_at(swa, d["swa"][2], b, p)
            ok, r = O.check_rounded_row(gv, v, fmt, gs, _oracle_scale(ores["swa"], b, p))
            note("window_row", ok, r, (b, p))
            if ok:
                stored["swa"].append(tuple(int(x) for x in ores["swa"].locate(b, p)))
        st = cpu_cache("state")
        W = inputs.LOGITS_PER_ENTRY[cfg.ratio]
        raw = d["new_raw"]
        for b in range(cfg.batch):
            L0, L1 = d["L0"][b], d["L1"][b]
            for p in range(max(L0, L1 - W), L1):
                gv, _ = _rows_at(st, d["state"][2], b, p)
                ref = O.formats.decode_stored(O.np_rows(raw[int(d["cu_new"][b]) + p - L0]), cfg.raw_dtype)
                note("state_row", bool(np.array_equal(gv, ref)), 0.0 if np.array_equal(gv, ref) else 1e9, (b, p))
    if "compress_idx" in cfg.stages:
        ic = cpu_cache("idx")
        for (b, j), c in ores["idx_entries"].items():
            if cfg.idx_dtype == "fp4":
                rows, scales = ic
                rpb = rows.shape[1]
                blk, slot = int(d["idx"][2][b, j // rpb]), j % rpb
                ok, r = O.check_fp4_row(rows[blk, slot].numpy(), scales[blk, slot].numpy(), c)
            else:
                gv, gs = _rows_at(ic, d["idx"][2], b, j)
                ok, r = O.check_rounded_row(gv, c, cfg.idx_dtype, gs, _oracle_scale(ores["idx"], b, j))
            note("idx_entry", ok, r, (b, j))

    same_set = {}
    if "index" in cfg.stages:
        topk = step.topk.cpu().numpy()
        tsc = None if step.topk_score is None else step.topk_score.cpu().numpy()
        for i in ores["queries"]:
            s = ores["scores"][i]
            ok, why = O.topk_acceptable(topk[i], s, cfg.k)
            note("topk", ok, 0.0 if ok else 1e9, (i, why))
            gid = topk[i][topk[i] >= 0]
            oid = ores["topk"][i][ores["topk"][i] >= 0]
            same_set[i] = set(gid.tolist()) == set(oid.tolist())
            if tsc is not None and ok and len(gid):
                err = np.abs(tsc[i][: len(gid)] - s[gid])
                tol = 1e-5 * np.abs(s[gid]) + 1e-6 * max(1.0, float(np.max(np.abs(s))))
                note("topk_score", bool(np.all(err <= tol)), float(np.max(err / tol)), i)
        rep["near_tie_queries"] = [i for i, v in same_set.items() if not v]
    if "attn" in cfg.stages:
        out = step.out.cpu().numpy()
        lse = None if step.lse is None else step.lse.cpu().numpy()
        topk_gpu = step.topk.cpu().numpy() if "index" in cfg.stages else None
        res = ores
        if stored["kv"] or stored["swa"]:
            res = dict(ores, kv=_with_gpu_rows(ores["kv"], cpu_cache("kv"), stored["kv"]),
                       swa=_with_gpu_rows(ores["swa"], cpu_cache("swa"), stored["swa"]))
        for i in ores["queries"]:
            if "index" in cfg.stages and same_set.get(i, True) is False:
                # a near tie (accepted above): the oracle attends over the GPU's own selection
                ref_o, ref_l = O.attend_query(cfg, d, res, i, topk_gpu[i])
            elif res is ores:
                ref_o, ref_l = ores["out"][i], ores["lse"][i]
            else:
                ids = ores["topk"][i] if "index" in cfg.stages else (
                    None if "topk" not in d else d["topk"][i].numpy())
                ref_o, ref_l = O.attend_query(cfg, d, res, i, ids)
            ok, r = O.allclose_out(out[i], ref_o)
            note("out", ok, r, i)
            if lse is not None:
                ok, r = O.allclose_out(lse[i], ref_l, 1e-5, 2e-3)
                note("lse", ok, r, i)
    return rep


def run_step_parity(cfg, queries=None, verbose: bool = False, prep=None, overlap: bool = False,
                    fast: bool = False, with_scores: bool = True, fast_only: bool = False) -> dict:
    """Draw inputs, run the GPU step and the oracle, compare.  Returns the report.

    overlap: the two-stream schedule.  fast: the launch sequence the benchmark times (one
    run(), then the step again through the pre-marshalled calls; a step is idempotent because
    every cache row it writes is a function of rows it does not write).  with_scores: also
    request the top-k scores (the benchmark does not).  fast_only: the pre-marshalled calls on
    fresh inputs with no run() before them, so nothing the other path wrote can stand in for an
    output the fast path failed to write.  prep(d) may edit the drawn inputs."""
    from compressed_sparse_long_c4a_amd import pipeline
    d = inputs.draw(cfg)
    if prep is not None:
        prep(d)
    g = pipeline.to_device(d)
    step = pipeline.Step(cfg, g, with_scores=with_scores)
    if fast_only:
        step.fast(g)
    elif overlap:
        step.run_overlapped()
    else:
        step.run()
    if fast and not fast_only:
        torch.cuda.synchronize()
        step.lse = None
        step.fast(g)
    torch.cuda.synchronize()
    ores = O.run_oracle(cfg, d, queries=queries)
    rep = compare(cfg, d, step, ores)
    if verbose:
        print(f"[{cfg.name}] checked {rep['checked']} worst err/tol {rep['worst']} "
              f"near-ties {rep.get('near_tie_queries', [])} failures {len(rep['fail'])}", flush=True)
        for f in rep["fail"][:20]:
            print("   FAIL", f, flush=True)
    return rep


def run_small_decode(seed: int = 0, verbose: bool = False) -> None:
    import dataclasses
    cfg = dataclasses.replace(SMALL_DECODE, seed=seed)
    rep = run_step_parity(cfg, verbose=verbose)
    if rep["fail"]:
        raise AssertionError(f"{len(rep['fail'])} parity failures, first: {rep['fail'][:5]}")
