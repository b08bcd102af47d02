#!/usr/bin/env python3
"""Benchmark one layer's compressed sparse attention decode step on one MI355X.

Workload (default): c4a decode at 1M context, batch 4, sequences at the four compression
boundary residues (contexts 2^20 - {0,1,2,3}), fp8 E4M3 main KV with a per-token float32
scale, fp8 indexer keys (64 heads x 128), 128 query heads of 576, top-k 2048, window 128.
A step is the whole hot path: compress the new token (main KV + window row, and indexer
key), index scores + exact top-k, sparse K=V attention + inverse RoPE.  Inputs are resident
in HBM before timing; steps rotate over several copies of the caches so that repeated steps
cannot be served from the 256 MB Infinity Cache.  The headline time is the median of 5 timed
trials of K steps replayed from a HIP graph (one step per cache replica in the graph), as the
pages deploy with full graphs; the same K steps issued eagerly are timed too
(ms_per_step_eager), and so is the pages' two-stream schedule, eagerly and from a graph.  The
dominant kernel (the index score launch) is timed with HIP events around 20 of its launches
back to back in a graph, in short trials after the GPU has rested (as its launches inside the
step run), which is what the kernel trace's average duration measures; the
events around each launch inside the eager loop also hold the command processor's dispatch
(launch_us_in_step).

Prints one JSON line.  --gpus N > 1 is not supported (one GPU only).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "c4a sparse decode query-tokens/s and achieved HBM GB/s at 1M context"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_step_c4a_1m_b4_fp8_counters.txt")
CSRC = os.path.join(ROOT, "compressed_sparse_long_c4a_amd", "csrc")
TRIALS = 5  # timed trials of K steps; the median is reported


def row_bytes(dtype: str, dim: int) -> int:
    """Bytes of one stored row: fp8 codes + a float32 scale; fp4 two codes a byte + one E8M0
    byte per 16 values."""
    return {"f32": 4 * dim, "bf16": 2 * dim, "fp8": dim + 4, "fp4": dim // 2 + dim // 16}[dtype]


def _per_seq(cfg, d):
    """(query positions, entries visible to each query, sequence of each query)."""
    qpos = d["q_pos"].tolist()
    cu_q = d["cu_q"].tolist()
    seq = [b for b in range(cfg.batch) for _ in range(cu_q[b + 1] - cu_q[b])]
    return qpos, [(t + 1) // cfg.ratio for t in qpos], seq


def algorithmic_bytes(cfg, d) -> dict:
    """Bytes the method must move in one step (no scratch, no re-reads), per stage.  Keys and
    rows shared by several queries of a sequence count once: per sequence the indexer keys of
    its latest query, and at most the entries it has (or the sum of its queries' top-k) plus the
    window positions its queries span."""
    B, H, D, W = cfg.batch, cfg.n_heads, cfg.dim, cfg.window
    total_q = d["q_pos"].shape[0]
    qpos, n_vis, seq = _per_seq(cfg, d)
    n_seq = [max([n for n, b2 in zip(n_vis, seq) if b2 == b], default=0) for b in range(B)]
    kvrow = row_bytes(cfg.kv_dtype, D)
    idx_row = row_bytes(cfg.idx_dtype, 128)
    rawb = 2 if cfg.raw_dtype == "bf16" else 4
    Wc = 8 if cfg.ratio == 4 else 128
    e = int(d["cu_entries"][-1])
    new = int(d["cu_new"][-1])
    out = {}
    if "compress" in cfg.stages:
        out["compress"] = (e * (Wc * D * rawb + Wc * 4 + kvrow)          # window rows, logits, entry
                           + new * (D * rawb + kvrow + D * rawb))          # raw row, window row, state row
    if "compress_idx" in cfg.stages:
        out["compress_idx"] = e * (Wc * 128 * rawb + Wc * 4 + idx_row) + new * 2 * 128 * rawb
    if "index" in cfg.stages:
        qb = 2 if cfg.idx_q_dtype == "bf16" else 4
        out["index_score"] = sum(n_seq) * idx_row + total_q * cfg.idx_heads * (128 * qb + 4)
        out["index_select"] = total_q * cfg.k * 4
    if "attn" in cfg.stages:
        rows = 0
        for b in range(B):
            qs = [(n, t) for n, t, b2 in zip(n_vis, qpos, seq) if b2 == b]
            if not qs:
                continue
            sel = sum(min(cfg.k, n) for n, _ in qs) if "index" in cfg.stages else sum(n for n, _ in qs)
            t_lo, t_hi = min(t for _, t in qs), max(t for _, t in qs)
            rows += min(n_seq[b], sel) + (t_hi - max(0, t_lo - W + 1) + 1)
        qb = 2 if cfg.q_dtype == "bf16" else 4
        out["attn"] = rows * kvrow + total_q * H * (D * qb + D * 4 + 4)
    return out


def algorithmic_flops(cfg, d) -> dict:
    """Multiply-add work of the two contractions (2 flops each): the indexer's q.k over every
    (query, visible entry, indexer head) and attention's QK and PV over every (query, head, row)."""
    qpos, n_vis, _ = _per_seq(cfg, d)
    out = {}
    if "index" in cfg.stages:
        out["index_score"] = 2 * cfg.idx_heads * 128 * sum(n_vis)
    if "attn" in cfg.stages:
        rows = sum((min(cfg.k, n) if "index" in cfg.stages else n) + min(cfg.window, t + 1)
                   for n, t in zip(n_vis, qpos))
        out["attn"] = 4 * cfg.n_heads * cfg.dim * rows
    return out


def score_launch_bytes(step, ab: dict) -> int:
    """Algorithmic bytes of the index-score launch: the scores' keys and queries, plus the
    compressors' bytes when they run inside it."""
    extra = ab.get("compress", 0) + ab.get("compress_idx", 0) if step.fused else 0
    return ab["index_score"] + extra


def kernels_sha1() -> str:
    """SHA-1 over the text of every kernel source (csrc/*.hip and *.h), so the committed counter
    figures go stale as soon as any kernel changes."""
    h = hashlib.sha1()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def counters(cfg):
    """HBM bytes per launch of the score kernel and per step (all of the step's kernels), from
    the committed rocprofv3 counter summary: (score_bytes, step_bytes), or (None, None) when
    there is none, it was taken from different kernel sources, or the workload is not the one it
    was taken on (the 1M c4a fp8 decode)."""
    from workloads import configs
    if cfg.name != configs.HEADLINE.name or not os.path.exists(COUNTERS_FILE):
        return None, None
    kv = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha1") != kernels_sha1():
        return None, None
    try:
        return float(kv["score_traffic_bytes_per_launch"]), float(kv["step_traffic_bytes"])
    except (KeyError, ValueError):
        return None, None


def time_launches(fn, reps: int = 50, replays: int = 5) -> float:
    """Mean microseconds per call of fn (one launch each): `reps` calls captured in a HIP graph
    and replayed, HIP events around the replays (no host launch cost in the figure)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * replays)


def next_rows(cfg) -> dict:
    """Rows beyond the step, each timed on its own: the query norm + RoPE + window-key kernel
    (csa_q_norm_rope_swa) at the decode step's shapes and at the chunked prefill's."""
    import torch
    import compressed_sparse_long_c4a_amd as csa
    dev = "cuda"
    out = {}
    # (name, sequences, queries and new rows per sequence, heads, context after the step, window dtype)
    shapes = [("decode_1m_b4", 4, 1, 128, 1 << 20, "fp8"),
              ("prefill_4k_on_64k", 1, 4096, 64, 65536 + 4096, "bf16")]
    for name, batch, per, heads, ctx_after, swa_dt in shapes:
        total = batch * per
        q = torch.randn(total, heads, 576, device=dev).to(torch.bfloat16)
        q_pos = torch.tensor([ctx_after - per + i for _ in range(batch) for i in range(per)],
                             dtype=torch.int32, device=dev)
        ctx_lens = torch.full((batch,), ctx_after - per, dtype=torch.int32, device=dev)
        cu_new = torch.arange(0, total + 1, per, dtype=torch.int32, device=dev)
        raw = torch.randn(total, 576, device=dev).to(torch.bfloat16)
        nblk = (ctx_after + 255) // 256
        bt = torch.arange(batch * nblk, dtype=torch.int32, device=dev).view(batch, nblk)
        if swa_dt == "fp8":
            rows = torch.zeros(batch * nblk, 256, 576, dtype=torch.uint8, device=dev)
            scales = torch.ones(batch * nblk, 256, device=dev)
        else:
            rows = torch.zeros(batch * nblk, 256, 576, dtype=torch.bfloat16, device=dev)
            scales = None
        swa = csa.PagedCache(rows, bt, scales)
        q_out = torch.empty_like(q)
        gamma = torch.rand(576, device=dev) + 0.5
        fn = lambda: csa.q_norm_rope_swa(q_pos, q, q_out=q_out, gamma=gamma, ctx_lens=ctx_lens,
                                         cu_new=cu_new, new_raw=raw, swa=swa)
        us = time_launches(fn)
        row_out = 576 + 4 if swa_dt == "fp8" else 576 * 2
        # queries in and out (bf16), raw rows in (bf16), window rows out, the gain
        nbytes = 2 * q.numel() * 2 + raw.numel() * 2 + total * row_out + 576 * 4
        out[name] = {"kernel": "q_norm_rope_swa_kernel", "queries": total, "heads": heads,
                     "window_rows": total, "window_dtype": swa_dt, "us_per_launch": round(us, 2),
                     "algorithmic_bytes": nbytes, "achieved_gbs": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        del q, q_out, raw, rows, scales, swa
    return out


def attn_fp8_rows(cfg, step, g) -> dict:
    """The step's attention (partial + merge launches) with its output rows written as fp8
    codes + one scale per row (csa_sparse_attn_decode_fp8) against the float32 rows, on the
    benchmark workload's own inputs and top-k lists; HIP-graph timed like next_rows."""
    import torch
    import compressed_sparse_long_c4a_amd as csa
    topk = step.topk if "index" in cfg.stages else g.get("topk")
    args = (g["cu_q"], g["q_pos"], g["q"], g["kv"], cfg.ratio, topk, g["swa"], cfg.window,
            cfg.softmax_scale, cfg.max_context)
    total_q, heads, dim = g["q"].shape
    codes = torch.empty((total_q, heads, dim), dtype=torch.uint8, device="cuda")
    scales = torch.empty((total_q, heads), dtype=torch.float32, device="cuda")
    L = csa.lib()
    ws = step.attn_ws

    def fp8_call():
        st = L.csa_sparse_attn_decode_fp8(
            csa._stream(), g["cu_q"].shape[0] - 1, g["cu_q"].data_ptr(), g["q_pos"].data_ptr(),
            total_q, cfg.max_context, g["q"].data_ptr(), csa.dtype_code(g["q"].dtype), heads,
            csa._cref(g["kv"]), cfg.ratio, csa._ptr(topk), 0 if topk is None else topk.shape[1],
            csa._cref(g["swa"]), cfg.window, cfg.softmax_scale, cfg.rope_base, 64,
            codes.data_ptr(), scales.data_ptr(), None, None, ws.data_ptr(), ws.numel())
        assert st == 0, st

    us_fp8 = time_launches(fp8_call, reps=20)
    us_f32 = time_launches(lambda: step.attn(g, with_lse=False), reps=20)
    return {"kernels": "attn_partial_fp8 + attn_merge", "workload": cfg.name,
            "us_per_call_fp8_rows": round(us_fp8, 2), "us_per_call_f32_rows": round(us_f32, 2),
            "output_bytes_fp8": total_q * heads * (dim + 4), "output_bytes_f32": total_q * heads * dim * 4}


def fp4_indexer_rows(cfg, d, reps, steps: int) -> dict:
    """The same step with the indexer key cache in fp4 (two E2M1 codes a byte, one E8M0 scale
    per 16 values: 72-byte keys instead of 132), every other input shared with the timed step:
    the step time replayed from a graph and the score kernel's launch time (20 launches back
    to back), as for the fp8 step."""
    import dataclasses
    import torch
    from compressed_sparse_long_c4a_amd import PagedCache, pipeline
    from workloads import inputs
    cfg4 = dataclasses.replace(cfg, name=cfg.name + "_fp4idx", idx_dtype="fp4")
    rows, scales, bt = inputs.redraw_indexer(cfg4, d)["idx"]
    rows, scales, bt = rows.cuda(), scales.cuda(), bt.cuda()
    g4 = []
    for i, g in enumerate(reps):
        r = dict(g)
        r["idx"] = PagedCache(rows if i == 0 else rows.clone(), bt, scales if i == 0 else scales.clone())
        g4.append(r)
    step = pipeline.Step(cfg4, g4[0], with_scores=False)
    for i in range(5):
        step.run(g4[i % len(g4)], with_lse=False)
    for g in g4:
        step.fast(g)
    torch.cuda.synchronize()
    graph = graph_of(lambda g: step.fast(g), g4)
    ms = statistics.median(time_graph(graph, max(1, steps // len(g4)))) / len(g4)
    del graph
    launch = (lambda g: step.compress_index_score(g)) if step.via_score else (lambda g: step.index_score(g))
    score_us = back_to_back_ms(launch, g4) * 1e3
    nbytes = score_launch_bytes(step, algorithmic_bytes(cfg4, d))
    total_q = d["q_pos"].shape[0]
    return {"workload": cfg4.name, "kernel": "index_score_mfma (fp4 keys)",
            "ms_per_step": round(ms, 5), "query_tokens_per_s": round(total_q / (ms / 1e3), 1),
            "score_launch_us": round(score_us, 2), "score_algorithmic_bytes": nbytes,
            "score_achieved_gbs": round(nbytes / score_us / 1e3, 1),
            "score_frac": round(nbytes / score_us / 1e3 / HBM_PEAK_GBS, 4),
            "index_row_bytes": row_bytes("fp4", 128)}


def stream_read_gbs(nbytes: int = 2 << 30, reps: int = 10) -> float:
    """Achievable read bandwidth on this device: the library's streaming-read probe over
    `nbytes` (well beyond the 256 MB infinity cache), HIP events around `reps` launches;
    GB/s of bytes read."""
    import torch
    import compressed_sparse_long_c4a_amd as csa
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = csa.read_probe(x)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        csa.read_probe(x, sink)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    del x
    return nbytes / us / 1e3


def clone_caches(g: dict) -> dict:
    from compressed_sparse_long_c4a_amd import PagedCache
    from compressed_sparse_long_c4a_amd.pipeline import CACHE_KEYS
    r = dict(g)
    for k in CACHE_KEYS:
        if k in g:
            c = g[k]
            r[k] = PagedCache(c.rows.clone(), c.block_table.clone(), None if c.scales is None else c.scales.clone())
    return r


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, d) -> dict:
    """The float64 oracle running the same step (every query: compress, the full indexer scans,
    top-k, attention, inverse RoPE) on the host: the median of 3 runs with numpy's threads on
    every core this process may use, and one run on a single thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from tests import oracle_step as O
    caches = O.prepare(d)
    total_q = d["q_pos"].shape[0]
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    def one(threads=None):
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            O.run_oracle(cfg, d, caches=caches)   # (a repeat rewrites the same cache rows)
            return time.perf_counter() - t0
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    runs = [one(cores) for _ in range(3)]
    single = one(1)
    med = statistics.median(runs)
    return {"value": total_q / med, "unit": "query-tokens/s", "cores": used, "kind": "oracle",
            "cpu": cpu_model(), "nproc": cores,
            "single_thread_value": total_q / single,
            "sample": f"the whole step of the same workload ({total_q} queries: compress, index scores "
                      f"and top-k, attention, inverse RoPE) on the float64 oracle: median of 3 runs "
                      f"({', '.join(f'{r:.2f}' for r in runs)} s) with {used} BLAS threads, and one "
                      f"run on one thread ({single:.2f} s)"}


def graph_of(fn, reps):
    """A HIP graph holding fn(g) once for every input dict g of reps (warmed up on a side stream)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for g in reps:
            fn(g)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for g in reps:
            fn(g)
    graph.replay()
    torch.cuda.synchronize()
    return graph


def back_to_back_ms(launch, reps, n: int = 20, trials: int = 10, rest_s: float = 0.02) -> float:
    """Milliseconds per call of launch(g): n calls back to back in one HIP graph, g rotating over
    the cache replicas reps.  Each trial starts after the GPU has been idle for rest_s, replays
    the graph once untimed (the clocks come back up from idle, and the timed replay's packets are
    queued while it runs, so the host's submission is not timed) and then once between events;
    the median trial is taken.  Short trials see the kernel as the step does (between the step's
    latency-bound launches); hundreds of HBM-bound launches in a row raise the board's power to
    ~1.25 kW and lower the gfx clock, and the launch times then drift upward."""
    import torch
    graph = graph_of(lambda _g: [launch(reps[i % len(reps)]) for i in range(n)], reps[:1])
    out = []
    for _ in range(trials):
        time.sleep(rest_s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        graph.replay()
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / n)
    del graph
    torch.cuda.synchronize()
    return statistics.median(out)


def time_graph(graph, replays: int, trials: int = TRIALS) -> list:
    """Milliseconds per replay of `graph` in each of `trials` timed runs of `replays` replays."""
    import torch
    out = []
    for _ in range(trials):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / replays)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--config", default=None, help="workload name (default: the 1M c4a fp8 decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the separate timings of the rows beyond the step")
    ap.add_argument("--no-stream-probe", action="store_true",
                    help="skip the 2 GiB read that measures the achievable read bandwidth")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device-to-device copy (a reference for byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the sharded path is a design, not part of this build)", file=sys.stderr)
        return 2

    import torch
    from compressed_sparse_long_c4a_amd import pipeline
    from workloads import configs, inputs

    cfg = configs.HEADLINE
    if args.config:
        cfg = {c.name: c for c in configs.CONFIGS}[args.config]
    torch.cuda.set_device(0)
    print(f"# drawing inputs for {cfg.name}", file=sys.stderr, flush=True)
    d = inputs.draw(cfg)
    g0 = pipeline.to_device(d)
    reps = [g0] + [clone_caches(g0) for _ in range(max(1, args.replicas) - 1)]
    step = pipeline.Step(cfg, g0, with_scores=False)
    torch.cuda.synchronize()
    print("# inputs resident; warming up", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    K, Wm = args.steps, args.warmup
    for i in range(Wm):
        step.run(reps[i % len(reps)], with_lse=False)
    torch.cuda.synchronize()

    has_index = "index" in cfg.stages
    for g in reps:                       # marshal the C calls of every replica once
        step.fast(g)
    torch.cuda.synchronize()
    # the K steps issued eagerly, one launch at a time (events around every score launch)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        step.fast(reps[i % len(reps)], ev[i] if has_index else None)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    score_ms_in_step = statistics.mean(a.elapsed_time(b) for a, b in ev) if has_index else None
    print(f"# timed {K} eager steps: {ms_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    # the same K steps replayed from a HIP graph that holds one step per cache replica, timed in
    # TRIALS trials; the median trial is the headline
    graph_ms, graph_trials = None, None
    if not args.no_graph:
        try:
            graph = graph_of(lambda g: step.fast(g), reps)
            graph_trials = [t / len(reps) for t in time_graph(graph, max(1, K // len(reps)))]
            graph_ms = statistics.median(graph_trials)
            del graph
        except Exception as exc:  # graph capture is reported, never required
            print(f"# graph variant unavailable: {exc}", file=sys.stderr)

    # the dominant kernel's launch time: the step's own score launch (with the compressor
    # workgroups when it has them), 20 times back to back in a graph, rotating over the cache
    # replicas as the steps do (so the keys come from HBM, not the infinity cache), events
    # around the replays
    score_ms = None
    if has_index:
        launch = (lambda g: step.compress_index_score(g)) if step.via_score else (lambda g: step.index_score(g))
        score_ms = back_to_back_ms(launch, reps)

    # the pages' two-stream schedule (main-KV compressor and window rows on a second stream,
    # beside the indexer), issued eagerly and replayed from a graph
    ms_two = None
    if has_index and "compress" in cfg.stages:
        step.run_overlapped(reps[0], with_lse=False)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(K):
            step.run_overlapped(reps[i % len(reps)], with_lse=False)
        b.record()
        torch.cuda.synchronize()
        ms_two = {"eager": round(a.elapsed_time(b) / K, 5), "graph": None}
        if not args.no_graph:
            try:
                g2 = graph_of(lambda g: step.run_overlapped(g, with_lse=False), reps)
                ms_two["graph"] = round(statistics.median(time_graph(g2, max(1, K // len(reps)))) / len(reps), 5)
                del g2
            except Exception as exc:
                print(f"# two-stream graph unavailable: {exc}", file=sys.stderr)

    # per-stage breakdown (separate pass, events around every stage)
    stages = {}
    # ("compress" runs every compressor of the step -- main KV and indexer keys -- in one launch)
    # (with the compressors inside the score launch, "index_score" is that one launch)
    names = [s for s in ("compress", "index_score", "index_select", "attn")
             if (s in cfg.stages) or (s.startswith("index") and has_index)
             or (s == "compress" and "compress_idx" in cfg.stages)]
    if step.via_score:
        names.remove("compress")
    run_stage = {"compress": step.compress_all,
                 "index_score": step.compress_index_score if step.via_score else step.index_score,
                 "index_select": step.index_select, "attn": lambda g: step.attn(g, with_lse=False)}
    evs = {s: [] for s in names}
    for i in range(min(K, 100)):
        g = reps[i % len(reps)]
        for s in names:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run_stage[s](g)
            b.record()
            evs[s].append((a, b))
    torch.cuda.synchronize()
    for s in names:
        stages[s] = round(statistics.median(a.elapsed_time(b) for a, b in evs[s]) * 1e3, 2)

    ab = algorithmic_bytes(cfg, d)
    step_bytes = sum(ab.values())
    fl = algorithmic_flops(cfg, d)
    step_flops = sum(fl.values())
    total_q = d["q_pos"].shape[0]
    # the headline: the K steps replayed from the HIP graph (the pages deploy with full CUDA
    # graphs); the eager issue of the same K steps is reported beside it
    graph_head = graph_ms is not None
    ms_head = graph_ms if graph_head else ms_step
    score_traffic, step_traffic = counters(cfg)
    value = total_q / (ms_head / 1e3)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_head, 5),
        "timing": "hip_graph_replay" if graph_head else "eager",
        "ms_per_step_eager": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "hbm_gbs": round(step_bytes / (ms_head / 1e3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms_head / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "algorithmic_flops_per_step": step_flops,
        "mfma_frac": round(step_flops / (ms_head / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "stages_us": stages,
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 5),
        "ms_per_step_graph_trials": None if graph_trials is None else [round(t, 5) for t in graph_trials],
        "ms_per_step_two_stream": ms_two,
        "step_traffic_bytes": step_traffic,
        "config": {
            "workload": cfg.name, "ratio": cfg.ratio, "batch": cfg.batch,
            "context": list(cfg.ctx_after), "new_tokens": cfg.new_tokens,
            "queries_per_seq": cfg.q_per_seq, "heads": cfg.n_heads, "dim": cfg.dim,
            "kv_dtype": cfg.kv_dtype, "indexer": f"{cfg.idx_heads}x128 {cfg.idx_dtype}" if has_index else None,
            "top_k": cfg.k if has_index else None, "window": cfg.window,
            "cache_replicas": len(reps), "arithmetic": "fp8/bf16 operands on bf16 MFMA, fp32 accumulate",
        },
    }
    if has_index:
        launch_bytes = score_launch_bytes(step, ab)
        launch_flops = fl["index_score"]
        achieved = launch_bytes / (score_ms / 1e3) / 1e9
        kname = "index_score_mfma" + (" (with the compressor workgroups)" if step.fused else "")
        if launch_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > launch_bytes / (HBM_PEAK_GBS * 1e9):
            # many queries per sequence share each key: the bf16 contraction bounds the kernel
            tf = launch_flops / (score_ms / 1e3) / 1e12
            result["roofline"] = {
                "kernel": kname, "bound": "mfma", "achieved": round(tf, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None, "launch_us": round(score_ms * 1e3, 2),
                "launch_us_in_step": round(score_ms_in_step * 1e3, 2),
                "algorithmic_flops_per_launch": launch_flops, "algorithmic_bytes_per_launch": launch_bytes,
            }
        else:
            result["roofline"] = {
                "kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": score_traffic, "launch_us": round(score_ms * 1e3, 2),
                "launch_us_in_step": round(score_ms_in_step * 1e3, 2),
                "algorithmic_bytes_per_launch": launch_bytes,
            }
        if not args.no_stream_probe and result["roofline"]["bound"] == "hbm":
            sr = stream_read_gbs()
            result["roofline"]["stream_read_gbs"] = round(sr, 1)
            result["roofline"]["frac_of_stream_read"] = round(achieved / sr, 4)
            result["hbm_frac_of_stream_read"] = round(step_bytes / (ms_head / 1e3) / 1e9 / sr, 4)
    if not args.no_next_rows:
        print("# timing the rows beyond the step", file=sys.stderr, flush=True)
        result["next_rows"] = {"q_norm_rope_swa": next_rows(cfg),
                               "attn_fp8_output": attn_fp8_rows(cfg, step, reps[0])}
        if has_index and cfg.idx_dtype == "fp8" and cfg.idx_q_dtype == "bf16":
            result["next_rows"]["fp4_indexer"] = fp4_indexer_rows(cfg, d, reps, min(K, 100))
    if not args.no_cpu_baseline:
        print("# timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, d)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
