"""One layer's step through the C ABI: compress -> index/top-k -> sparse attention.

Marshalling only: every stage is one of the library calls in this package, launched on
torch's current HIP stream in order, with no host synchronisation.  ``cfg`` is any object
with the fields of a workload configuration (ratio, stages, k, window, softmax_scale, ...).
"""

from __future__ import annotations

import torch

import ctypes

from . import (OK, CompressJob, CsaError, PagedCache, compress_insert, compress_insert_many,
               compress_index_score, compress_index_score_launches, compress_jobs_array, dtype_code,
               index_score, index_select,
               index_workspace_size, lib,
               sparse_attn_decode, sparse_attn_workspace_size)

CACHE_KEYS = ("kv", "swa", "state", "idx", "idx_state")


def to_device(d: dict, device: str | torch.device = "cuda") -> dict:
    """Move a CPU input dict to the GPU; (rows, scales, block_table) triples become PagedCache."""
    g = {}
    for key, v in d.items():
        if key in CACHE_KEYS:
            rows, scales, bt = v
            g[key] = PagedCache(rows.to(device), bt.to(device), None if scales is None else scales.to(device))
        elif isinstance(v, torch.Tensor):
            g[key] = v.to(device)
        else:
            g[key] = v
    return g


class Step:
    """Preallocated outputs and workspaces for repeated steps of one configuration."""

    def __init__(self, cfg, g: dict, with_scores: bool = True):
        self.cfg, self.g = cfg, g
        dev = g["q"].device
        total_q, H, D = g["q"].shape
        self.total_q = total_q
        self.topk = self.topk_score = self.idx_ws = None
        if "index" in cfg.stages:
            self.topk = torch.empty((total_q, cfg.k), dtype=torch.int32, device=dev)
            self.topk_score = torch.empty((total_q, cfg.k), dtype=torch.float32, device=dev) if with_scores else None
            n = index_workspace_size(total_q, cfg.max_context, cfg.k)
            self.idx_ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        self.attn_topk = self.topk if "index" in cfg.stages else g.get("topk")
        has_topk = self.attn_topk is not None
        k = self.attn_topk.shape[1] if has_topk else 0
        n = sparse_attn_workspace_size(total_q, H, D, cfg.ratio, has_topk, k, cfg.max_context, cfg.window)
        self.attn_ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        self.out = torch.empty((total_q, H, D), dtype=torch.float32, device=dev)
        self.lse = None
        self.side = None  # second stream for the overlapped schedule (created on first use)
        # fast(): with an indexer-key compressor and an index stage, the step's compressors go
        # through csa_compress_index_score (the indexer-key job is the last of _jobs), which runs
        # them inside the index-score launch or as a launch of their own; the library decides and
        # `fused` records its answer (one launch).  run() always launches the compressors first.
        self.via_score = "compress_idx" in cfg.stages and "index" in cfg.stages
        self.fused = False
        if self.via_score:
            jobs = self._jobs(g)
            self.fused = compress_index_score_launches(jobs, len(jobs) - 1, g["new_raw"].shape[0], total_q,
                                                       g["q_idx"].dtype, g["q_idx"].shape[1]) == 1
        self._bound = {}  # id(g) -> (g, pre-marshalled C calls of the step, refs) (see fast())

    def compress(self, g=None):
        g = g or self.g
        c = self.cfg
        compress_insert(c.ratio, g["ctx_lens"], g["cu_new"], g["new_raw"], g["cu_entries"], g["logits"],
                        g["state"], g["kv"], g["swa"], g.get("gamma"), c.eps, c.rope_base, 64)

    def _jobs(self, g) -> list:
        c = self.cfg
        jobs = []
        if "compress" in c.stages:
            jobs.append(CompressJob(c.ratio, g["new_raw"], g["cu_entries"], g["logits"], g["state"], g["kv"],
                                    g["swa"], g.get("gamma"), c.eps, c.rope_base, 64))
        if "compress_idx" in c.stages:
            jobs.append(CompressJob(4, g["new_idx_raw"], g["cu_entries"], g["idx_logits"], g["idx_state"],
                                    g["idx"], None, None, c.eps, c.rope_base, 64))
        return jobs

    def compress_all(self, g=None):
        """Every compressor of the step (main KV with window rows, indexer keys) in one launch."""
        g = g or self.g
        jobs = self._jobs(g)
        if jobs:
            compress_insert_many(g["ctx_lens"], g["cu_new"], g["new_raw"].shape[0], jobs)

    def compress_idx(self, g=None):
        g = g or self.g
        c = self.cfg
        compress_insert(4, g["ctx_lens"], g["cu_new"], g["new_idx_raw"], g["cu_entries"], g["idx_logits"],
                        g["idx_state"], g["idx"], None, None, c.eps, c.rope_base, 64)

    def compress_index_score(self, g=None):
        """Every compressor of the step inside the index-score launch (see fast())."""
        g = g or self.g
        c = self.cfg
        jobs = self._jobs(g)
        compress_index_score(g["ctx_lens"], g["cu_new"], g["new_raw"].shape[0], jobs, len(jobs) - 1,
                             g["cu_q"], g["q_pos"], g["q_idx"], g["head_w"], g["idx"], c.k, c.max_context,
                             self.idx_ws)

    def index_score(self, g=None):
        g = g or self.g
        c = self.cfg
        index_score(g["cu_q"], g["q_pos"], g["q_idx"], g["head_w"], g["idx"], c.k, c.max_context, self.idx_ws)

    def index_select(self, g=None):
        g = g or self.g
        c = self.cfg
        index_select(g["cu_q"], g["q_pos"], c.k, c.max_context, self.idx_ws, self.topk, self.topk_score)

    def attn(self, g=None, with_lse: bool = True):
        g = g or self.g
        c = self.cfg
        topk = self.topk if "index" in c.stages else g.get("topk")
        out, lse = sparse_attn_decode(g["cu_q"], g["q_pos"], g["q"], g["kv"], c.ratio, topk, g["swa"],
                                      c.window, c.softmax_scale, c.max_context, c.rope_base, 64,
                                      with_lse=with_lse, out=self.out, workspace=self.attn_ws)
        self.lse = lse
        return out, lse

    def run_overlapped(self, g=None, with_lse: bool = True):
        """The whole step with the main-KV compressor (and window-row insert) on a second stream,
        concurrent with the indexer pipeline (indexer compress, score, top-k) on the current one;
        attention waits for both.  This is the schedule of the c4a decode path in the pages'
        multi-stream design; every stream keeps the default priority."""
        st = self.cfg.stages
        if "compress" not in st or "index" not in st:
            return self.run(g, with_lse)
        main = torch.cuda.current_stream()
        if self.side is None:
            self.side = torch.cuda.Stream(device=main.device)
            self.ev_fork = torch.cuda.Event()
            self.ev_join = torch.cuda.Event()
        self.ev_fork.record(main)
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.ev_fork)
            self.compress(g)
            self.ev_join.record(self.side)
        if "compress_idx" in st:
            self.compress_idx(g)
        self.index_score(g)
        self.index_select(g)
        main.wait_event(self.ev_join)
        if "attn" in st:
            self.attn(g, with_lse)
        return self

    def _bind(self, g: dict):
        """Marshal every C call of the step for input dict g once: (name, function, arguments
        without the leading stream).  The argument checks of the wrappers ran when the same calls
        went through them (fast() requires one run() of g first)."""
        c, L = self.cfg, lib()
        P = ctypes.c_void_p
        calls = []
        refs = []  # keep the ctypes structs alive

        def cache(x):
            r = ctypes.pointer(x.c())
            refs.append(r)
            return r
        B = g["ctx_lens"].shape[0] if "ctx_lens" in g else g["cu_q"].shape[0] - 1
        jobs = self._jobs(g)
        total_q = g["q_pos"].shape[0]
        fused = self.via_score and bool(jobs)
        if jobs and not fused:  # every compressor of the step in one launch
            arr = compress_jobs_array(jobs)
            refs.extend([jobs, arr])
            calls.append(("compress", L.csa_compress_insert_many, (
                B, g["ctx_lens"].data_ptr(), g["cu_new"].data_ptr(), g["new_raw"].shape[0], len(jobs), arr)))
        if "index" in c.stages and fused:  # the compressors with the score (one or two launches)
            arr = compress_jobs_array(jobs)
            refs.extend([jobs, arr])
            calls.append(("index_score", L.csa_compress_index_score, (
                B, g["ctx_lens"].data_ptr(), g["cu_new"].data_ptr(), g["new_raw"].shape[0], len(jobs), arr,
                len(jobs) - 1, g["cu_q"].data_ptr(), g["q_pos"].data_ptr(), total_q, c.max_context,
                g["q_idx"].data_ptr(), dtype_code(g["q_idx"].dtype), g["q_idx"].shape[1],
                g["head_w"].data_ptr(), cache(g["idx"]), c.k, self.idx_ws.data_ptr(), self.idx_ws.numel())))
        elif "index" in c.stages:
            calls.append(("index_score", L.csa_index_score, (
                B, g["cu_q"].data_ptr(), g["q_pos"].data_ptr(), total_q, c.max_context, g["q_idx"].data_ptr(),
                dtype_code(g["q_idx"].dtype), g["q_idx"].shape[1], g["head_w"].data_ptr(), cache(g["idx"]),
                c.k, self.idx_ws.data_ptr(), self.idx_ws.numel())))
        if "index" in c.stages:
            calls.append(("index_select", L.csa_index_select, (
                B, g["cu_q"].data_ptr(), g["q_pos"].data_ptr(), total_q, c.max_context, c.k,
                self.topk.data_ptr(), None if self.topk_score is None else self.topk_score.data_ptr(),
                self.idx_ws.data_ptr(), self.idx_ws.numel())))
        if "attn" in c.stages:
            topk = self.topk if "index" in c.stages else g.get("topk")
            calls.append(("attn", L.csa_sparse_attn_decode, (
                B, g["cu_q"].data_ptr(), g["q_pos"].data_ptr(), total_q, c.max_context, g["q"].data_ptr(),
                dtype_code(g["q"].dtype), g["q"].shape[1], cache(g["kv"]), c.ratio,
                None if topk is None else topk.data_ptr(), 0 if topk is None else topk.shape[1],
                cache(g["swa"]), c.window, c.softmax_scale, c.rope_base, 64, self.out.data_ptr(), None,
                self.attn_ws.data_ptr(), self.attn_ws.numel())))
        return calls, refs

    def fast(self, g=None, score_events=None):
        """The whole step (no lse) through pre-marshalled C calls, on the current stream: the same
        calls as run(), with the host-side Python work done once per input dict.  score_events:
        optional (before, after) torch events recorded around the index-score launch."""
        g = g or self.g
        key = id(g)
        # the entry holds g itself, so the tensors whose pointers it marshalled stay alive and an
        # id reused by another dict after g is gone can never match
        if key not in self._bound or self._bound[key][0] is not g:
            self._bound[key] = (g,) + self._bind(g)
        stream = torch.cuda.current_stream().cuda_stream
        for name, fn, args in self._bound[key][1]:
            if score_events is not None and name == "index_score":
                score_events[0].record()
            st = fn(stream, *args)
            if score_events is not None and name == "index_score":
                score_events[1].record()
            if st != OK:
                raise CsaError(name, st)
        return self

    def run(self, g=None, with_lse: bool = True):
        """The whole step, in stage order, on the current stream."""
        st = self.cfg.stages
        self.compress_all(g)
        if "index" in st:
            self.index_score(g)
            self.index_select(g)
        if "attn" in st:
            self.attn(g, with_lse)
        return self
