"""One layer's step through the C ABI: compress -> index/top-k -> sparse attention.

Marshalling only: every stage is one of the library calls in this package, launched on
torch's current HIP stream in order, with no host synchronisation.  ``cfg`` is any object
with the fields of a workload configuration (ratio, stages, k, window, softmax_scale, ...).
"""

from __future__ import annotations

import torch

from . import (PagedCache, compress_insert, index_score, index_select, index_workspace_size,
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

    def compress(self, g=None):
        g = g or self.g
        c = self.cfg
        compress_insert(c.ratio, g["ctx_lens"], g["cu_new"], g["new_raw"], g["cu_entries"], g["logits"],
                        g["state"], g["kv"], g["swa"], g.get("gamma"), c.eps, c.rope_base, 64)

    def compress_idx(self, g=None):
        g = g or self.g
        c = self.cfg
        compress_insert(4, g["ctx_lens"], g["cu_new"], g["new_idx_raw"], g["cu_entries"], g["idx_logits"],
                        g["idx_state"], g["idx"], None, None, c.eps, c.rope_base, 64)

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

    def run(self, g=None, with_lse: bool = True):
        """The whole step, in stage order, on the current stream."""
        st = self.cfg.stages
        if "compress" in st:
            self.compress(g)
        if "compress_idx" in st:
            self.compress_idx(g)
        if "index" in st:
            self.index_score(g)
            self.index_select(g)
        if "attn" in st:
            self.attn(g, with_lse)
        return self
