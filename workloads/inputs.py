"""Input recipe of one step of a workload (CPU tensors), built only from seeded draws.

Array sizes follow the workload descriptions: a c4a entry has 8 compression logits and a
c128a entry 128; the sequence holds floor(L / ratio) compressed entries after L raw tokens;
window and compressor-state caches are backed only around the positions a step can touch.
Values are synthetic draws (see gen.py); rows the step itself writes are drawn too and are
overwritten by the step.
"""

from __future__ import annotations

import torch

from .configs import StepConfig
from .gen import Gen, paged_rows

LOGITS_PER_ENTRY = {4: 8, 128: 128}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def draw(cfg: StepConfig) -> dict:
    g = Gen(cfg.seed)
    B, R, D = cfg.batch, cfg.ratio, cfg.dim
    Wc = LOGITS_PER_ENTRY[R]
    L1 = list(cfg.ctx_after)
    new = [cfg.new_of(b) for b in range(B)]
    nq = [cfg.q_of(b) for b in range(B)]
    L0 = [l - m for l, m in zip(L1, new)]
    assert all(0 <= q <= m for q, m in zip(nq, new)), "queries sit at new positions"
    assert min(L0) >= 0
    n0 = [l // R for l in L0]
    n1 = [l // R for l in L1]
    e = [b - a for a, b in zip(n0, n1)]
    d: dict = {"L0": L0, "L1": L1}
    d["ctx_lens"] = torch.tensor(L0, dtype=torch.int32)
    d["cu_new"] = torch.tensor([0] + list(torch.tensor(new).cumsum(0).tolist()), dtype=torch.int32)
    d["cu_entries"] = torch.tensor([0] + list(torch.tensor(e).cumsum(0).tolist()), dtype=torch.int32)
    raw_t = TORCH_DTYPE[cfg.raw_dtype]
    d["new_raw"] = g.normal("new_raw", (sum(new), D), raw_t)
    d["logits"] = g.normal("logits", (sum(e), Wc))
    d["gamma"] = g.uniform("gamma", (D,), 0.5, 1.5) if cfg.gamma else None

    maxL = max(L1)
    kv = paged_rows(g, "kv", B, 256 // R, D, cfg.kv_dtype, max(n1), [(0, n) for n in n1])
    swa = paged_rows(g, "swa", B, 256, D, cfg.kv_dtype, maxL,
                     [(max(0, a - cfg.window), b) for a, b in zip(L0, L1)])
    state = paged_rows(g, "state", B, 256, D, cfg.raw_dtype, maxL,
                       [(max(0, a - Wc), b) for a, b in zip(L0, L1)])
    d["kv"], d["swa"], d["state"] = kv, swa, state

    d["q_pos"] = torch.tensor([l - c + i for l, c in zip(L1, nq) for i in range(c)], dtype=torch.int32)
    d["cu_q"] = torch.tensor([0] + list(torch.tensor(nq).cumsum(0).tolist()), dtype=torch.int32)
    total_q = sum(nq)
    d["q"] = g.normal("q", (total_q, cfg.n_heads, D), TORCH_DTYPE[cfg.q_dtype])

    if cfg.has_indexer:
        d["idx"] = paged_rows(g, "idx", B, 64, 128, cfg.idx_dtype, max(n1), [(0, n) for n in n1])
        d["q_idx"] = g.normal("q_idx", (total_q, cfg.idx_heads, 128), TORCH_DTYPE[cfg.idx_q_dtype])
        d["head_w"] = g.uniform("head_w", (total_q, cfg.idx_heads))
        if "compress_idx" in cfg.stages:
            d["new_idx_raw"] = g.normal("new_idx_raw", (sum(new), 128), raw_t)
            d["idx_logits"] = g.normal("idx_logits", (sum(e), Wc))
            d["idx_state"] = paged_rows(g, "idx_state", B, 256, 128, cfg.raw_dtype, maxL,
                                        [(max(0, a - Wc), b) for a, b in zip(L0, L1)])
    return d


def redraw_indexer(cfg: StepConfig, d: dict) -> dict:
    """The inputs d of the same step with the indexer key cache drawn in cfg.idx_dtype (same
    block table); every other array is shared with d."""
    g = Gen(cfg.seed)
    n1 = [l // cfg.ratio for l in d["L1"]]
    r = dict(d)
    r["idx"] = paged_rows(g, "idx", cfg.batch, 64, 128, cfg.idx_dtype, max(n1), [(0, n) for n in n1])
    return r


def random_topk(cfg: StepConfig, d: dict, fill: float = 1.0, seed_name: str = "topk") -> torch.Tensor:
    """A synthetic top-k list per query: distinct ids below each query's causal limit, in random
    order, with the tail padded by -1 (``fill`` = fraction of the k slots used)."""
    g = Gen(cfg.seed)
    rows = []
    for i, t in enumerate(d["q_pos"].tolist()):
        limit = (t + 1) // cfg.ratio
        cnt = min(limit, int(cfg.k * fill))
        ids = g.distinct_ints(f"{seed_name}.{i}", cnt, max(limit, 1)) if cnt else torch.zeros(0, dtype=torch.int32)
        row = torch.full((cfg.k,), -1, dtype=torch.int32)
        row[:cnt] = ids
        rows.append(row)
    return torch.stack(rows)
