"""fp8-row attention at row counts whose splits end in a partial step.

The fp8-row attention cuts its splits at 32 rows while it works in steps of 128 rows, so a
split's last step can hold 1 to 127 rows; the 32-row blocks past them are not staged, multiplied
or read.  These cases pick query counts, top-k sizes and windows for which the plan gives such
splits (the rows per split and the rows of every last step are printed), and compare every
(query, head) output row with the oracle's attention over the same top-k lists and window
(tolerance 1e-5 + 2e-3 relative, as in every attention test).
"""

import dataclasses

import pytest

from tests import oracle_step as O
from workloads import configs as C, inputs

D = dataclasses.replace
F8 = dict(stages=("attn",), n_heads=128)

CASES = [
    # 4 queries x 8 head groups, 1,100 rows: 7 splits of 160 (128 + 32), the last of 140 (128 + 12)
    D(C.C4A_1M_B4_FP8, name="splits_1100_rows", ctx_after=(40000, 39999, 39998, 39997), k=1000,
      window=100, **F8),
    # 2 queries, 337 rows: splits of 32 rows, one partial step each, the last of 17 rows
    D(C.C4A_1M_B4_FP8, name="splits_337_rows", ctx_after=(20000, 19999), k=300, window=37, **F8),
    # 3 queries of 2,176 rows with short and padded top-k lists (early positions): 10 splits of
    # 224 rows (128 + 96), the last of 160 (128 + 32), over the padding rows of the short lists
    D(C.C4A_1M_B4_FP8, name="splits_early_positions", ctx_after=(40000, 2000, 131), k=2048, **F8),
]


def _plan(cfg):
    """The row splits the library plans for this call (a copy of its rule, printed only)."""
    rows = cfg.k + min(cfg.window, cfg.max_context)
    units = len(cfg.ctx_after) * ((cfg.n_heads + 15) // 16)
    blocks32 = max(1, (rows + 31) // 32)
    bpw = max(1, -(-blocks32 * units // 256))
    bpw = min(bpw, blocks32, 1024 // 32)
    return bpw * 32, -(-blocks32 // bpw), rows


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_fp8_attention_partial_steps(gpu, cfg):
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    rps, splits, rows = _plan(cfg)
    last = [min(rps, rows - s * rps) % 128 or 128 for s in range(splits)]
    print(f"case {cfg.name}: {rows} rows, {splits} splits of {rps}; rows of the last steps {sorted(set(last))}",
          flush=True)
    d = inputs.draw(cfg)
    topk = inputs.random_topk(cfg, d, fill=0.93)
    g = pipeline.to_device(d)
    out, lse = csa.sparse_attn_decode(g["cu_q"], g["q_pos"], g["q"], g["kv"], cfg.ratio, topk.cuda(),
                                      g["swa"], cfg.window, cfg.softmax_scale, cfg.max_context)
    out = out.cpu().numpy()
    caches = O.prepare(d)
    worst = 0.0
    for i in range(out.shape[0]):
        want, _ = O.attend_query(cfg, d, caches, i, topk[i].numpy())
        ok, r = O.allclose_out(out[i], want)
        worst = max(worst, r)
        assert ok, f"query {i}: err/tol {r:.3g}"
    print(f"  worst err/tol {worst:.3f}", flush=True)
