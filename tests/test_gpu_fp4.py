"""FP4 caches on the GPU (CSA_FP4_E2M1: two E2M1 codes a byte, one E8M0 scale per 16 values).

* whole steps with the indexer cache in fp4: the compressor writes fp4 indexer entries (each
  checked with tests/oracle_step.check_fp4_row against the oracle's exact entry), the MFMA
  score kernel (bf16 queries) or the float32 score kernel reads fp4 keys, and the top-k and
  the attention over it follow the acceptance rules of tests/pipeline_check.py;
* the compressor writing fp4 entries at the main-KV width (576 = 36 scale blocks), c4a and
  c128a, every entry of a ragged prefill checked the same way.
"""

import dataclasses

import numpy as np
import pytest
import torch

from tests import oracle_step as O
from tests import pipeline_check as P
from workloads import configs as C, inputs

D = dataclasses.replace

STEP_CASES = {
    # the 1M fp8 decode's shapes (128 heads, 64 indexer heads) at shorter contexts
    "c4a_fp4idx_decode": C.scaled(C.C4A_1M_B4_FP4IDX, (9220, 4099, 2562, 2049), k=256),
    # a chunked prefill: 512 queries, 128 new indexer entries written in fp4 and read back
    "c4a_fp4idx_prefill": C.scaled(C.C4A_PREFILL_64K, (2048 + 512,), new_tokens=512, q_per_seq=512,
                                   k=128, idx_dtype="fp4"),
    # float32 queries: the float32 score kernel decoding fp4 keys
    "ref_fp4idx_f32q": D(C.REF, name="ref_c4a_1k_fp4idx", idx_dtype="fp4"),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(STEP_CASES))
def test_step_with_fp4_indexer(gpu, name):
    cfg = STEP_CASES[name]
    print(f"case {name}: {cfg}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True)
    assert not rep["fail"], rep["fail"][:10]
    assert rep["checked"].get("topk", 0) > 0
    if "compress_idx" in cfg.stages:
        assert rep["checked"].get("idx_entry", 0) > 0


@pytest.mark.gpu
@pytest.mark.parametrize("ratio", [4, 128])
def test_compressor_writes_fp4_entries(gpu, ratio):
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    from oracle import compress
    base = C.C4A_PREFILL_64K if ratio == 4 else C.C128A_1M_B8
    cfg = D(base, name=f"fp4_entries_r{ratio}", ctx_after=(700, 1500, 300, 290) if ratio == 4 else
            (1100, 700, 129, 5000), new_tokens=(300, 3, 300, 40) if ratio == 4 else (600, 1, 129, 300),
            q_per_seq=0, n_heads=16, kv_dtype="fp4", stages=("compress",), gamma=True)
    print(f"case {cfg.name}", flush=True)
    d = inputs.draw(cfg)
    g = pipeline.to_device(d)
    csa.compress_insert(ratio, g["ctx_lens"], g["cu_new"], g["new_raw"], g["cu_entries"], g["logits"],
                        g["state"], g["kv"], swa=None, gamma=g["gamma"], eps=cfg.eps,
                        rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    kv_o, state_o = O.oracle_cache(d["kv"]), O.oracle_cache(d["state"])
    raw, rdt = O.raw_values(d["new_raw"])
    ent, _ = compress.compress_insert(ratio, d["ctx_lens"].tolist(), d["cu_new"].tolist(), raw, rdt,
                                      d["cu_entries"].tolist(), d["logits"].numpy(),
                                      d["gamma"].numpy().astype(np.float64), cfg.eps, cfg.rope_base, 64,
                                      state_o, kv_o, None)
    rows, scales = g["kv"].rows.cpu().numpy(), g["kv"].scales.cpu().numpy()
    bt = d["kv"][2]
    rpb = rows.shape[1]
    worst = 0.0
    for (b, j), c in ent.items():
        blk, slot = int(bt[b, j // rpb]), j % rpb
        ok, r = O.check_fp4_row(rows[blk, slot], scales[blk, slot], c)
        worst = max(worst, r)
        assert ok, f"entry {(b, j)}: err/tol {r:.3g}"
    assert len(ent) == int(d["cu_entries"][-1]) > 0
    print(f"  {len(ent)} fp4 entries of 576 values; worst err/tol {worst:.3f}", flush=True)


# the first positions of a sequence with the indexer cache in fp4: no entry yet, entry 0 with
# its zero-padded slots (a block scale from a partly zero row), k >= n and k < n
EARLY_FP4 = D(C.C4A_1M_B4_FP4IDX, name="c4a_early_positions_fp4idx", ctx_after=(1, 2, 3, 4, 5, 8, 9, 130),
              n_heads=16, k=8)


@pytest.mark.gpu
def test_early_positions_fp4_indexer(gpu):
    print(f"case {EARLY_FP4.name}", flush=True)
    rep = P.run_step_parity(EARLY_FP4, verbose=True)
    assert not rep["fail"], rep["fail"][:10]


def _zero_fp4_keys(d):
    rows, scales, _ = d["idx"]
    rows.zero_()
    scales.fill_(127)


@pytest.mark.gpu
def test_all_scores_tied_fp4(gpu):
    """Every fp4 key decodes to zero: the selection is the k' lowest entry ids, scores 0."""
    cfg = D(C.C4A_1M_B4_FP4IDX, name="c4a_all_ties_fp4idx", ctx_after=(20000, 9000, 5), n_heads=16,
            k=700, stages=("index", "attn"))
    print(f"case {cfg.name}", flush=True)
    from compressed_sparse_long_c4a_amd import pipeline
    d = inputs.draw(cfg)
    _zero_fp4_keys(d)
    g = pipeline.to_device(d)
    step = pipeline.Step(cfg, g)
    step.run()
    torch.cuda.synchronize()
    topk, sc = step.topk.cpu().numpy(), step.topk_score.cpu().numpy()
    for i, t in enumerate(d["q_pos"].tolist()):
        kk = min(cfg.k, (t + 1) // 4)
        assert np.array_equal(topk[i, :kk], np.arange(kk)), i
        assert np.all(topk[i, kk:] == -1) and np.all(sc[i] == 0.0)
