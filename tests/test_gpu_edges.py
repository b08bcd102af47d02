"""Edge cases of the HIP path against the oracle: empty calls, the first positions of a sequence
(no entries yet, zero-padded entry 0, a one-row window), ragged batches, a zero window, exact
score ties, selections too large for the select kernel's LDS, and the largest k the ABI accepts.
"""

import dataclasses

import numpy as np
import pytest
import torch

from tests import pipeline_check as P
from workloads import configs as C, inputs

D = dataclasses.replace

# c4a decode of 8 sequences at the very start of their context: t = 0..4, 7, 8, 129 gives
# 0, 0, 0, 1, 1, 2, 2 and 32 visible entries (no entry, entry 0 with its zero-padded slots, k >= n
# and k < n); the window holds t + 1 rows.
EARLY_C4A = D(C.C4A_1M_B4_FP8, name="c4a_early_positions", ctx_after=(1, 2, 3, 4, 5, 8, 9, 130),
              n_heads=16, k=8)
# c128a: entries complete at positions 127 and 255 only.
EARLY_C128A = D(C.C128A_1M_B8, name="c128a_early_positions", ctx_after=(1, 127, 128, 129, 256, 300),
                n_heads=16)
# a ragged prefill batch: a sequence starting at position 0, one with three new tokens, one
# without queries, one whose chunk spans a block edge; every query sees its own chunk causally.
RAGGED = D(C.C4A_PREFILL_64K, name="c4a_ragged_prefill", ctx_after=(700, 1500, 300, 290),
           new_tokens=(300, 3, 300, 40), q_per_seq=(5, 3, 0, 40), k=64, n_heads=32)
# attention over top-k entries only (window 0); t = 2 has no row at all (out 0, lse -inf).
NO_WINDOW = D(C.C4A_1M_B4_FP8, name="c4a_window0", ctx_after=(3, 4097, 9000), n_heads=16, k=256,
              window=0, stages=("index", "attn"))


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [EARLY_C4A, EARLY_C128A, RAGGED, NO_WINDOW], ids=lambda c: c.name)
def test_edge_step_parity(gpu, cfg):
    print(f"case {cfg.name}: {cfg}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True)
    assert not rep["fail"], rep["fail"][:10]


def _zero_index_keys(d):
    rows, scales, bt = d["idx"]
    rows.zero_()
    if scales is not None:
        scales.fill_(1.0)


@pytest.mark.gpu
def test_all_scores_tied(gpu):
    """Every indexer key is zero, so every score is exactly 0: the selection must be the k'
    lowest entry ids (ties go to lower ids), with scores 0."""
    cfg = D(C.C4A_1M_B4_FP8, name="c4a_all_ties", ctx_after=(20000, 9000, 5), n_heads=16, k=700,
            stages=("index", "attn"))
    print(f"case {cfg.name}", flush=True)
    from compressed_sparse_long_c4a_amd import pipeline
    d = inputs.draw(cfg)
    _zero_index_keys(d)
    g = pipeline.to_device(d)
    step = pipeline.Step(cfg, g)
    step.run()
    torch.cuda.synchronize()
    topk = step.topk.cpu().numpy()
    sc = step.topk_score.cpu().numpy()
    for i, t in enumerate(d["q_pos"].tolist()):
        n = (t + 1) // 4
        kk = min(cfg.k, n)
        assert np.array_equal(topk[i, :kk], np.arange(kk)), i
        assert np.all(topk[i, kk:] == -1)
        assert np.all(sc[i] == 0.0)
    rep = P.run_step_parity(cfg, verbose=True, prep=_zero_index_keys)
    assert not rep["fail"], rep["fail"][:10]


@pytest.mark.gpu
@pytest.mark.parametrize("ctx,k", [(80000, 12000), (20000, 4500)], ids=["cand-beyond-lds", "bound-disabled"])
def test_large_selections(gpu, ctx, k):
    """More candidates than the select kernel holds in LDS (the global-memory path), and a k so
    large relative to n that the per-chunk bounds cannot filter (every entry is a candidate)."""
    cfg = D(C.C4A_128K_B32, name=f"c4a_large_k_{k}", ctx_after=(ctx, ctx - 3), n_heads=16, k=k)
    print(f"case {cfg.name}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True)
    assert not rep["fail"], rep["fail"][:10]


def _cluster_winners(d):
    """Scale the first 4,096 indexer keys of every sequence by 8 (their fp8 row scales), so
    nearly all of the top k lie in the first two 2,048-entry chunks: far more than those chunks'
    candidate quotas."""
    rows, scales, bt = d["idx"]
    for b in range(bt.shape[0]):
        for lb in range(64):  # 64 entries per logical block: blocks 0..63 hold entries 0..4095
            scales[int(bt[b, lb])] *= 8.0


@pytest.mark.gpu
def test_clustered_winners_take_the_full_scan(gpu):
    """When the winners crowd into a few chunks, the candidates' k'-th largest key falls below
    those chunks' bounds, so the select kernel must run its exact fallback over every stored
    score; the result must still be the oracle's top-k (fused compressor launch included)."""
    cfg = D(C.C4A_1M_B4_FP8, name="c4a_clustered_winners", ctx_after=(200000, 199999, 60000), k=1024)
    print(f"case {cfg.name}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True, prep=_cluster_winners, fast=True)
    assert not rep["fail"], rep["fail"][:10]



@pytest.mark.gpu
@pytest.mark.parametrize("clustered", [False, True], ids=["spread", "clustered"])
def test_select_past_128_chunks(gpu, clustered):
    """Contexts past 1M tokens (more than 128 chunks of 2,048 entries per query): the select
    kernel's candidate lists beyond those its first trip loads, on the candidate path and on
    the full-scan fallback."""
    cfg = D(C.C4A_1M_B4_FP8, name="c4a_select_wide", ctx_after=(1300000, 1100000), n_heads=16, k=2048)
    print(f"case {cfg.name} clustered={clustered}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True, prep=_cluster_winners if clustered else None, fast=True)
    assert not rep["fail"], rep["fail"][:10]

SLICE_CASES = [
    # ragged chunked prefill (the query-tiled score kernel when whole; a slice boundary cuts
    # through sequences and query tiles)
    D(C.C4A_PREFILL_64K, name="slices_prefill", ctx_after=(6000, 3000, 9000), new_tokens=(37, 3, 64),
      q_per_seq=(37, 3, 64), k=256, n_heads=16, stages=("index",)),
    # decode, one query per sequence
    D(C.C4A_1M_B4_FP8, name="slices_decode", ctx_after=(70000, 69999, 5000, 9), k=512, n_heads=16,
      stages=("index",)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", SLICE_CASES, ids=lambda c: c.name)
def test_index_topk_in_slices(gpu, cfg):
    """csa_index_topk with a workspace for fewer queries than the call takes them in slices
    (slices of 10, 3 and 1 queries, those smaller than the call): the ids and scores must equal
    the one-pass call's bit for bit, and the one-pass call must pass the oracle's top-k checks."""
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    from tests import oracle_step as O
    print(f"case {cfg.name}", flush=True)
    d = inputs.draw(cfg)
    g = pipeline.to_device(d)
    args = (g["cu_q"], g["q_pos"], g["q_idx"], g["head_w"], g["idx"], cfg.k, cfg.max_context)
    whole, whole_sc = csa.index_topk(*args, with_scores=True)
    torch.cuda.synchronize()
    nq = whole.shape[0]
    for per in [p for p in (10, 3, 1) if p < nq]:
        limit = csa.index_workspace_size(per, cfg.max_context, cfg.k)
        assert limit < csa.index_workspace_size(nq, cfg.max_context, cfg.k)
        part, part_sc = csa.index_topk(*args, with_scores=True, workspace_limit=limit)
        torch.cuda.synchronize()
        assert torch.equal(part, whole), f"ids differ with slices of {per}"
        assert torch.equal(part_sc, whole_sc), f"scores differ with slices of {per}"
    res = O.run_oracle(cfg, d)
    ids = whole.cpu().numpy()
    for i in range(nq):
        ok, why = O.topk_acceptable(ids[i], res["scores"][i], cfg.k)
        assert ok, f"query {i}: {why}"


@pytest.mark.gpu
def test_max_k(gpu):
    """k = 65536, the largest the ABI accepts, over a 300K-token context (75,000 entries): the
    index selection and an attention over 65,536 + 128 rows."""
    cfg = D(C.C4A_128K_B32, name="c4a_max_k", ctx_after=(300000,), n_heads=16, k=65536)
    print(f"case {cfg.name}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True)
    assert not rep["fail"], rep["fail"][:10]


@pytest.mark.gpu
def test_attention_list_padding_and_out_of_range_ids(gpu):
    """Attention-only with caller lists: -1 padding, ids past the causal limit and negative ids
    are skipped; repeated calls reuse one workspace."""
    cfg = D(C.C4A_128K_B32, name="c4a_attn_lists", ctx_after=(5000, 700, 64), n_heads=16, k=300,
            stages=("attn",))

    def prep(d):
        top = inputs.random_topk(cfg, d, fill=0.6)
        top[0, -5:] = torch.tensor([5000, 1 << 30, -7, 1249, 1250], dtype=torch.int32)  # n = 1250
        top[2, :] = -1                                                            # window only
        d["topk"] = top

    print(f"case {cfg.name}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True, prep=prep)
    assert not rep["fail"], rep["fail"][:10]


@pytest.mark.gpu
def test_empty_calls_launch_nothing(gpu):
    """total_q = 0 and total_new = total_entries = 0 are valid and return without launching."""
    import compressed_sparse_long_c4a_amd as csa
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    kv = csa.PagedCache(torch.zeros((2, 64, 576), dtype=torch.bfloat16, device=dev), torch.zeros((1, 1), **i32))
    sw = csa.PagedCache(torch.zeros((2, 256, 576), dtype=torch.bfloat16, device=dev), torch.zeros((1, 1), **i32))
    st = csa.PagedCache(torch.zeros((2, 256, 576), dtype=torch.bfloat16, device=dev), torch.zeros((1, 1), **i32))
    csa.compress_insert(4, torch.zeros(1, **i32), torch.zeros(2, **i32),
                        torch.zeros((0, 576), dtype=torch.bfloat16, device=dev), torch.zeros(2, **i32),
                        torch.zeros((0, 8), dtype=torch.float32, device=dev), st, kv, sw)
    q = torch.zeros((0, 16, 576), dtype=torch.bfloat16, device=dev)
    out, _ = csa.sparse_attn_decode(torch.zeros(2, **i32), torch.zeros(0, **i32), q, kv, 4,
                                    torch.zeros((0, 8), **i32), sw, 128, 0.04, 256)
    assert out.shape == (0, 16, 576)
    ic = csa.PagedCache(torch.zeros((2, 64, 128), dtype=torch.bfloat16, device=dev), torch.zeros((1, 1), **i32))
    topk, _ = csa.index_topk(torch.zeros(2, **i32), torch.zeros(0, **i32),
                             torch.zeros((0, 64, 128), dtype=torch.bfloat16, device=dev),
                             torch.zeros((0, 64), dtype=torch.float32, device=dev), ic, 8, 256)
    assert topk.shape == (0, 8)
    torch.cuda.synchronize()


@pytest.mark.gpu
@pytest.mark.parametrize("misalign", [False, True], ids=["aligned", "new-rows-2-bytes-off"])
def test_c128a_compress_row_alignment(gpu, misalign):
    """c128a entries from 128-row windows: with 16-byte aligned raw rows the compressor reads
    them with 16-byte loads, with raw rows 2 bytes off 16-byte alignment it falls back to
    element loads; both match the oracle's entries (rounded-row rule of tests/oracle_step)."""
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    from oracle import compress
    from tests import oracle_step as O
    cfg = D(C.C128A_1M_B8, name="c128a_compress_align", ctx_after=(1100, 700, 129, 5000),
            new_tokens=(600, 1, 129, 300), q_per_seq=0, n_heads=16, stages=("compress",), gamma=True)
    print(f"case {cfg.name} misaligned={misalign}", flush=True)
    d = inputs.draw(cfg)
    g = pipeline.to_device(d)
    raw = g["new_raw"]
    if misalign:
        buf = torch.empty(raw.numel() + 1, dtype=raw.dtype, device=raw.device)
        shifted = buf[1:].view(raw.shape)
        shifted.copy_(raw)
        raw = shifted
        assert raw.data_ptr() % 16 == 2 and raw.is_contiguous()
    csa.compress_insert(128, g["ctx_lens"], g["cu_new"], raw, g["cu_entries"], g["logits"], g["state"],
                        g["kv"], swa=None, gamma=g["gamma"], eps=cfg.eps, rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    kv_o, state_o = O.oracle_cache(d["kv"]), O.oracle_cache(d["state"])
    rv, rdt = O.raw_values(d["new_raw"])
    ent, _ = compress.compress_insert(128, d["ctx_lens"].tolist(), d["cu_new"].tolist(), rv, rdt,
                                      d["cu_entries"].tolist(), d["logits"].numpy(),
                                      d["gamma"].numpy().astype(np.float64), cfg.eps, cfg.rope_base, 64,
                                      state_o, kv_o, None)
    rows = g["kv"].rows.cpu()
    bt = d["kv"][2]
    assert len(ent) == int(d["cu_entries"][-1]) > 0
    for (b, j), c in ent.items():
        blk, slot = int(bt[b, j // 2]), j % 2
        gv = O.formats.decode_stored(O.np_rows(rows[blk, slot]), "bf16")
        ok, r = O.check_rounded_row(gv, c, "bf16")
        assert ok, f"entry {(b, j)}: err/tol {r:.3g}"
