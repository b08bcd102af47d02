"""Robustness of the HIP path beyond single-call parity (GPU).

* Chunk invariance ([vLLM-V4] section 3 part 1: the compressor state is what a call hands to
  the next, so a prefix can be resumed at any position): the same raw token stream fed to the
  compressors in one call, or token by token, or in chunks of 3, 255, 256 or 257 tokens, leaves
  bit-identical compressed entries (main KV and indexer keys, codes and scales), window rows,
  and live compressor state (the last coff * ratio raw rows of every sequence).
* Split-count consistency: the same attention queries computed alone, in a batch of four and
  in a batch of 32 copies are planned with different numbers of row splits per query (17, 6 and
  3 for the 128-head fp8 case; 5, 5 and 2 for the 64-head bf16 one); their outputs and
  log-sum-exps must agree to the attention tolerance (1e-5 + 2e-3 relative), and with the
  oracle; copies of one query in one call are identical.
"""

import dataclasses

import numpy as np
import pytest
import torch

from tests import oracle_step as O
from workloads import configs as C, inputs

D = dataclasses.replace


def _run_chunked(cfg, d, chunk):
    """Feed every sequence's raw stream (all of d's new tokens, from position 0) in calls of at
    most `chunk` tokens per sequence; returns the caches afterwards (GPU)."""
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    g = pipeline.to_device(d)
    R = cfg.ratio
    B = cfg.batch
    L = list(cfg.ctx_after)
    cu_new = d["cu_new"].tolist()
    cu_ent = d["cu_entries"].tolist()
    done = [0] * B
    while any(done[b] < L[b] for b in range(B)):
        n_b = [min(chunk, L[b] - done[b]) for b in range(B)]
        raw, idx_raw, lg, ilg, ents = [], [], [], [], []
        for b in range(B):
            s0 = cu_new[b] + done[b]
            raw.append(g["new_raw"][s0:s0 + n_b[b]])
            if "compress_idx" in cfg.stages:
                idx_raw.append(g["new_idx_raw"][s0:s0 + n_b[b]])
            e0, e1 = done[b] // R, (done[b] + n_b[b]) // R
            ents.append(e1 - e0)
            lg.append(g["logits"][cu_ent[b] + e0:cu_ent[b] + e1])
            if "compress_idx" in cfg.stages:
                ilg.append(g["idx_logits"][cu_ent[b] + e0:cu_ent[b] + e1])
        ctx = torch.tensor(done, dtype=torch.int32, device="cuda")
        cn = torch.tensor([0] + list(np.cumsum(n_b)), dtype=torch.int32, device="cuda")
        ce = torch.tensor([0] + list(np.cumsum(ents)), dtype=torch.int32, device="cuda")
        new_raw = torch.cat(raw).contiguous()
        jobs = [csa.CompressJob(R, new_raw, ce, torch.cat(lg).contiguous(), g["state"], g["kv"], g["swa"],
                                None, cfg.eps, cfg.rope_base, 64)]
        if "compress_idx" in cfg.stages:
            jobs.append(csa.CompressJob(4, torch.cat(idx_raw).contiguous(), ce, torch.cat(ilg).contiguous(),
                                        g["idx_state"], g["idx"], None, None, cfg.eps, cfg.rope_base, 64))
        csa.compress_insert_many(ctx, cn, new_raw.shape[0], jobs)
        done = [done[b] + n_b[b] for b in range(B)]
    torch.cuda.synchronize()
    return g


def _cache_rows(c, bt_rows, rows_per_block, positions):
    """Stored rows (and scales) of the given logical rows of one sequence's cache, CPU."""
    blk = bt_rows[np.asarray(positions) // rows_per_block]
    slot = np.asarray(positions) % rows_per_block
    r = c.rows.cpu()[blk, slot]
    s = None if c.scales is None else c.scales.cpu()[blk, slot]
    return r, s


CHUNK_CASES = [
    # c4a: fp8 main KV and window rows, fp8 indexer keys, bf16 raw rows; two ragged sequences
    D(C.C4A_1M_B4_FP8, name="chunks_c4a_fp8", ctx_after=(1029, 600), new_tokens=(1029, 600),
      q_per_seq=1, stages=("compress", "compress_idx", "index")),
    # c128a: bf16 main KV, a 128-row compressor window
    D(C.C128A_1M_B8, name="chunks_c128a_bf16", ctx_after=(1029, 300), new_tokens=(1029, 300), q_per_seq=1,
      stages=("compress",)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CHUNK_CASES, ids=lambda c: c.name)
def test_chunk_invariance(gpu, cfg):
    print(f"case {cfg.name}", flush=True)
    d = inputs.draw(cfg)
    ref = _run_chunked(cfg, d, max(cfg.ctx_after))           # one call
    R = cfg.ratio
    Wc = 8 if R == 4 else 128
    for chunk in (1, 3, 255, 256, 257):
        print(f"  chunks of {chunk}", flush=True)
        got = _run_chunked(cfg, d, chunk)
        for b, Lb in enumerate(cfg.ctx_after):
            checks = [("kv", 256 // R, range(Lb // R)), ("swa", 256, range(Lb)),
                      ("state", 256, range(max(0, Lb - Wc), Lb))]
            if "compress_idx" in cfg.stages:
                checks += [("idx", 64, range(Lb // 4)), ("idx_state", 256, range(max(0, Lb - 8), Lb))]
            for name, rpb, pos in checks:
                bt = ref[name].block_table.cpu().numpy()[b]
                r0, s0 = _cache_rows(ref[name], bt, rpb, list(pos))
                r1, s1 = _cache_rows(got[name], bt, rpb, list(pos))
                assert torch.equal(r0, r1), f"{name} rows differ (seq {b}, chunks of {chunk})"
                if s0 is not None:
                    assert torch.equal(s0, s1), f"{name} scales differ (seq {b}, chunks of {chunk})"


def _attend(csa, g, cfg, sel, reps=1):
    """Attention of the queries `sel` (indices into g's queries), each repeated `reps` times in
    its sequence, in one call; returns (out, lse) on the CPU, one row per (selected query, copy)."""
    cu = g["cu_q"].tolist()
    seq = [b for b in range(len(cu) - 1) for _ in range(cu[b + 1] - cu[b])]
    order = [i for i in sel for _ in range(reps)]
    counts = [sum(1 for i in order if seq[i] == b) for b in range(len(cu) - 1)]
    order.sort(key=lambda i: seq[i])
    idx = torch.tensor(order, device="cuda")
    cu_q = torch.tensor([0] + list(np.cumsum(counts)), dtype=torch.int32, device="cuda")
    q_pos = g["q_pos"][idx].contiguous()
    q = g["q"][idx].contiguous()
    topk = g["topk_dev"][idx].contiguous()
    out, lse = csa.sparse_attn_decode(cu_q, q_pos, q, g["kv"], cfg.ratio, topk, g["swa"], cfg.window,
                                      cfg.softmax_scale, cfg.max_context, cfg.rope_base, 64, with_lse=True)
    torch.cuda.synchronize()
    return order, out.cpu().numpy(), lse.cpu().numpy()


SPLIT_CASES = [
    # fp8 rows, 128 heads, k = 2048: the 1M decode's attention shape on shorter contexts
    D(C.C4A_1M_B4_FP8, name="splits_fp8_h128", ctx_after=(40000, 39999, 39998, 39997), k=2048,
      stages=("attn",)),
    # bf16 rows, 64 heads, k = 512 (the generic kernel)
    D(C.C4A_128K_B32, name="splits_bf16_h64", ctx_after=(30000, 29999, 29998, 29997), k=512,
      stages=("attn",)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", SPLIT_CASES, ids=lambda c: c.name)
def test_split_count_consistency(gpu, cfg):
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    print(f"case {cfg.name}", flush=True)
    d = inputs.draw(cfg)
    topk = inputs.random_topk(cfg, d, fill=1.0)
    g = pipeline.to_device(d)
    g["topk_dev"] = topk.cuda()
    nq = d["q_pos"].shape[0]
    results = {}
    # four queries in one call; each query alone; 32 copies (8 of each query) in one call
    order, out4, lse4 = _attend(csa, g, cfg, list(range(nq)))
    results["batch4"] = {i: (out4[r], lse4[r]) for r, i in enumerate(order)}
    alone = {}
    for i in range(nq):
        _, o1, l1 = _attend(csa, g, cfg, [i])
        alone[i] = (o1[0], l1[0])
    results["alone"] = alone
    order, o32, l32 = _attend(csa, g, cfg, list(range(nq)), reps=8)
    results["batch32"] = {}
    for r, i in enumerate(order):
        results["batch32"].setdefault(i, []).append((o32[r], l32[r]))
    caches = O.prepare(d)
    worst = 0.0
    for i in range(nq):
        want, want_lse = O.attend_query(cfg, d, caches, i, topk[i].numpy())
        variants = [("batch4", *results["batch4"][i]), ("alone", *results["alone"][i])]
        variants += [(f"batch32[{c}]", o, l) for c, (o, l) in enumerate(results["batch32"][i])]
        for name, o, l in variants:
            ok, r = O.allclose_out(o, want)
            worst = max(worst, r)
            assert ok, f"query {i} {name}: out err/tol {r:.3g} against the oracle"
            ok, r = O.allclose_out(l, want_lse)
            assert ok, f"query {i} {name}: lse err/tol {r:.3g}"
            ok, r = O.allclose_out(o, variants[0][1])
            assert ok, f"query {i} {name}: out err/tol {r:.3g} against the four-query call"
        # copies in one call take the same plan and the same kernels: identical rows
        for c, (o, l) in enumerate(results["batch32"][i][1:]):
            assert np.array_equal(o, results["batch32"][i][0][0]), f"query {i} copy {c + 1} differs"
    print(f"  worst err/tol against the oracle {worst:.3f}", flush=True)
