"""csa_q_norm_rope_swa on the GPU against the oracle (oracle/qnorm.py), element by element.

Every query head of every query is compared with the oracle's float64 result as a rounding of
it (tests/oracle_step.check_rounded_row: half an ulp of the stored dtype plus the float32
accuracy of the kernel); every window row it writes is compared the same way in the window
cache's dtype (fp8: codes and scales).  The window rows must also equal, bit for bit, the rows
the compressor writes for the same new tokens when it is given the window cache.
"""

import dataclasses

import numpy as np
import pytest
import torch

from tests import oracle_step as O
from workloads import configs as C, inputs

D = dataclasses.replace

CASES = [
    # the 1M fp8 decode's shapes (128 heads x 576, fp8 window cache) at a shorter context
    D(C.C4A_1M_B4_FP8, name="qnorm_fp8_decode", ctx_after=(40000, 39999, 39998, 39997)),
    # a ragged bf16 prefill: several new rows and queries per sequence, one sequence at
    # position 0, one without queries, rows crossing a 256-position block edge
    D(C.C4A_PREFILL_64K, name="qnorm_bf16_ragged", ctx_after=(700, 1500, 300, 290),
      new_tokens=(300, 3, 300, 40), q_per_seq=(5, 3, 0, 40), n_heads=16),
    # float32 queries and raw rows (the 1k reference workload)
    D(C.REF, name="qnorm_f32_ref"),
]


def _gamma(dim, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(dim, generator=g, dtype=torch.float64) + 0.5).to(torch.float32)


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_q_norm_rope_swa_parity(gpu, cfg):
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    from oracle.qnorm import q_norm_rope_swa as oracle_fn
    print(f"case {cfg.name}", flush=True)
    d = inputs.draw(cfg)
    g = pipeline.to_device(d)
    gamma = _gamma(cfg.dim, 7)
    q_out = csa.q_norm_rope_swa(g["q_pos"], g["q"], gamma=gamma.cuda(), eps=cfg.eps,
                                rope_base=cfg.rope_base, rope_dims=64, ctx_lens=g["ctx_lens"],
                                cu_new=g["cu_new"], new_raw=g["new_raw"], swa=g["swa"])
    torch.cuda.synchronize()

    swa_o = O.oracle_cache(d["swa"])
    q_np, q_dt = O.raw_values(d["q"])
    raw_np, raw_dt = O.raw_values(d["new_raw"])
    want_q, want_rows = oracle_fn(d["q_pos"].numpy(), q_np, q_dt, gamma.numpy(), cfg.eps,
                                  cfg.rope_base, 64, d["ctx_lens"].numpy(), d["cu_new"].numpy(),
                                  raw_np, raw_dt, swa_o)
    got_q = O.formats.decode_stored(O.np_rows(q_out.cpu()), q_dt)
    worst = 0.0
    for i in range(got_q.shape[0]):
        for h in range(got_q.shape[1]):
            ok, r = O.check_rounded_row(got_q[i, h], want_q[i, h], q_dt)
            worst = max(worst, r)
            assert ok, f"query {i} head {h}: err/tol {r:.3g}"
    rows, scales, bt = d["swa"]
    g_rows = g["swa"].rows.cpu()
    g_scales = None if g["swa"].scales is None else g["swa"].scales.cpu()
    fmt = O.DT[rows.dtype]
    for (b, p), v in want_rows.items():
        blk, slot = int(bt[b, p // 256]), p % 256
        gs = None if g_scales is None else float(g_scales[blk, slot])
        gv = O.formats.decode_stored(O.np_rows(g_rows[blk, slot]), fmt,
                                     None if gs is None else np.float32(gs))
        oblk, oslot = swa_o.locate(b, p)
        os_ = None if swa_o.scales is None else float(swa_o.scales[oblk, oslot])
        ok, r = O.check_rounded_row(gv, v, fmt, gs, os_)
        worst = max(worst, r)
        assert ok, f"window row {(b, p)}: err/tol {r:.3g}"
    assert len(want_rows) == int(d["cu_new"][-1])
    print(f"  {got_q.shape[0] * got_q.shape[1]} query heads, {len(want_rows)} window rows; "
          f"worst err/tol {worst:.3f}", flush=True)


@pytest.mark.gpu
def test_window_rows_match_the_compressor(gpu):
    """The same new tokens through the compressor's window output and through this kernel give
    bit-identical window caches."""
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    cfg = D(C.C4A_PREFILL_64K, name="qnorm_vs_compress", ctx_after=(700, 1500, 300, 290),
            new_tokens=(300, 3, 300, 40), q_per_seq=(5, 3, 0, 40), n_heads=16, kv_dtype="fp8")
    print(f"case {cfg.name}", flush=True)
    d = inputs.draw(cfg)
    g = pipeline.to_device(d)
    swa_a = g["swa"]
    swa_b = csa.PagedCache(swa_a.rows.clone(), swa_a.block_table,
                           None if swa_a.scales is None else swa_a.scales.clone())
    csa.compress_insert(4, g["ctx_lens"], g["cu_new"], g["new_raw"], g["cu_entries"], g["logits"],
                        g["state"], g["kv"], swa=swa_a, gamma=g.get("gamma"), eps=cfg.eps,
                        rope_base=cfg.rope_base)
    csa.q_norm_rope_swa(g["q_pos"], g["q"], eps=cfg.eps, rope_base=cfg.rope_base,
                        ctx_lens=g["ctx_lens"], cu_new=g["cu_new"], new_raw=g["new_raw"], swa=swa_b)
    torch.cuda.synchronize()
    assert torch.equal(swa_a.rows, swa_b.rows)
    if swa_a.scales is not None:
        assert torch.equal(swa_a.scales, swa_b.scales)
