"""csa_sparse_attn_decode_fp8 (inverse RoPE + fp8 output rows in one launch) on the GPU.

Three checks per case, on every (query, head) row:
* the float32 rows it returns beside the codes match the oracle's attention (the tolerance of
  every attention test: 1e-5 + 2e-3 relative) and equal, bit for bit, what
  csa_sparse_attn_decode returns for the same inputs;
* the fp8 codes and scale of each row are the oracle's row quantiser (oracle.attention.
  output_fp8) applied to that float32 row, compared as roundings (tests/oracle_step.
  check_rounded_row: half an E4M3 step plus float32 accuracy; scales to 1e-6);
* a call without the float32 rows writes the same codes and scales.
"""

import dataclasses

import numpy as np
import pytest
import torch

from tests import oracle_step as O
from workloads import configs as C, inputs

D = dataclasses.replace

CASES = [
    # fp8 caches and 128 heads at the 1M decode's shapes (shorter context), caller top-k lists
    D(C.C4A_1M_B4_FP8, name="attn_fp8out_c4a_fp8", ctx_after=(40000, 39999, 9000, 3), k=512,
      stages=("attn",)),
    # bf16 caches, c128a (every causal entry), window 128
    D(C.C128A_1M_B8, name="attn_fp8out_c128a_bf16", ctx_after=(70000, 300, 129, 1),
      stages=("attn",)),
    # many queries with few rows each: one split per query, so csa_sparse_attn_decode finishes
    # the rows in the partial kernel while the fp8 entry point merges; the float32 rows of the
    # two must agree bit for bit (fp8 rows, then bf16 rows)
    D(C.C4A_1M_B4_FP8, name="attn_fp8out_one_split_fp8", ctx_after=(40000, 39999, 9000, 300),
      new_tokens=64, q_per_seq=64, n_heads=16, k=256, stages=("attn",)),
    D(C.C4A_PREFILL_64K, name="attn_fp8out_one_split_bf16", ctx_after=(2048 + 256,), new_tokens=256,
      q_per_seq=256, k=128, stages=("attn",)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_attention_fp8_output(gpu, cfg):
    import compressed_sparse_long_c4a_amd as csa
    from compressed_sparse_long_c4a_amd import pipeline
    from oracle.attention import output_fp8
    print(f"case {cfg.name}", flush=True)
    d = inputs.draw(cfg)
    topk = inputs.random_topk(cfg, d, fill=0.9) if cfg.ratio == 4 else None
    g = pipeline.to_device(d)
    tk = None if topk is None else topk.cuda()
    args = (g["cu_q"], g["q_pos"], g["q"], g["kv"], cfg.ratio, tk, g["swa"], cfg.window,
            cfg.softmax_scale, cfg.max_context)
    codes, scales, out32, _ = csa.sparse_attn_decode_fp8(*args, with_f32=True)
    codes2, scales2, none32, _ = csa.sparse_attn_decode_fp8(*args)
    plain, _ = csa.sparse_attn_decode(*args)
    torch.cuda.synchronize()
    assert none32 is None
    assert torch.equal(out32, plain), "float32 rows differ from csa_sparse_attn_decode"
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)

    # float32 rows against the oracle's attention
    caches = O.prepare(d)
    out32 = out32.cpu().numpy()
    worst = 0.0
    for i in range(out32.shape[0]):
        ids = None if topk is None else topk[i].numpy()
        want, _ = O.attend_query(cfg, d, caches, i, ids)
        ok, r = O.allclose_out(out32[i], want)
        worst = max(worst, r)
        assert ok, f"query {i}: err/tol {r:.3g}"
    # fp8 rows against the oracle's quantiser applied to the same float32 rows
    ref_codes, ref_scales = output_fp8(out32.astype(np.float64))
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    wq = 0.0
    for i in range(out32.shape[0]):
        for h in range(out32.shape[1]):
            gv = O.formats.fp8_e4m3_to_f64(codes[i, h]) * np.float64(scales[i, h])
            ok, r = O.check_rounded_row(gv, out32[i, h].astype(np.float64), "fp8",
                                        scales[i, h], ref_scales[i, h])
            wq = max(wq, r)
            assert ok, f"query {i} head {h}: fp8 row err/tol {r:.3g}"
    same = float(np.mean(codes == ref_codes))
    print(f"  attention worst err/tol {worst:.3f}; fp8 rows worst err/tol {wq:.3f}, "
          f"{100 * same:.4f}% codes identical to the oracle's", flush=True)
