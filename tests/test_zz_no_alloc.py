"""csa_sparse_attn_decode_noalloc (the library's own scratch, no workspace) on the GPU.

Two calls in a row through the C ABI, the second on a smaller input (fewer queries, heads and
rows), each compared element by element with csa_sparse_attn_decode on the same inputs with a
caller workspace: the outputs and log-sum-exps must agree to the attention tolerance
(1e-5 + 2e-3 relative; the two share their kernels and launch plan, so they are expected to be
bit-identical, and that is checked too).  (The refusal of a request beyond the array's 16 MiB
is a host-side check, tested on the CPU in tests/test_abi_cpu.py.)
"""

import dataclasses

import pytest
import torch

from tests import oracle_step as O
from workloads import configs as C, inputs

D = dataclasses.replace

CALLS = [
    # the 1M decode's attention shape (128 heads, k = 2048, fp8 rows) on shorter contexts
    D(C.C4A_1M_B4_FP8, name="noalloc_fp8_b4_h128", ctx_after=(40000, 39999, 39998, 30001), k=2048,
      stages=("attn",)),
    # then a smaller one: two queries, 64 heads, bf16 rows, k = 256
    D(C.C4A_128K_B32, name="noalloc_bf16_b2_h64", ctx_after=(9000, 1203), k=256, stages=("attn",)),
]


def _call_pair(csa, cfg):
    from compressed_sparse_long_c4a_amd import pipeline
    d = inputs.draw(cfg)
    topk = inputs.random_topk(cfg, d, fill=0.95).cuda()
    g = pipeline.to_device(d)
    L = csa.lib()
    total_q, H, Dm = g["q"].shape
    B = g["cu_q"].shape[0] - 1
    common = (B, g["cu_q"].data_ptr(), g["q_pos"].data_ptr(), total_q, cfg.max_context, g["q"].data_ptr(),
              csa.dtype_code(g["q"].dtype), H, csa._cref(g["kv"]), cfg.ratio, topk.data_ptr(), cfg.k,
              csa._cref(g["swa"]), cfg.window, cfg.softmax_scale, cfg.rope_base, 64)
    out_ref = torch.full((total_q, H, Dm), float("nan"), device="cuda")
    lse_ref = torch.full((total_q, H), float("nan"), device="cuda")
    nws = L.csa_sparse_attn_workspace_size(total_q, H, Dm, cfg.ratio, 1, cfg.k, cfg.max_context, cfg.window)
    assert 0 < nws <= 16 << 20, nws
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    st = L.csa_sparse_attn_decode(csa._stream(), *common, out_ref.data_ptr(), lse_ref.data_ptr(),
                                  ws.data_ptr(), nws)
    assert st == csa.OK, st
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    st = L.csa_sparse_attn_decode_noalloc(csa._stream(), *common, out.data_ptr(), lse.data_ptr())
    assert st == csa.OK, st
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), out_ref.cpu().numpy(), lse_ref.cpu().numpy(), nws


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point(gpu):
    csa = gpu
    for cfg in CALLS:  # in this order: the second call is the smaller one
        print(f"case {cfg.name}", flush=True)
        out, lse, out_ref, lse_ref, nws = _call_pair(csa, cfg)
        ok, r = O.allclose_out(out, out_ref)
        assert ok, f"{cfg.name}: out err/tol {r:.3g}"
        ok, r = O.allclose_out(lse, lse_ref)
        assert ok, f"{cfg.name}: lse err/tol {r:.3g}"
        same = bool((out == out_ref).all() and (lse == lse_ref).all())
        print(f"  scratch {nws} bytes; bit-identical to the workspace call: {same}", flush=True)
        assert same
