"""Parity at the full sizes of the five workloads, launched exactly as bench.py launches a step.

Each case draws the workload at its real shape (1M-token contexts, 128 heads, top-k 2048, ...),
runs the step through the same pre-marshalled C calls the benchmark times (no top-k scores, no
lse), and compares with the oracle on every output it can compute one by one in seconds:
every compressed entry, window row and state row the step writes; for the sampled queries the
whole score vector (exact top-k acceptance) and the attention output over the GPU's selection.
"""

import pytest

from tests import pipeline_check as P
from workloads import configs as C

# workload -> queries checked (None = every query of the step)
FULL = {
    "ref_c4a_1k_fp32": (C.REF, None),
    "c4a_decode_128k_b32_bf16": (C.C4A_128K_B32, None),
    "c128a_decode_1m_b8_bf16": (C.C128A_1M_B8, None),
    "c4a_decode_1m_b4_fp8": (C.C4A_1M_B4_FP8, None),
    # the same decode with the indexer cache in fp4 (72-byte keys)
    "c4a_decode_1m_b4_fp8_fp4idx": (C.C4A_1M_B4_FP4IDX, None),
    # first and last queries of the chunk, each residue mod 4 at both ends, block edges
    "c4a_prefill_4k_on_64k_bf16": (C.C4A_PREFILL_64K, [0, 1, 2, 3, 252, 255, 256, 1023, 2048, 3071,
                                                       4092, 4093, 4094, 4095]),
}


@pytest.mark.gpu
@pytest.mark.slow
@pytest.mark.parametrize("name", list(FULL))
def test_full_size_parity(gpu, name):
    cfg, queries = FULL[name]
    print(f"case {name} (full size, benchmark launch sequence): {cfg}", flush=True)
    rep = P.run_step_parity(cfg, queries=queries, verbose=True, fast=True, with_scores=False)
    assert not rep["fail"], rep["fail"][:10]
    assert rep["checked"].get("out", 0) > 0
