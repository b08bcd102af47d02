"""The compressors inside the index-score launch (csa_compress_index_score, the step's fast
path): the score workgroups skip the entries the step inserts, the indexer-key compressor scores
them, and the whole step must still match the oracle (rules of tests/pipeline_check.py).

Cases: the 1M fp8 decode's shapes at shorter contexts; sequences whose new entry opens a chunk
(no entry of that chunk existed before: the score workgroup only writes padding) or closes a
full chunk (the chunk bound counts 2,047 scored entries); a k so large that the full chunk's
bound needs more entries than were scored (bound 0); the first positions of a sequence (entry 0
new); an fp4 indexer cache; several queries over several new tokens per sequence, ragged.
"""

import dataclasses

import pytest

from tests import pipeline_check as P
from workloads import configs as C

D = dataclasses.replace

CASES = {
    "decode_fp8": C.scaled(C.C4A_1M_B4_FP8, (9220, 4099, 2562, 2049), k=256, name_suffix="fused"),
    # 8196: entry 2048 opens chunk 1; 16384: entry 4095 closes the full chunk 1
    "chunk_edges": D(C.C4A_1M_B4_FP8, name="fused_chunk_edges", ctx_after=(8196, 16384, 16383, 12),
                     k=256, n_heads=16),
    # k' = 4095 of n = 4096: kc = 2048 > the 2,047 scored entries of the full chunk
    "bound_zero": D(C.C4A_1M_B4_FP8, name="fused_bound_zero", ctx_after=(16384, 16380), k=4095,
                    n_heads=16),
    "early": D(C.C4A_1M_B4_FP8, name="fused_early", ctx_after=(1, 2, 3, 4, 5, 8, 9, 130), n_heads=16,
               k=8),
    "fp4_indexer": C.scaled(C.C4A_1M_B4_FP4IDX, (9220, 4099, 2562, 2049), k=256, name_suffix="fused"),
    # several queries per sequence over several new tokens: a new entry is seen by the queries at
    # or after its anchor only (9220: the last query; 4099: all four)
    "multi_query": D(C.C4A_1M_B4_FP8, name="fused_multi_query", ctx_after=(9220, 4099, 2562, 2049),
                     new_tokens=4, q_per_seq=4, k=256, n_heads=16),
    # ragged: two entries in one sequence, none in another, queries fewer than new tokens
    "ragged": D(C.C4A_1M_B4_FP8, name="fused_ragged", ctx_after=(8200, 4099, 2563, 2049),
                new_tokens=(8, 5, 3, 1), q_per_seq=(8, 2, 3, 1), k=256, n_heads=16),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_fused_step_parity(gpu, name):
    cfg = CASES[name]
    print(f"case {name}: {cfg}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True, fast_only=True, with_scores=True)
    assert not rep["fail"], rep["fail"][:10]
    assert rep["checked"].get("topk", 0) > 0
