"""Whole-step parity on the GPU: the HIP library against the oracle on reduced workloads.

Each case runs every stage of its workload (compress, index/top-k, attention) through the C
ABI on identical seeded inputs and applies the acceptance rules of tests/pipeline_check.py.
"""

import dataclasses
import pytest

from tests import pipeline_check as P
from workloads import configs as C

CASES = {
    "ref_c4a_fp32": C.REF,
    "c4a_fp8_decode": P.SMALL_DECODE,
    "c4a_bf16_decode": C.scaled(C.C4A_128K_B32, (20480, 12288, 8191, 4102), k=512),
    "c128a_bf16_decode": C.scaled(C.C128A_1M_B8, (16384, 8192, 19456 - 1000, 300), gamma=True),
    "c4a_bf16_prefill": C.scaled(C.C4A_PREFILL_64K, (2048 + 512,), new_tokens=512, q_per_seq=512, k=128),
    # fp8 caches, four new tokens and four queries per sequence (queries see the step's own
    # entries and window rows, some in a block the step opens)
    "c4a_fp8_multi_query": dataclasses.replace(P.SMALL_DECODE, name="c4a_fp8_multi_query", new_tokens=4,
                                               q_per_seq=4, n_heads=16),
    # fp8 caches, a 64-token chunk per sequence: each query's rows are one split, finished by
    # the partial kernel without the merge
    "c4a_fp8_chunk": dataclasses.replace(P.SMALL_DECODE, name="c4a_fp8_chunk", new_tokens=64, q_per_seq=64,
                                         n_heads=16),
    # the query-tiled score kernel with bf16 indexer keys and 24 indexer heads (a partial head
    # tile): ragged query counts per sequence (tiles of four queries ending early, a sequence of
    # one query), the longest sequence spanning three chunks of entries (the last one ragged)
    "c4a_bf16idx_ragged_prefill": C.scaled(C.C4A_PREFILL_64K, (4800, 2100, 16800), new_tokens=(9, 1, 16),
                                           q_per_seq=(9, 1, 16), idx_dtype="bf16", idx_heads=24, k=128,
                                           n_heads=16),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_step_parity(gpu, name):
    cfg = CASES[name]
    print(f"case {name}: {cfg}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True)
    assert not rep["fail"], rep["fail"][:10]


@pytest.mark.gpu
def test_two_stream_schedule_parity(gpu):
    """The main-KV compressor on a second stream, concurrent with the indexer pipeline."""
    cfg = P.SMALL_DECODE
    print(f"case two-stream: {cfg.name}", flush=True)
    rep = P.run_step_parity(cfg, verbose=True, overlap=True)
    assert not rep["fail"], rep["fail"][:10]
