"""The step captured in a HIP graph (as the benchmark replays it) gives exactly the eager step's
outputs on every replay, with eager work and synchronisations between the replays.

The graph holds only the library's own launches (no memset nodes).  Before each replay the
outputs are overwritten eagerly with values no step produces, so a replay that skipped or
reordered a launch shows up as a mismatch.  A replay repeats the same step on the same caches:
the compressor writes the same rows to the same places, so every replay must match bit for bit.
"""

import dataclasses

import pytest
import torch

from workloads import configs as C, inputs

D = dataclasses.replace

CASES = [
    # the 1M-context fp8 decode at a shorter context (every stage: compress, index, attention)
    D(C.C4A_1M_B4_FP8, name="c4a_fp8_decode_graph", ctx_after=(40000, 39999, 39998, 39997)),
    # c128a: compress and attention over every causal entry, no index stage
    D(C.C128A_1M_B8, name="c128a_decode_graph", ctx_after=(70000, 65536, 300, 129)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_graph_replays_match_eager(gpu, cfg):
    from compressed_sparse_long_c4a_amd import pipeline
    print(f"case {cfg.name}", flush=True)
    g = pipeline.to_device(inputs.draw(cfg))
    step = pipeline.Step(cfg, g, with_scores=False)
    step.fast(g)
    torch.cuda.synchronize()
    ref_out = step.out.clone()
    ref_topk = step.topk.clone() if step.topk is not None else None

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.fast(g)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.fast(g)
    torch.cuda.synchronize()

    for rep in range(4):
        step.out.fill_(float("nan"))
        if step.topk is not None:
            step.topk.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out), f"replay {rep}: attention output differs"
        if ref_topk is not None:
            assert torch.equal(step.topk, ref_topk), f"replay {rep}: top-k differs"
        step.fast(g)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out)
