"""The benchmark's algorithmic byte and flop counts (host logic, no GPU) against closed forms.

Keys and attention rows that several queries of one sequence share are counted once; flops are
counted per (query, row) visit."""

import dataclasses

import bench
from workloads import configs as C, inputs

D = dataclasses.replace


def _draw(cfg):
    return inputs.draw(cfg)


def test_decode_counts_one_query_per_sequence():
    cfg = C.scaled(C.C4A_1M_B4_FP8, (9220, 4099, 2562, 2049), k=256, n_heads=16)
    d = _draw(cfg)
    ab, fl = bench.algorithmic_bytes(cfg, d), bench.algorithmic_flops(cfg, d)
    n = [L // 4 for L in cfg.ctx_after]                  # the query sits at t = L - 1
    assert ab["index_score"] == sum(n) * 132 + 4 * 64 * (128 * 2 + 4)
    rows = sum(min(256, x) + 128 for x in n)
    assert ab["attn"] == rows * 580 + 4 * 16 * (576 * 2 + 576 * 4 + 4)
    assert fl["index_score"] == 2 * 64 * 128 * sum(n)
    assert fl["attn"] == 4 * 16 * 576 * rows


def test_shared_keys_and_rows_count_once():
    cfg = D(C.C4A_1M_B4_FP8, name="acct_multi", ctx_after=(8200,), new_tokens=8, q_per_seq=8, k=256,
            n_heads=16)
    d = _draw(cfg)
    ab, fl = bench.algorithmic_bytes(cfg, d), bench.algorithmic_flops(cfg, d)
    ts = range(8192, 8200)
    n = [(t + 1) // 4 for t in ts]
    # one sequence: the keys of its latest query once; the queries' blocks each
    assert ab["index_score"] == max(n) * 132 + 8 * 64 * (128 * 2 + 4)
    # entries: at most the sequence's entries; window: positions 8192 - 127 .. 8199
    rows = min(max(n), 8 * 256) + (8199 - (8192 - 127) + 1)
    assert ab["attn"] == rows * 580 + 8 * 16 * (576 * 2 + 576 * 4 + 4)
    # flops per visit
    assert fl["index_score"] == 2 * 64 * 128 * sum(n)
    assert fl["attn"] == 4 * 16 * 576 * sum(min(256, x) + 128 for x in n)
