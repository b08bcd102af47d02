"""Pins of the row-size arithmetic and entry counts against the numbers the pages print (CPU only).

The printed values, each with its citation, live in tests/golden/page_numbers.json.  (The
[SGLang-pools] 78.2 KB figure for a 16-bit MLA part mixes decimal and binary kilobytes, so it is
not used as a pin.)
"""

import json
import os

from oracle import geometry, sizes

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def val(key):
    return GOLDEN[key]["value"]


def test_golden_entries_cite_a_page():
    for key, entry in GOLDEN.items():
        if not key.startswith("_"):
            assert entry["cite"].startswith("["), key


def test_sglang_rows():
    assert sizes.row_bytes(val("mla_row_values"), "bf16") == val("mla_row_bytes_bf16")
    layers = GOLDEN["deepseek_v2_kb_per_token"]["layers"]
    assert abs(sizes.mla_bytes_per_token(layers, "bf16") / 1024 - val("deepseek_v2_kb_per_token")) < 1e-9
    assert sizes.row_bytes(128, "fp8", 128) == val("indexer_row_bytes")
    layers = GOLDEN["deepseek_v3_fp8_bytes_per_token"]["layers"]
    assert sizes.dsa_bytes_per_token(layers, "fp8") == val("deepseek_v3_fp8_bytes_per_token")


def test_v4_memory_totals():
    v4 = sizes.per_sequence_gib(sizes.v4_bytes_per_token())
    v32 = sizes.per_sequence_gib(sizes.v32_bytes_per_token())
    assert round(v4, 2) == val("v4_gib_per_1m_sequence")
    assert round(v32, 1) == val("v32_gib_per_1m_sequence")
    assert round(v32 / v4, 1) == val("v4_over_v32_ratio")
    assert round(100 * (1 - v4 / v32), 1) == val("v4_percent_smaller")


def test_entry_counts():
    assert geometry.entries_per_block(4) == val("c4a_entries_per_256_block")
    assert geometry.entries_per_block(128) == val("c128a_entries_per_256_block")
    # the pages round these two; the exact counts are within 5%
    assert abs(geometry.num_entries(1 << 20, 4) / val("c4a_entries_at_1m_approx") - 1) < 0.05
    assert abs(geometry.num_entries(1 << 20, 128) / val("c128a_entries_at_1m_approx") - 1) < 0.05
    # c128a framed as top-k 8192 covers every entry of a 2^20-token sequence exactly
    assert geometry.num_entries(1 << 20, 128) == val("c128a_topk")
