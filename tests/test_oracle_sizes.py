"""Pins of the row-size arithmetic against the numbers the pages print (CPU only).

[SGLang-pools] section 3: 576 values per MLA row, 1,152 bytes per layer per
token in 16-bit, 69,120 bytes (67.5 KB) per token for DeepSeek-V2 (60 layers).
[SGLang-pools] section 4: 132 bytes per indexer row; DeepSeek-V3 fp8 totals
43,188 bytes per token over 61 layers.  (The page's 78.2 KB for a 16-bit
MLA part mixes decimal and binary kilobytes, so it is not used as a pin.)
[vLLM-V4] appendix, the 8.7x arithmetic, and [V4-digest-2]: 9.62 GiB against
83.9 GiB per 1M-token sequence, about 8.7x, 88.5% smaller.
"""

from oracle import sizes


def test_sglang_rows():
    assert sizes.row_bytes(576, "bf16") == 1152
    assert sizes.mla_bytes_per_token(60, "bf16") == 69120
    assert abs(sizes.mla_bytes_per_token(60, "bf16") / 1024 - 67.5) < 1e-9
    assert sizes.row_bytes(128, "fp8", 128) == 132
    assert sizes.dsa_bytes_per_token(61, "fp8") == 43188


def test_v4_memory_totals():
    v4 = sizes.per_sequence_gib(sizes.v4_bytes_per_token())
    v32 = sizes.per_sequence_gib(sizes.v32_bytes_per_token())
    assert round(v4, 2) == 9.62
    assert round(v32, 1) == 83.9
    assert round(v32 / v4, 1) == 8.7
    assert round(100 * (1 - v4 / v32), 1) == 88.5
