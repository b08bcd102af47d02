"""Entry geometry of the c4a / c128a compressors (oracle; test infrastructure only).

[vLLM-V4] appendix, "exact position ranges and causality":
* c4a entry i (i from 0) is a weighted sum of the raw tokens at positions
  [4i - 4, 4i + 3] (negative positions count as value 0) and takes RoPE at
  its anchor position 4i + 3;
* c128a entry i covers [128i, 128i + 127] and takes RoPE at 128i + 127;
* a query at position m may use entry i only if 4i + 3 <= m (c4a) or
  128i + 127 <= m (c128a).
[vLLM-V4] section 2: c4a compresses 8 tokens with stride 4, c128a 128 tokens
with stride 128.  [vLLM-V4] section 3 part 1: a logical block is 256 native
positions, so a c4a block holds 64 entries and a c128a block 2.

Reading: after L raw tokens (positions 0 .. L-1) the entries whose anchors
are present are i = 0 .. floor(L / R) - 1, so n(L) = floor(L / R).
"""

from __future__ import annotations

BLOCK_POSITIONS = 256


def coff(ratio: int) -> int:
    """Overlap factor: 2 for c4a (8-token window, stride 4), 1 for c128a."""
    if ratio == 4:
        return 2
    if ratio == 128:
        return 1
    raise ValueError(f"ratio must be 4 or 128, got {ratio}")


def window_len(ratio: int) -> int:
    """Raw tokens per entry: coff * ratio (8 for c4a, 128 for c128a)."""
    return coff(ratio) * ratio


def entry_start(j: int, ratio: int) -> int:
    """First raw position of entry j: 4j - 4 (c4a) or 128j (c128a)."""
    return ratio * j - (coff(ratio) - 1) * ratio


def entry_anchor(j: int, ratio: int) -> int:
    """RoPE position (last raw position) of entry j: 4j + 3 or 128j + 127."""
    return ratio * j + ratio - 1


def num_entries(num_tokens: int, ratio: int) -> int:
    """Entries whose anchor lies in [0, num_tokens): floor(num_tokens / ratio)."""
    return num_tokens // ratio


def visible_entries(t: int, ratio: int) -> int:
    """Entries a query at position t may use (anchor <= t): n(t + 1)."""
    return num_entries(t + 1, ratio)


def entries_per_block(ratio: int) -> int:
    """Compressed entries in one 256-position logical block: 64 (c4a) or 2 (c128a)."""
    return BLOCK_POSITIONS // ratio
