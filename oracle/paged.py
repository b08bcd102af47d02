"""Paged caches with 256-position logical blocks (oracle; test infrastructure only).

[vLLM-V4] section 3 part 1: every compressed layer uses one logical block of
256 native positions; a c4a block physically holds 64 entries, a c128a block
2, an uncompressed (sliding-window) block 256 rows.  Each sequence owns a
block table from logical block to physical block.

Reading: logical row r of sequence b (an entry index for compressed caches,
a raw position for window and compressor-state caches) lives in physical
block ``block_table[b, r // rows_per_block]`` at slot ``r % rows_per_block``.
The compressor state is itself a paged cache of raw rows addressed by
position ([vLLM-V4] section 3 part 1, "compressor state as a sliding
window": registered as sliding-window KV with window coff * ratio).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats


@dataclass
class PagedCache:
    rows: np.ndarray                 # [num_blocks, rows_per_block, dim]: float32 | uint16 (bf16) |
                                     # uint8 (fp8 codes); fp4: [..., dim / 2] uint8, two codes a byte
    dtype: str                       # "f32" | "bf16" | "fp8" | "fp4"
    block_table: np.ndarray          # int32 [batch, bt_stride]
    scales: np.ndarray | None = None  # fp8: float32 [num_blocks, rows_per_block];
                                      # fp4: uint8 E8M0 [num_blocks, rows_per_block, dim / 16]

    @property
    def rows_per_block(self) -> int:
        return self.rows.shape[1]

    @property
    def dim(self) -> int:
        return self.rows.shape[2] * (2 if self.dtype == "fp4" else 1)

    def locate(self, b: int, r):
        r = np.asarray(r, dtype=np.int64)
        blk = self.block_table[b][r // self.rows_per_block].astype(np.int64)
        return blk, r % self.rows_per_block

    def read(self, b: int, r) -> np.ndarray:
        """Exact float64 values of logical rows r (scalar or array) of sequence b."""
        blk, slot = self.locate(b, r)
        vals = self.rows[blk, slot]
        sc = None if self.scales is None else self.scales[blk, slot]
        return formats.decode_stored(vals, self.dtype, sc)

    def write(self, b: int, r: int, value: np.ndarray) -> None:
        """Store one float64 row at logical row r of sequence b, rounded to the cache dtype."""
        blk, slot = self.locate(b, r)
        stored, scale = formats.encode_row(value, self.dtype)
        self.rows[blk, slot] = stored
        if self.dtype in ("fp8", "fp4"):
            self.scales[blk, slot] = scale

    @staticmethod
    def empty(batch: int, logical_rows: int, rows_per_block: int, dim: int, dtype: str,
              perm_seed: int | None = None) -> "PagedCache":
        """A zeroed cache with room for ``logical_rows`` rows per sequence.

        Physical blocks are numbered in sequence order, or shuffled with
        ``perm_seed`` to exercise the block table.
        """
        nb = -(-logical_rows // rows_per_block)
        ids = np.arange(batch * nb, dtype=np.int32)
        if perm_seed is not None:
            ids = np.random.default_rng(perm_seed).permutation(ids).astype(np.int32)
        store = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "fp4": np.uint8}[dtype]
        rows = np.zeros((batch * nb, rows_per_block, dim // 2 if dtype == "fp4" else dim), dtype=store)
        scales = None
        if dtype == "fp8":
            scales = np.ones((batch * nb, rows_per_block), dtype=np.float32)
        elif dtype == "fp4":
            scales = np.full((batch * nb, rows_per_block, dim // 16), 127, dtype=np.uint8)
        return PagedCache(rows, dtype, ids.reshape(batch, nb), scales)

    def copy(self) -> "PagedCache":
        return PagedCache(self.rows.copy(), self.dtype, self.block_table.copy(),
                          None if self.scales is None else self.scales.copy())
