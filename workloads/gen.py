"""Seeded random draws (CPU torch generators, one per named tensor).

Each named tensor gets its own ``torch.Generator('cpu')`` seeded with
``seed * 1000 + id(name)``, where id is a stable 3-digit hash of the name, so a
tensor's values do not depend on which other tensors were drawn before it.

Value recipes:
* activations, queries, raw rows and stored bf16/f32 rows: N(0, 1) in float32,
  cast to bfloat16 by torch's round-to-nearest-even where the row is bf16;
* head weights: U(0, 1); compression logits: N(0, 1);
* fp8 rows: E4M3 codes of N(0, 1) * 100 draws (clamped to the format's +-448
  range before torch's cast) and per-row float32 scales U(0.5, 1.5) / 100, so
  code * scale is roughly N(0, 1) with a per-row spread;
* fp4 rows (indexer keys): uniformly random E2M1 codes, two per byte, and one E8M0 scale byte
  per 16 values drawn uniformly from 124..128 (2**-3 .. 2**1), drawn as codes directly;
* block tables: a random permutation of the physical block ids in use.
"""

from __future__ import annotations

import zlib

import torch

_FP8_SPAN = 100.0


def _name_id(name: str) -> int:
    return zlib.crc32(name.encode()) % 997 + 1


class Gen:
    def __init__(self, seed: int = 0):
        self.seed = int(seed)

    def gen(self, name: str) -> torch.Generator:
        return torch.Generator().manual_seed(self.seed * 1000 + _name_id(name))

    def normal(self, name: str, shape, dtype=torch.float32) -> torch.Tensor:
        x = torch.randn(*shape, generator=self.gen(name), dtype=torch.float32)
        return x.to(dtype)

    def uniform(self, name: str, shape, lo: float = 0.0, hi: float = 1.0) -> torch.Tensor:
        x = torch.rand(*shape, generator=self.gen(name), dtype=torch.float32)
        return x * (hi - lo) + lo

    def fp8_codes(self, name: str, shape) -> torch.Tensor:
        x = torch.randn(*shape, generator=self.gen(name), dtype=torch.float32) * _FP8_SPAN
        return x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)

    def fp8_scales(self, name: str, shape) -> torch.Tensor:
        return self.uniform(name, shape, 0.5, 1.5) / _FP8_SPAN

    def fp4_bytes(self, name: str, shape) -> torch.Tensor:
        """Packed E2M1 codes: shape[-1] logical values -> shape[-1] / 2 bytes."""
        nib = torch.randint(0, 16, (*shape[:-1], shape[-1]), generator=self.gen(name), dtype=torch.int32)
        return (nib[..., 0::2] | (nib[..., 1::2] << 4)).to(torch.uint8)

    def fp4_scales(self, name: str, shape) -> torch.Tensor:
        """E8M0 bytes, one per 16 values: shape[-1] logical values -> shape[-1] / 16 bytes."""
        return torch.randint(124, 129, (*shape[:-1], shape[-1] // 16), generator=self.gen(name),
                             dtype=torch.int32).to(torch.uint8)

    def permutation(self, name: str, n: int) -> torch.Tensor:
        return torch.randperm(n, generator=self.gen(name)).to(torch.int32)

    def distinct_ints(self, name: str, count: int, upper: int) -> torch.Tensor:
        """`count` distinct integers drawn from [0, upper), in random order."""
        return torch.randperm(upper, generator=self.gen(name))[:count].to(torch.int32)

    def rows(self, name: str, shape, dtype: str):
        """Stored rows of a cache dtype: returns (rows, scales or None)."""
        if dtype == "fp8":
            return self.fp8_codes(name, shape), self.fp8_scales(name + ".scale", shape[:-1])
        if dtype == "fp4":
            return self.fp4_bytes(name, shape), self.fp4_scales(name + ".scale", shape)
        return self.normal(name, shape, torch.bfloat16 if dtype == "bf16" else torch.float32), None


def paged_rows(g: Gen, name: str, batch: int, rows_per_block: int, dim: int, dtype: str,
               logical_rows: int, live: list[tuple[int, int]]):
    """A paged cache whose logical rows [lo_b, hi_b) of each sequence b are backed by memory.

    Physical block 0 is a zero dummy that every unbacked logical block points at; the backed
    blocks get ids 1.. in a random order.  Returns (rows, scales or None, block_table), CPU.
    """
    bt_stride = max(1, -(-logical_rows // rows_per_block))
    bt = torch.zeros((batch, bt_stride), dtype=torch.int32)
    need = []
    for b, (lo, hi) in enumerate(live):
        if hi > lo:
            for blk in range(lo // rows_per_block, -(-hi // rows_per_block)):
                need.append((b, blk))
    perm = g.permutation(name + ".bt", len(need)) + 1
    for (b, blk), pid in zip(need, perm.tolist()):
        bt[b, blk] = pid
    nb = len(need) + 1
    rows, scales = g.rows(name, (nb, rows_per_block, dim), dtype)
    rows[0].zero_()
    if scales is not None:
        scales[0].fill_(127 if dtype == "fp4" else 1.0)
    return rows, scales, bt
