"""Workload shapes: the five configurations of the benchmark plus reduced variants for tests.

A step appends ``new_tokens`` raw tokens to each sequence (ending at ctx_after[b]) and runs
queries at the last ``q_per_seq`` new positions of each sequence.  Either may be one count for
every sequence or a tuple with one count per sequence (ragged batches).  ``stages`` lists what the
timed step runs: "compress" (main KV, plus window rows), "compress_idx" (indexer keys),
"index" (scores and top-k) and "attn" (sparse attention and inverse RoPE).
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class StepConfig:
    name: str
    ratio: int                       # 4 (c4a) or 128 (c128a)
    ctx_after: tuple[int, ...]       # raw tokens per sequence after the step
    new_tokens: int | tuple[int, ...]  # raw tokens appended per sequence by the step
    q_per_seq: int | tuple[int, ...]   # queries per sequence (at its last new positions)
    n_heads: int
    kv_dtype: str                    # "f32" | "bf16" | "fp8" (main and window caches)
    q_dtype: str                     # "f32" | "bf16"
    raw_dtype: str                   # "f32" | "bf16"
    stages: tuple[str, ...]
    idx_heads: int = 64
    idx_dtype: str = "fp8"           # indexer key cache ("fp8", "fp4", "bf16" or "f32")
    idx_q_dtype: str = "bf16"
    k: int = 512
    window: int = 128
    dim: int = 576
    softmax_scale: float = 1.0 / 24.0
    rope_base: float = 10000.0
    eps: float = 1e-6
    gamma: bool = False              # draw a random RMSNorm gain instead of 1
    seed: int = 0

    @property
    def batch(self) -> int:
        return len(self.ctx_after)

    def new_of(self, b: int) -> int:
        return self.new_tokens[b] if isinstance(self.new_tokens, tuple) else self.new_tokens

    def q_of(self, b: int) -> int:
        return self.q_per_seq[b] if isinstance(self.q_per_seq, tuple) else self.q_per_seq

    @property
    def max_context(self) -> int:
        return max(self.ctx_after)

    @property
    def has_indexer(self) -> bool:
        return "index" in self.stages


# --- the five configurations -----------------------------------------------------------------

REF = StepConfig(
    name="ref_c4a_1k_fp32", ratio=4, ctx_after=(1024,), new_tokens=1024, q_per_seq=1, n_heads=8,
    kv_dtype="f32", q_dtype="f32", raw_dtype="f32", stages=("compress", "index", "attn"),
    idx_heads=4, idx_dtype="f32", idx_q_dtype="f32", k=64)

C4A_128K_B32 = StepConfig(
    name="c4a_decode_128k_b32_bf16", ratio=4, ctx_after=(131072,) * 32, new_tokens=1, q_per_seq=1,
    n_heads=64, kv_dtype="bf16", q_dtype="bf16", raw_dtype="bf16", stages=("index", "attn"), k=512)

C128A_1M_B8 = StepConfig(
    name="c128a_decode_1m_b8_bf16", ratio=128, ctx_after=(1 << 20,) * 8, new_tokens=1, q_per_seq=1,
    n_heads=64, kv_dtype="bf16", q_dtype="bf16", raw_dtype="bf16", stages=("compress", "attn"))

C4A_1M_B4_FP8 = StepConfig(
    name="c4a_decode_1m_b4_fp8", ratio=4, ctx_after=tuple((1 << 20) - b for b in range(4)),
    new_tokens=1, q_per_seq=1, n_heads=128, kv_dtype="fp8", q_dtype="bf16", raw_dtype="bf16",
    stages=("compress", "compress_idx", "index", "attn"), k=2048)

C4A_PREFILL_64K = StepConfig(
    name="c4a_prefill_4k_on_64k_bf16", ratio=4, ctx_after=(65536 + 4096,), new_tokens=4096,
    q_per_seq=4096, n_heads=64, kv_dtype="bf16", q_dtype="bf16", raw_dtype="bf16",
    stages=("compress", "compress_idx", "index", "attn"), k=512)

CONFIGS = [REF, C4A_128K_B32, C128A_1M_B8, C4A_1M_B4_FP8, C4A_PREFILL_64K]

# The 1M fp8 decode with the indexer cache in FP4 (two E2M1 codes a byte, one power-of-two
# scale per 16 values): 72-byte keys instead of 132.
C4A_1M_B4_FP4IDX = replace(C4A_1M_B4_FP8, name="c4a_decode_1m_b4_fp8_fp4idx", idx_dtype="fp4")
HEADLINE = C4A_1M_B4_FP8


def scaled(cfg: StepConfig, ctx_after, name_suffix: str = "small", **kw) -> StepConfig:
    """The same workload at other lengths (and optionally other fields) for quick parity runs."""
    return replace(cfg, name=f"{cfg.name}_{name_suffix}", ctx_after=tuple(ctx_after), **kw)
