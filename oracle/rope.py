"""Rotary position embedding and its inverse (oracle; test infrastructure only).

[vLLM-V4] appendix, "why inverse RoPE is needed when K = V": a rotation
R_m parameterised by position m, with R_m^T R_m = I and R_m R_n = R_{m+n};
keys and values are the same rotated rows, so the attention output is
multiplied by R_m^{-1} at the query position m, leaving only R_{n-m}.
The rotation is the block-diagonal form of the RoPE paper the appendix cites
(arXiv 2104.09864): each 2-D pair is turned by the angle m * theta_i with
theta_i = base ** (-2 i / rope_dims).

Readings (parity unpinned: nothing on the pages fixes them):
* the rotated dimensions are the LAST ``rope_dims`` of a row: the shared KV
  row is the 512 latent dimensions followed by the 64 RoPE dimensions
  ([SGLang-pools] section 3: kv_cache_dim = kv_lora_rank + qk_rope_head_dim);
* pairs are consecutive, (2i, 2i+1) within that span.
Angles are formed in float64 (at m near 2**20 a float32 product m * theta
would be off by up to about 0.05 rad).
"""

from __future__ import annotations

import numpy as np


def rope_theta(base: float, rope_dims: int) -> np.ndarray:
    """theta_i = base ** (-2 i / rope_dims), i = 0 .. rope_dims/2 - 1, in float64."""
    i = np.arange(rope_dims // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / rope_dims)


def rope(x: np.ndarray, pos, base: float = 10000.0, rope_dims: int = 64) -> np.ndarray:
    """Rotate the last ``rope_dims`` dimensions of each row of x by R_pos.

    x: [..., d] float64; pos: scalar or array broadcastable to x.shape[:-1]
    (negative positions give the inverse rotation).  For the pair
    (a, b) = (x[2i], x[2i+1]) of the rotated span:
        a' = a cos(pos theta_i) - b sin(pos theta_i)
        b' = a sin(pos theta_i) + b cos(pos theta_i)
    which is the complex product (a + i b) * exp(i pos theta_i).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert rope_dims % 2 == 0 and 0 < rope_dims <= d
    out = x.copy()
    theta = rope_theta(base, rope_dims)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta          # [..., rope_dims/2]
    c, s = np.cos(ang), np.sin(ang)
    span = x[..., d - rope_dims:]
    a, b = span[..., 0::2], span[..., 1::2]
    out[..., d - rope_dims + 0::2] = a * c - b * s
    out[..., d - rope_dims + 1::2] = a * s + b * c
    return out


def inverse_rope(x: np.ndarray, pos, base: float = 10000.0, rope_dims: int = 64) -> np.ndarray:
    """R_pos^{-1} x = R_{-pos} x ([vLLM-V4] appendix: Output = Attention(Q, K, V) R_m^{-1})."""
    return rope(x, -np.asarray(pos, dtype=np.float64), base, rope_dims)
