"""Test-local rotation by complex multiplication, independent of the oracle's code.

Pair i of the rotated span (the last rope_dims dimensions, consecutive pairs)
is the complex number x[2i] + 1j * x[2i+1]; RoPE at position m multiplies it
by exp(1j * m * theta_i), theta_i = base ** (-2 i / rope_dims).
"""

import cmath
import math

import numpy as np


def rotate(x, pos, base=10000.0, rope_dims=64):
    x = np.array(x, dtype=np.float64)
    d = x.shape[-1]
    out = x.copy()
    flat = out.reshape(-1, d)
    for r in range(flat.shape[0]):
        for i in range(rope_dims // 2):
            a = d - rope_dims + 2 * i
            theta = base ** (-2.0 * i / rope_dims)
            z = complex(flat[r, a], flat[r, a + 1]) * cmath.exp(1j * (pos * theta))
            flat[r, a], flat[r, a + 1] = z.real, z.imag
    return out


def unit_rms_row(rng, d):
    """A row of +-1 values: mean square exactly 1, so RMSNorm with eps = 0 is the identity."""
    return rng.choice([-1.0, 1.0], size=d)


def close(a, b, tol=1e-12):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) <= tol * max(1.0, float(np.max(np.abs(b))))


__all__ = ["rotate", "unit_rms_row", "close", "math"]
