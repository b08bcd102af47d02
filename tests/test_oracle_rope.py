"""Pins of the oracle's RoPE (CPU only).

[vLLM-V4] appendix, why inverse RoPE: R_m^T R_m = I and R_m R_n = R_{m+n};
q_m . k_n depends only on n - m; R_m^{-1} R_n = R_{n-m}.  The rotation itself
is checked against complex multiplication written independently in _rot.py.
"""

import numpy as np

from oracle.rope import inverse_rope, rope
from tests._rot import close, rotate


def test_matches_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 96))
    for pos in [0, 1, 7, 1023, 1048575]:
        assert close(rope(x, pos), rotate(x, pos), 1e-9)


def test_only_last_rope_dims_move():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(576)
    y = rope(x, 12345)
    assert np.array_equal(y[:512], x[:512])
    assert not np.allclose(y[512:], x[512:])


def test_orthogonal_and_group_law():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 128))
    for m, n in [(3, 5), (1000, -1000), (1048575, 17), (-7, 2 ** 19)]:
        assert close(np.linalg.norm(rope(x, m), axis=1), np.linalg.norm(x, axis=1))
        assert close(rope(rope(x, m), n), rope(x, m + n), 1e-9)
        assert close(inverse_rope(rope(x, m), m), x, 1e-9)


def test_dot_product_depends_on_offset_only():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(576), rng.standard_normal(576)
    base = rope(q, 100) @ rope(k, 140)
    for shift in [1, 256, 65536, 999999]:
        assert abs(rope(q, 100 + shift) @ rope(k, 140 + shift) - base) < 1e-8
