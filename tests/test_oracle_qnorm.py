"""Pins of the oracle's query normalisation + RoPE and window keys (CPU only).

[vLLM-V4] section 3 part 2, third fusion (query normalisation, KV RoPE, K insert).  The
values are fixed independently of oracle/qnorm.py: unit mean square after the norm (a
rotation keeps it), the closed form of a normalised unit vector turned by the textbook RoPE
angle (math.cos / math.sin at pos * base^(-2i/64)), the gain applied before the rotation,
and the rotation checked by complex multiplication (tests/_rot.py).
"""

import math

import numpy as np

from oracle import formats
from oracle.paged import PagedCache
from oracle.qnorm import q_norm_rope, q_norm_rope_swa
from tests._rot import close, rotate, unit_rms_row


def test_heads_leave_with_unit_mean_square():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((8, 576)) * rng.uniform(0.1, 30.0, size=(8, 1))
    out = q_norm_rope(q, None, 0.0, 1048575, 10000.0, 64)
    assert close(np.mean(out * out, axis=1), np.ones(8), 1e-12)


def test_pm1_row_passes_the_norm_unchanged_then_rotates():
    """A +-1 row has mean square 1: with eps = 0 the norm is the identity, leaving the rotation
    (checked by complex multiplication, written apart from the oracle)."""
    rng = np.random.default_rng(1)
    q = np.stack([unit_rms_row(rng, 576) for _ in range(3)])
    for pos in (0, 5, 262143):
        assert close(q_norm_rope(q, None, 0.0, pos, 10000.0, 64), rotate(q, pos), 1e-9)


def test_unit_vector_closed_form():
    """q = e_(512 + 2i): the norm scales it to sqrt(576 / (1 + 576 eps)); RoPE at t turns the
    pair (512 + 2i, 513 + 2i) by t * 10000^(-2i/64)."""
    eps = 1e-6
    for i, t in [(0, 1), (5, 1000), (31, 1048575)]:
        q = np.zeros((1, 576))
        q[0, 512 + 2 * i] = 1.0
        out = q_norm_rope(q, None, eps, t, 10000.0, 64)[0]
        mag = math.sqrt(576.0 / (1.0 + 576.0 * eps))
        ang = t * 10000.0 ** (-2.0 * i / 64)
        want = np.zeros(576)
        want[512 + 2 * i] = mag * math.cos(ang)
        want[513 + 2 * i] = mag * math.sin(ang)
        assert close(out, want, 1e-9)


def test_gain_is_applied_before_the_rotation():
    """gamma weights the pair (512, 513) as (2, 1): the rotated pair is 2a, a turned by the
    angle, not a, a turned and then weighted."""
    q = np.zeros((1, 576))
    q[0, 512] = q[0, 513] = 1.0
    gamma = np.ones(576)
    gamma[512] = 2.0
    t = 3
    out = q_norm_rope(q, gamma, 0.0, t, 10000.0, 64)[0]
    s = math.sqrt(576.0 / 2.0)            # 1 / rms of the input row
    a, b = 2.0 * s, 1.0 * s
    c, sn = math.cos(t), math.sin(t)      # theta_0 = 1
    assert close(out[512:514], np.array([a * c - b * sn, a * sn + b * c]), 1e-12)


def test_zero_query_stays_zero():
    out = q_norm_rope(np.zeros((2, 576)), None, 1e-6, 77, 10000.0, 64)
    assert np.all(out == 0.0)


def test_window_keys_land_at_their_positions():
    """Sequence 0 held 5 tokens and gets 2 rows, sequence 1 held 0 and gets 1: window rows
    at (0, 5), (0, 6), (1, 0), each the raw row turned by its own position."""
    rng = np.random.default_rng(4)
    raw = rng.standard_normal((3, 576)).astype(np.float32)
    swa = PagedCache.empty(2, 256, 256, 576, "f32")
    _, rows = q_norm_rope_swa(np.zeros(0, np.int32), np.zeros((0, 4, 576), np.float32), "f32",
                              None, 1e-6, 10000.0, 64, ctx_lens=[5, 0], cu_new=[0, 2, 3],
                              new_raw=raw, raw_dtype="f32", swa=swa)
    assert sorted(rows) == [(0, 5), (0, 6), (1, 0)]
    for (b, p), r in [((0, 5), 0), ((0, 6), 1), ((1, 0), 2)]:
        want = rotate(raw[r].astype(np.float64), p)
        assert close(rows[(b, p)], want, 1e-9)
        assert close(swa.read(b, p), want, 1e-6)


def test_bf16_query_is_decoded_exactly():
    """Stored bf16 bits decode exactly; a +-1 query row survives the norm unchanged."""
    rng = np.random.default_rng(5)
    qf = np.stack([unit_rms_row(rng, 576)])[None]          # [1, 1, 576]
    bits = formats.f64_to_bf16_bits(qf)
    out, _ = q_norm_rope_swa(np.array([0]), bits, "bf16", None, 0.0, 10000.0, 64)
    assert np.array_equal(out, qf.astype(np.float64))
