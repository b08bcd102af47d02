"""Pins of the fp4 row acceptance check used by the GPU parity tests (CPU only).

tests/oracle_step.check_fp4_row decides whether a stored fp4 row (packed E2M1 codes plus E8M0
block scales) is a correct rounding of an exact row.  It must accept the oracle's own
quantisation of random rows, a code rounded the other way at an exact tie, and a scale one
step off only where amax lies within float32 accuracy of the boundary; it must reject a code
moved by one step, a scale one step too large or too small, and swapped nibbles.
"""

import numpy as np

from oracle import formats
from tests.oracle_step import check_fp4_row


def _rows(seed, n=20, d=128):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)) * rng.uniform(0.01, 50.0, size=(n, 1))


def test_accepts_the_oracle_quantisation():
    for row in _rows(0):
        packed, sb = formats.fp4_quantize_row(row)
        ok, r = check_fp4_row(packed, sb, row)
        assert ok, r


def test_accepts_either_rounding_within_float32_accuracy_of_a_tie():
    """Value 1.25 * 2^k (a tie between codes 1.0 and 1.5, nearest even: 1.0) stored as 1.5: the
    kernel's float32 value may sit just above the tie."""
    row = np.zeros(16)
    row[0], row[1] = 6.0, 1.25 * (1 + 1e-7)
    packed, sb = formats.fp4_quantize_row(row)
    assert formats.fp4_unpack(packed, sb)[1] == 1.5
    row[1] = 1.25
    assert formats.fp4_unpack(*formats.fp4_quantize_row(row))[1] == 1.0
    ok, _ = check_fp4_row(packed, sb, row)
    assert ok


def _nibble(packed, i):
    return (packed[i // 2] >> (4 * (i % 2))) & 0xF


def _set_nibble(packed, i, v):
    p = packed.copy()
    sh = 4 * (i % 2)
    keep = 0xF0 if sh == 0 else 0x0F
    p[i // 2] = (int(p[i // 2]) & keep) | (int(v) << sh)
    return p


def test_rejects_a_code_one_step_off():
    row = _rows(1, n=1)[0]
    packed, sb = formats.fp4_quantize_row(row)
    i = int(np.argmax(np.abs(row[:16])))          # the block maximum: code 6 or 7 (4 or 6)
    c = _nibble(packed, i)
    step = c - 1 if (c & 7) > 1 else c + 1
    ok, _ = check_fp4_row(_set_nibble(packed, i, step), sb, row)
    assert not ok


def test_rejects_a_scale_one_step_off():
    row = _rows(2, n=1)[0]
    packed, sb = formats.fp4_quantize_row(row)
    for delta in (1, -1):
        s2 = sb.copy()
        s2[3] = int(s2[3]) + delta
        ok, _ = check_fp4_row(packed, s2, row)
        assert not ok


def test_accepts_a_scale_step_only_at_the_boundary():
    """amax = 6 * 2^k exactly: k is correct; k + 1 is also accepted when amax sits within float32
    accuracy above the boundary (the oracle's own choice there is k + 1)."""
    row = np.zeros(16)
    row[0] = 6.0 * (1 + 1e-7)
    packed, sb = formats.fp4_quantize_row(row)
    assert int(sb[0]) == 128                           # k = 1: amax > 6
    exact = row.copy()
    exact[0] = 6.0
    assert check_fp4_row(packed, sb, exact)[0]         # within delta of the boundary
    p0, s0 = formats.fp4_quantize_row(exact)
    assert int(s0[0]) == 127 and check_fp4_row(p0, s0, exact)[0]
    far = row.copy()
    far[0] = 5.0                                       # amax 5: k = 0 only
    assert not check_fp4_row(packed, sb, far)[0]


def test_rejects_swapped_nibbles():
    row = np.zeros(16)
    row[0], row[1] = 6.0, -0.5
    packed, sb = formats.fp4_quantize_row(row)
    swapped = ((packed >> 4) | ((packed & 0xF) << 4)).astype(np.uint8)
    assert check_fp4_row(packed, sb, row)[0]
    assert not check_fp4_row(swapped, sb, row)[0]


def test_zero_block_needs_scale_one():
    row = np.zeros(32)
    row[16] = 3.0
    packed, sb = formats.fp4_quantize_row(row)
    assert int(sb[0]) == 127
    assert check_fp4_row(packed, sb, row)[0]
    s2 = sb.copy()
    s2[0] = 126
    assert not check_fp4_row(packed, s2, row)[0]
