"""Pins of the acceptance checks that the GPU parity tests rest on (CPU only).

Every GPU verdict goes through one of three functions of tests/oracle_step.py:
* check_rounded_row -- a stored bf16 / fp8 / float32 row against the oracle's exact row;
* topk_acceptable   -- a GPU top-k id list against the oracle's scores (reading R11);
* allclose_out      -- attention outputs and log-sum-exps against the oracle's.
Each must accept what a correct kernel may produce and reject the plausible mistakes: a code
rounded to the wrong neighbour, a scale off by more than float32 accuracy, a missing winner,
an extra loser, a duplicate or non-causal id, bad padding, an error just over the tolerance,
a NaN or a one-sided infinity.  If any of them were changed to accept everything, these
tests fail.
"""

import numpy as np
import pytest

from oracle import formats, indexer
from tests.oracle_step import allclose_out, check_rounded_row, half_ulp_bf16, topk_acceptable


def _rows(seed, n=16, d=576):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)) * rng.uniform(0.05, 20.0, size=(n, 1))


def _bf16(x):
    return formats.bf16_bits_to_f64(formats.f64_to_bf16_bits(np.asarray(x, dtype=np.float64)))


def _next_bf16(v, direction):
    """The bf16 neighbour of the bf16 value v (float64) in the given direction (+1 / -1)."""
    bits = formats.f64_to_bf16_bits(np.array([v]))[0].astype(np.int64)
    step = direction if v >= 0 else -direction
    return float(formats.bf16_bits_to_f64(np.array([bits + step], dtype=np.uint16))[0])


# ---------------------------------------------------------------- check_rounded_row, bf16

def test_bf16_accepts_the_oracle_rounding():
    for row in _rows(0):
        ok, r = check_rounded_row(_bf16(row), row, "bf16")
        assert ok, r


def test_bf16_accepts_either_rounding_at_a_midpoint_within_float32_accuracy():
    """1 + 2^-8 lies halfway between the bf16 values 1 and 1 + 2^-7 (nearest even: 1); a float32
    result a hair above the tie rounds up.  Both stored values pass."""
    row = np.full(8, 0.5)
    row[0] = 1.0 + 2.0 ** -8
    lo = row.copy()
    lo[0] = 1.0
    hi = row.copy()
    hi[0] = 1.0 + 2.0 ** -7
    assert check_rounded_row(lo, row, "bf16")[0]
    assert check_rounded_row(hi, row, "bf16")[0]


@pytest.mark.parametrize("frac", [1.0, 0.3, 0.05, 1e-2])
def test_bf16_rejects_the_wrong_neighbour(frac):
    """An element exactly representable in bf16, stored as its neighbour (one ulp away), at
    magnitudes from the row maximum down to 1e-2 of it."""
    row = _bf16(_rows(1, n=1)[0])
    i = int(np.argmax(np.abs(row)))
    j = (i + 1) % row.size
    row[j] = _bf16(frac * row[i])
    for direction in (+1, -1):
        bad = row.copy()
        bad[j] = _next_bf16(row[j], direction)
        ok, r = check_rounded_row(bad, row, "bf16")
        assert not ok, (frac, direction, r)


def test_bf16_absolute_allowance_is_float32_accuracy_of_the_row():
    """The allowance beyond half an ulp is 1e-5 |x| + 1e-6 max|row|: an element that cancels to
    nearly zero keeps the absolute float32 error of the row's magnitude.  An error of 0.9e-6 max
    on a 1e-4 max element passes; 1.2e-6 max (beyond half an ulp plus the allowance) fails."""
    row = np.zeros(64)
    row[0] = 1.0
    row[1] = 1e-4
    half = float(half_ulp_bf16(np.array([1e-4]))[0])
    exact = row.copy()
    exact[1] = _bf16(1e-4)
    ok_vals = exact.copy()
    ok_vals[1] = exact[1]
    assert check_rounded_row(ok_vals, exact, "bf16")[0]
    shifted = exact.copy()
    shifted[1] = exact[1] + half + 0.9e-6 - 1e-5 * exact[1]
    assert check_rounded_row(shifted, exact, "bf16")[0]
    shifted[1] = exact[1] + half + 1.2e-6
    assert not check_rounded_row(shifted, exact, "bf16")[0]


def test_f32_rows_allow_float32_accuracy_only():
    row = _rows(2, n=1)[0]
    m = float(np.max(np.abs(row)))
    assert check_rounded_row(row.astype(np.float32).astype(np.float64), row, "f32")[0]
    bad = row.copy()
    bad[3] += 3e-6 * m + 1e-5 * abs(row[3])
    assert not check_rounded_row(bad, row, "f32")[0]


# ---------------------------------------------------------------- check_rounded_row, fp8

def _fp8(row):
    codes, scale = formats.fp8_quantize_row(row)
    return formats.decode_stored(codes[None], "fp8", np.array([scale]))[0], scale


def test_fp8_accepts_the_oracle_quantisation():
    for row in _rows(3):
        vals, sc = _fp8(row)
        ok, r = check_rounded_row(vals, row, "fp8", sc, sc)
        assert ok, r


@pytest.mark.parametrize("code_mag", [400.0, 100.0, 12.0, 1.5])
def test_fp8_rejects_the_wrong_neighbour(code_mag):
    """An element whose exact value is an E4M3 value (in code units of the row scale) stored as
    the next code up or down."""
    rng = np.random.default_rng(4)
    row = rng.standard_normal(576)
    row[0] = 10.0                    # the row maximum: scale = 10 / 448
    vals, sc = _fp8(row)
    sc64 = float(sc)
    exact = vals.copy()              # a row whose exact values are exactly representable
    code = float(formats.round_to_fp8_e4m3(np.array([code_mag]))[0])
    exact[5] = code * sc64
    exact_codes = formats.f64_to_fp8_e4m3(exact / sc64)
    assert check_rounded_row(exact, exact, "fp8", sc, sc)[0]
    for step in (+1, -1):
        c = exact_codes.astype(np.int64)
        c[5] = c[5] + step               # (positive codes: the next magnitude up or down)
        c = c.astype(np.uint8)
        bad = formats.decode_stored(c[None], "fp8", np.array([sc]))[0]
        ok, r = check_rounded_row(bad, exact, "fp8", sc, sc)
        assert not ok, (code_mag, step, r)


def test_fp8_rejects_a_scale_off_by_2e6():
    row = _rows(5, n=1)[0]
    vals, sc = _fp8(row)
    off = np.float32(float(sc) * (1 + 2e-6))
    assert off != sc
    ok, _ = check_rounded_row(vals * (float(off) / float(sc)), row, "fp8", off, sc)
    assert not ok


# ---------------------------------------------------------------- topk_acceptable

def _scores(seed, n=400):
    return np.random.default_rng(seed).uniform(0.0, 100.0, n)


def _ref(s, k):
    ids = indexer.topk(s, k)
    sel = np.sort(ids[ids >= 0])
    return np.concatenate([sel, np.full(k - sel.size, -1)])


def test_topk_accepts_the_oracle_selection():
    s = _scores(0)
    for k in (1, 16, 64, 399, 400, 512):
        ok, why = topk_acceptable(_ref(s, k), s, k)
        assert ok, (k, why)


def test_topk_rejects_a_missing_clear_winner():
    s = _scores(1)
    k = 32
    ids = _ref(s, k)
    best = int(np.argmax(s))
    runner = int(indexer.topk(s, k + 1)[k])          # the (k+1)-th: a clear loser by > 1e-5
    bad = np.sort(np.concatenate([ids[ids != best], [runner]]))
    ok, why = topk_acceptable(bad, s, k)
    assert not ok and why == "missing a clear winner"


def test_topk_rejects_a_clear_loser():
    s = _scores(2)
    k = 32
    ids = _ref(s, k)
    kth = int(indexer.topk(s, k)[k - 1])
    worst = int(np.argmin(s))
    bad = np.sort(np.concatenate([ids[ids != kth], [worst]]))
    ok, why = topk_acceptable(bad, s, k)
    assert not ok


def test_topk_rejects_duplicates_order_and_non_causal_ids():
    s = _scores(3)
    k = 8
    ids = _ref(s, k)
    dup = ids.copy()
    dup[1] = dup[0]
    assert not topk_acceptable(dup, s, k)[0]
    rev = ids[::-1].copy()
    assert not topk_acceptable(rev, s, k)[0]
    # an id past the visible entries (a future entry) in place of the last winner
    future = ids.copy()
    future[-1] = len(s)
    assert not topk_acceptable(future, s, k)[0]


def test_topk_rejects_bad_padding():
    s = _scores(4, n=10)
    k = 16                                          # k' = 10, six -1 slots
    ids = _ref(s, k)
    assert topk_acceptable(ids, s, k)[0]
    short = ids.copy()
    short[9] = -1                                   # only 9 ids
    assert not topk_acceptable(short, s, k)[0]
    junk = ids.copy()
    junk[12] = 3                                    # an id after the padding starts
    assert not topk_acceptable(junk, s, k)[0]
    hole = ids.copy()
    hole[[2, 10]] = hole[[10, 2]]                   # a -1 inside the id block
    assert not topk_acceptable(hole, s, k)[0]


def test_topk_accepts_either_side_of_an_exact_tie_and_a_near_tie():
    s = np.arange(100, dtype=np.float64)
    s[50] = s[60] = 200.0                           # tie at the k-th place for k = 1 + ...
    s[70] = 300.0
    k = 2                                           # {70} plus one of {50, 60}
    assert topk_acceptable(np.array([50, 70]), s, k)[0]
    assert topk_acceptable(np.array([60, 70]), s, k)[0]
    s2 = s.copy()
    s2[60] = 200.0 * (1 + 5e-6)                     # within 1e-5 relative of the k-th score
    assert topk_acceptable(np.array([50, 70]), s2, k)[0]
    s2[60] = 200.0 * (1 + 5e-5)                     # a clear winner now
    assert not topk_acceptable(np.array([50, 70]), s2, k)[0]


def test_topk_zero_filler_when_fewer_positive_scores_than_k():
    s = np.zeros(50)
    s[[3, 7]] = [5.0, 6.0]
    k = 4                                           # tau = 0: any two zero-score ids fill in
    assert topk_acceptable(np.array([3, 7, 20, 40]), s, k)[0]
    assert topk_acceptable(np.array([0, 1, 3, 7]), s, k)[0]
    assert not topk_acceptable(np.array([0, 1, 2, 3]), s, k)[0]   # misses 7


# ---------------------------------------------------------------- allclose_out

def test_allclose_accepts_within_and_rejects_just_beyond_2e3():
    ref = np.random.default_rng(6).standard_normal(1000) * 10.0
    ref[np.abs(ref) < 1.0] = 1.0                    # atol negligible against 2e-3 |ref|
    assert allclose_out(ref * (1 + 1.9e-3), ref)[0]
    assert allclose_out(ref * (1 - 1.9e-3), ref)[0]
    bad = ref.copy()
    bad[17] *= 1 + 2.1e-3
    assert not allclose_out(bad, ref)[0]
    bad = ref.copy()
    bad[17] *= 1 - 2.1e-3
    assert not allclose_out(bad, ref)[0]


def test_allclose_absolute_floor():
    ref = np.zeros(10)
    assert allclose_out(np.full(10, 0.9e-5), ref)[0]
    assert not allclose_out(np.full(10, 1.1e-5), ref)[0]


def test_allclose_rejects_nan_and_one_sided_inf():
    ref = np.linspace(-3, 3, 20)
    g = ref.copy()
    g[4] = np.nan
    assert not allclose_out(g, ref)[0]
    both = ref.copy()
    both[4] = np.nan
    assert not allclose_out(both, both)[0]          # a NaN is never a match
    g = ref.copy()
    g[5] = np.inf
    assert not allclose_out(g, ref)[0]
    r2 = ref.copy()
    r2[5] = -np.inf
    assert not allclose_out(ref, r2)[0]


def test_allclose_equal_infinities_pass():
    """The lse of a query with no visible row is -inf on both sides."""
    ref = np.array([-np.inf, 1.0, 2.0])
    assert allclose_out(ref.copy(), ref)[0]
