"""Pins of the oracle's number formats against torch's own casts (CPU only).

bf16: torch's float32 -> bfloat16 cast is round-to-nearest-even, so on
float32-representable inputs it must agree with the oracle's float64 rounding.
fp8: torch.float8_e4m3fn is the OCP E4M3 format; decoding every code and
encoding in-range values must agree bit for bit.  torch's cast turns values
beyond the range into NaN, so saturation is checked against the format's
definition (largest finite value 448) instead.
"""

import numpy as np
import pytest
import torch

from oracle import formats


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = formats.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


@pytest.mark.parametrize("seed", [0, 1])
def test_bf16_rounding_matches_torch(seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.standard_normal(20000),
        rng.standard_normal(2000) * 1e-38,            # subnormal range of bf16
        rng.standard_normal(2000) * 1e30,
        # exact midpoints between neighbouring bf16 values (ties to even)
        (np.arange(1, 2000) * 2 + 1).astype(np.float64) * 2.0 ** -9,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = formats.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_fp8_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.nanmax(ours) == 448.0
    assert ours[1] == 2.0 ** -9          # smallest subnormal


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    vals = formats.fp8_e4m3_to_f64(np.arange(256, dtype=np.uint8))
    vals = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = (vals[1:] + vals[:-1]) / 2          # every tie between neighbours
    x = np.concatenate([vals, mids, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 0.01]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = formats.f64_to_fp8_e4m3(x.astype(np.float64))
    # torch keeps the sign of negative zero; so does the oracle
    assert np.array_equal(ours, ref)


def test_fp8_saturates_by_definition():
    x = np.array([448.0, 449.0, 500.0, 1e6, -1e6])
    codes = formats.f64_to_fp8_e4m3(x)
    assert list(codes) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_fp8_row_quantization():
    rng = np.random.default_rng(3)
    c = rng.standard_normal(576)
    codes, scale = formats.fp8_quantize_row(c)
    assert scale == np.float32(np.max(np.abs(c)) / 448.0)
    back = formats.fp8_e4m3_to_f64(codes) * np.float64(scale)
    # the amax element maps to the largest code; every element within half a step
    assert np.max(np.abs(formats.fp8_e4m3_to_f64(codes))) == 448.0
    assert np.all(np.abs(back - c) <= np.abs(c) * 2.0 ** -4 + 2.0 ** -10 * float(scale))
    z_codes, z_scale = formats.fp8_quantize_row(np.zeros(8))
    assert z_scale == 1.0 and not z_codes.any()


# ------------------------------------------------------------------------------------- fp4

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # the OCP E2M1 magnitudes by code 0..7


def test_fp4_decode_all_codes():
    from oracle.formats import fp4_e2m1_to_f64
    got = fp4_e2m1_to_f64(np.arange(16))
    want = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    assert np.array_equal(np.abs(got), np.abs(want)) and np.all(np.signbit(got[8:]))


def test_fp4_encode_round_trip_and_ties_to_even():
    from oracle.formats import f64_to_fp4_e2m1, fp4_e2m1_to_f64
    for code in range(16):
        if code == 8:
            continue                                   # -0 encodes as +0
        v = fp4_e2m1_to_f64(np.array([code]))
        assert f64_to_fp4_e2m1(v)[0] == code
    # midpoints go to the even mantissa; beyond 6 saturates
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             5.01: 6.0, 7.0: 6.0, 1e9: 6.0, -2.5: -2.0, -0.74: -0.5}
    for x, r in cases.items():
        assert fp4_e2m1_to_f64(f64_to_fp4_e2m1(np.array([x])))[0] == r, x


def test_fp4_row_quantization():
    """Per block of 16: the scale byte is the smallest power of two keeping the block's largest
    magnitude within 6 (found here by counting up), codes decode within half a step, element
    2i sits in the low nibble, an all-zero block gets 2**0."""
    from oracle.formats import fp4_quantize_row, fp4_unpack, fp4_e2m1_to_f64
    rng = np.random.default_rng(7)
    row = rng.standard_normal(128) * np.repeat(rng.uniform(1e-3, 100.0, 8), 16)
    row[32:48] = 0.0
    packed, sc = fp4_quantize_row(row)
    assert packed.shape == (64,) and sc.shape == (8,)
    for blk in range(8):
        x = row[16 * blk:16 * blk + 16]
        amax = np.max(np.abs(x))
        k = -200
        while amax > 0 and amax / 2.0 ** k > 6.0:
            k += 1
        if amax == 0:
            k = 0
        elif k == -200:
            while amax / 2.0 ** (k - 1) <= 6.0:
                k -= 1
        assert int(sc[blk]) == k + 127, blk
    dec = fp4_unpack(packed, sc)
    scale = np.repeat(2.0 ** (sc.astype(np.int64) - 127), 16)
    q = np.abs(row) / scale
    step = np.where(q < 2.0, 0.5, np.where(q < 4.0, 1.0, 2.0)) * scale
    assert np.all(np.abs(dec - row) <= step / 2 * (1 + 1e-12))
    assert np.all(dec[32:48] == 0.0)
    # nibble order: element 0 of the row is the low nibble of byte 0
    lo = fp4_e2m1_to_f64(packed[:1] & 0xF)[0] * scale[0]
    assert lo == dec[0]


def test_fp4_paged_row_round_trip():
    """A row of E2M1 magnitudes times a per-block power of two (exactly representable) stored in
    an fp4 paged cache reads back exactly; the cache's logical dim is twice its byte width."""
    from oracle.paged import PagedCache
    rng = np.random.default_rng(9)
    vals = rng.choice(np.array(E2M1_TABLE + [-v for v in E2M1_TABLE[1:]]), size=128)
    vals[::16] = 6.0                                  # every block reaches the top code
    row = vals * np.repeat(2.0 ** rng.integers(-20, 20, 8), 16)
    c = PagedCache.empty(2, 300, 64, 128, "fp4", perm_seed=3)
    assert c.dim == 128 and c.rows.shape[2] == 64
    c.write(1, 257, row)
    assert np.array_equal(c.read(1, 257), row)
