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
