"""Stored number formats, written from their definitions (oracle; test infrastructure only).

* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits;
  the prefill-side cache precision of [vLLM-V4] section 3 ("prefill uses a
  bfloat16 KV cache").  Stored here as its 16-bit pattern (numpy uint16).
* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits, no infinities, one NaN pattern per sign (S.1111.111), largest finite
  value 448, subnormals m * 2**-9.  [SGLang-pools] section 4 stores indexer
  keys as 128 such codes plus one float32 scale; [vLLM-V4] section 3 uses a
  per-token fp8 attention cache in decode.  Stored as numpy uint8 codes.

* FP4 (indexer cache rows, [SGLang-pools] section 7): two 4-bit values per byte and one scale
  per 16 original values.  Readings (the pages fix neither the element nor the scale format):
  the element is OCP E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6), element 2i in the low nibble of byte i; the scale is a power of
  two stored as an E8M0 byte (value 2**(byte - 127)), the smallest one that keeps the block's
  largest magnitude within 6 (no clipping; 1 for an all-zero block).

Rounding is round-to-nearest-even from the exact float64 value, done once.
"""

from __future__ import annotations

import numpy as np

FP8_MAX = 448.0
FP8_MIN_NORMAL_EXP = -6      # smallest normal: 2**-6
FP8_SUBNORMAL_QUANTUM = 2.0 ** -9
BF16_MIN_NORMAL_EXP = -126


def _binade_exponent(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for positive finite a, exactly (via frexp)."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


# --------------------------------------------------------------------- bf16

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns: they are the upper half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even); returns float64.

    A normal bfloat16 in the binade [2**E, 2**(E+1)) has spacing 2**(E-7);
    below 2**-126 the spacing stays 2**-133 (subnormals).  Dividing by a power
    of two is exact in float64 and numpy's ``rint`` rounds half to even.
    Values beyond the largest finite bfloat16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    a = np.abs(x)
    nz = (a > 0) & np.isfinite(a)
    e = np.maximum(_binade_exponent(a[nz]), BF16_MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - 7)
    out[nz] = np.rint(x[nz] / quantum) * quantum
    over = np.abs(out) >= 2.0 ** 128          # rounded past the largest finite value
    out[over] = np.copysign(np.inf, out[over])
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (ties to even) and return the 16-bit patterns."""
    r = round_to_bf16(x).astype(np.float32)          # exact: bf16 values are float32 values
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------- fp8

def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 codes (uint8) to float64 by the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = man * FP8_SUBNORMAL_QUANTUM
    val = np.where(exp == 0, subnormal, normal)
    val = np.where((exp == 0xF) & (man == 0x7), np.nan, val)
    return sign * val


def round_to_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value (ties to even), saturating at +-448; returns float64.

    In a normal binade [2**E, 2**(E+1)) with E >= -6 the spacing is 2**(E-3);
    below 2**-6 the spacing is the subnormal quantum 2**-9.  Magnitudes above
    448 saturate to 448 (the OCP "saturating" conversion).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP8_MAX)
    out = np.zeros_like(a)
    nz = a > 0
    e = np.maximum(_binade_exponent(a[nz]), FP8_MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - 3)
    out[nz] = np.minimum(np.rint(a[nz] / quantum) * quantum, FP8_MAX)
    out = np.copysign(out, x)
    out[np.isnan(x)] = np.nan
    return out


def f64_to_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Round (ties to even, saturating) and encode to E4M3 codes (uint8)."""
    r = round_to_fp8_e4m3(x)
    a = np.abs(r)
    codes = np.zeros(r.shape, dtype=np.int64)
    sub = (a > 0) & (a < 2.0 ** FP8_MIN_NORMAL_EXP)
    codes[sub] = np.rint(a[sub] / FP8_SUBNORMAL_QUANTUM).astype(np.int64)
    nrm = a >= 2.0 ** FP8_MIN_NORMAL_EXP
    e = _binade_exponent(a[nrm])
    man = np.rint((a[nrm] / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    codes[nrm] = ((e + 7) << 3) | man
    codes[np.signbit(r)] |= 0x80
    codes[np.isnan(r)] = 0x7F
    return codes.astype(np.uint8)


# --------------------------------------------------------------------- fp4

FP4_MAX = 6.0
FP4_BLOCK = 16


def fp4_e2m1_to_f64(nibbles: np.ndarray) -> np.ndarray:
    """Decode E2M1 4-bit codes (values 0..15) by the format's definition."""
    c = np.asarray(nibbles, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    exp = (c >> 1) & 0x3
    man = c & 0x1
    val = np.where(exp == 0, man * 0.5, np.ldexp(1.0 + man / 2.0, exp - 1))
    return sign * val


def round_to_fp4_e2m1(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 value (ties to the even mantissa), saturating at +-6; returns float64.

    Spacing: 0.5 below 2, 1 in [2, 4), 2 in [4, 6].
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP4_MAX)
    quantum = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.rint(a / quantum) * quantum        # rint: half to even on the quantum grid
    return np.copysign(np.minimum(r, FP4_MAX), x)


def f64_to_fp4_e2m1(x: np.ndarray) -> np.ndarray:
    """Round (ties to even, saturating) and encode to E2M1 nibbles (values 0..15)."""
    r = round_to_fp4_e2m1(x)
    a = np.abs(r)
    code = np.zeros(r.shape, dtype=np.int64)
    code[a == 0.5] = 0x1
    nz = a >= 1.0
    e = _binade_exponent(a[nz])                # 0, 1 or 2
    man = np.rint((a[nz] / np.ldexp(1.0, e) - 1.0) * 2.0).astype(np.int64)
    code[nz] = ((e + 1) << 1) | man
    code[np.signbit(r) & (a > 0)] |= 0x8
    return code.astype(np.uint8)


def e8m0_to_f64(b: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes: 2**(b - 127)."""
    return np.ldexp(1.0, np.asarray(b, dtype=np.int64) - 127)


def fp4_quantize_row(c: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """One row (length a multiple of 16) to FP4: (packed bytes [d/2], E8M0 scale bytes [d/16]).

    Per block of 16 values: scale = 2**ceil(log2(amax / 6)) (1 for an all-zero block), codes =
    nearest-even E2M1 of value / scale; element 2i in the low nibble of byte i.
    """
    c = np.asarray(c, dtype=np.float64)
    d = c.shape[-1]
    assert d % FP4_BLOCK == 0
    blocks = c.reshape(d // FP4_BLOCK, FP4_BLOCK)
    amax = np.max(np.abs(blocks), axis=1)
    k = np.zeros(len(amax), dtype=np.int64)
    nz = amax > 0
    # smallest k with amax / 2**k <= 6: k = ceil(log2(amax / 6)), found exactly with frexp
    m, e = np.frexp(amax[nz] / FP4_MAX)      # amax/6 = m * 2**e, m in [0.5, 1)
    k[nz] = np.where(m == 0.5, e - 1, e)
    nib = f64_to_fp4_e2m1(blocks / np.ldexp(1.0, k)[:, None]).reshape(d)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    return packed, (k + 127).astype(np.uint8)


def fp4_unpack(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of FP4 rows: packed [..., d/2] bytes, scales [..., d/16] E8M0."""
    p = np.asarray(packed, dtype=np.uint8)
    nib = np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    v = fp4_e2m1_to_f64(nib)
    sc = e8m0_to_f64(scales)
    return v * np.repeat(sc, FP4_BLOCK, axis=-1)


def fp8_quantize_row(c: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Per-row fp8 quantization: one float32 scale = amax / 448 and E4M3 codes of c / scale.

    Reading taken for the per-token fp8 format ([vLLM-V4] section 3; one
    scale per 128-value indexer row in [SGLang-pools] section 4): the scale
    is amax/448 rounded to float32 (1 when the row is all zero), and the codes
    are the saturating nearest-even encoding of c divided by the stored
    scale.
    """
    c = np.asarray(c, dtype=np.float64)
    amax = float(np.max(np.abs(c))) if c.size else 0.0
    scale = np.float32(amax / FP8_MAX) if amax > 0 else np.float32(1.0)
    return f64_to_fp8_e4m3(c / np.float64(scale)), scale


# --------------------------------------------------------------- generic

DTYPES = ("f32", "bf16", "fp8", "fp4")


def decode_stored(values: np.ndarray, dtype: str, scales: np.ndarray | None = None) -> np.ndarray:
    """Exact float64 value of stored rows: float32 as is, bf16 widened, fp8 code * row scale."""
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(values)
    if dtype == "fp8":
        v = fp8_e4m3_to_f64(values)
        return v * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
    if dtype == "fp4":
        return fp4_unpack(values, scales)
    raise ValueError(dtype)


def encode_row(c: np.ndarray, dtype: str):
    """Store one float64 row in ``dtype``: returns (stored values, scale or None)."""
    if dtype == "f32":
        return np.asarray(c, dtype=np.float64).astype(np.float32), None
    if dtype == "bf16":
        return f64_to_bf16_bits(c), None
    if dtype == "fp8":
        return fp8_quantize_row(c)
    if dtype == "fp4":
        return fp4_quantize_row(c)
    raise ValueError(dtype)
