"""Decoders for the stored number formats, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bfloat16: the upper 16 bits of an IEEE-754 binary32; decoding appends 16
  zero bits.
* float8 E4M3FN, as in the OCP "8-bit Floating Point Specification (OFP8)":
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  encodes subnormals m/8 * 2^-6; the pattern S.1111.111 is NaN; there are no
  infinities, so exponent field 15 with mantissa 0..6 is an ordinary number
  (largest finite 448).  The pages call the cache format "fp8" and the packed
  DeepSeek sparse-MLA layout "fp8_ds_mla" ("GLM-5.2 vLLM Decode Context
  Parallelism", sections "Understand the cache-copy opportunity" and "See why
  vLLM 0.26.0 fails"); the E4M3 flavour is the one stated for the workload.
* The packed fp8 latent row: 512 codes in four groups of 128, each group
  with one float32 scale; the value of dimension d is
  decode(code[d]) * scale[d // 128].  Rope dimensions are stored as bf16.
"""

import numpy as np

FP8_GROUP = 128


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):
        return f32.astype(np.float64)


def f32_to_f64(x):
    """float32 -> float64 (exact widening)."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def e4m3fn_to_f64(codes):
    """OCP E4M3FN codes (uint8) -> float64, exactly, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    subnormal = (man / 8.0) * np.exp2(-6.0)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return sign * mag


def fp8_ds_latent_to_f64(codes, scales):
    """Packed fp8 latent rows -> float64 values.

    codes  uint8  [..., 512]   E4M3FN codes
    scales float32 [..., 4]    one scale per group of 128 dimensions
    returns float64 [..., 512] with value[d] = decode(code[d]) * scale[d // 128]
    """
    codes = np.asarray(codes)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    d = codes.shape[-1]
    assert d % FP8_GROUP == 0 and scales.shape[-1] == d // FP8_GROUP
    per_dim = np.repeat(scales, FP8_GROUP, axis=-1)
    return e4m3fn_to_f64(codes) * per_dim
