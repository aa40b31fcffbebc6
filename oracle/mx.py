"""MXFP8 decoding for the oracle — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  It shares no code with the GPU library.

The pages report MXFP8-based attention (ultra-low-precision training of
attention modules, with the quantisation fused into the upstream projection
and normalisation kernels: "Meta redesigns AI training infrastructure...",
sections "Custom Kernels and 5D Parallelism for Trillion-Parameter Scale" and
"Key Numbers"; "GEM Training: How Meta Doubled the Efficiency of an LLM-Scale
Ads Foundation Model", body) without defining the format.  The reading here is
the OCP Microscaling (MX) format MXFP8 with E4M3 elements:

  * a block of 32 consecutive elements shares one scale X stored as E8M0, an
    8-bit biased exponent: X = 2^(E - 127), code 255 = NaN;
  * each element is FP8 E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 encodes subnormals m/8 * 2^-6, the all-ones
    exponent with all-ones mantissa is NaN (no infinities), largest finite
    magnitude 1.75 * 2^8 = 448;
  * the value of an element is X times its E4M3 value.

In the attention tensors a block is 32 consecutive head-dimension elements of
one row and head: codes [T, H, D] and scale codes [T, H, D / 32], both uint8.
Attention on MXFP8 inputs is the plain definition applied to the decoded
values (decoding is exact in float64).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def e4m3_value(codes) -> np.ndarray:
    """Float64 value of FP8 E4M3 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)


def e8m0_value(codes) -> np.ndarray:
    """Float64 value 2^(E - 127) of E8M0 scale codes (uint8 array); 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def decode(codes, scales) -> np.ndarray:
    """Values [T, H, D] of MXFP8 codes [T, H, D] with scale codes [T, H, D / 32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    T, H, D = codes.shape
    assert D % BLOCK == 0 and scales.shape == (T, H, D // BLOCK), (codes.shape, scales.shape)
    x = e4m3_value(codes).reshape(T, H, D // BLOCK, BLOCK)
    return (x * e8m0_value(scales)[..., None]).reshape(T, H, D)


def decode_f32(codes, scales) -> np.ndarray:
    """decode() as float32, for the oracle's float32 inputs.  Every finite MXFP8
    value with a scale code up to 246 is a float32 value; anything else is refused."""
    v = decode(codes, scales)
    with np.errstate(over="ignore"):
        f = v.astype(np.float32)
    assert np.isfinite(v).all() and np.array_equal(f.astype(np.float64), v), \
        "MXFP8 values outside what float32 holds exactly"
    return f
