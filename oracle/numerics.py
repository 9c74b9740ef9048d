"""Bit-level decoding of the number formats the decode path consumes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.  The FP8 KV-cache
  deep dive (Hopper FP8 sparse decode, "The FP8 KVCache Format") has the MMA
  inputs in bfloat16 with float32 outputs.
* float8_e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities,
  S.1111.111 is NaN, so the largest finite magnitude is 448 (the
  "matrices, attention & GPU" explainer quotes e4m3 with a maximum of 448 in
  its DeepGEMM section).  Decoded here from that definition, not from a library.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16 array) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def f32_to_bf16_bits_rne(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns uint16 bit patterns.  NaN stays a quiet NaN; values that round past
    the largest finite bfloat16 become infinity, as IEEE rounding requires.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(is_nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def e4m3fn_decode(codes):
    """float8_e4m3fn codes (uint8 array) -> float64 values (NaN for 0x7F/0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    subnormal = sign * np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, subnormal, normal)
    v = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)
    return v


E4M3_MAX = 448.0
