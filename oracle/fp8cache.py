"""The 656-byte FP8 latent KV-cache record and its dequantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the FlashMLA "Hopper FP8 sparse decode" deep dive, section "The FP8
KVCache Format" (also its translations on the FlashMLA-deep-dive page and the
bilingual FlashMLA documentation page).  Per token, the first 512 latent values
are quantised in tiles of 1x128 to float8_e4m3 with one float32 scale per tile;
the 64 RoPE values stay bfloat16; one token takes 512 + 4*4 + 64*2 = 656 bytes.
Inside the kernel the e4m3 values are dequantised to bfloat16 and concatenated
with the RoPE part before bfloat16 MMAs.

Readings where the pages leave a step open (each listed in the design notes):
* byte order inside the record: [512 e4m3 | 4 float32 scales | 64 bfloat16],
  i.e. offsets 0 / 512 / 528, little-endian, in the order the pages list them;
* dequantised value: bf16_rne(float32(e4m3) * float32 scale) -- the e4m3 to
  float32 step is exact, the product is one float32 rounding, then one
  bfloat16 round-to-nearest-even.
"""

import numpy as np

from .numerics import bf16_bits_to_f64, e4m3fn_decode, f32_to_bf16_bits_rne

RECORD_BYTES = 656
LATENT = 512
ROPE = 64
TILE = 128
SCALE_OFFSET = 512
ROPE_OFFSET = 528


def record_layout():
    """(bytes of e4m3 data, bytes of scales, bytes of RoPE) per token."""
    return LATENT * 1, (LATENT // TILE) * 4, ROPE * 2


def dequant_records(rec):
    """uint8 records [..., 656] -> float64 K values [..., 576] (bf16-exact).

    Columns 0..511 are the dequantised latent part, 512..575 the RoPE part.
    """
    rec = np.asarray(rec, dtype=np.uint8)
    assert rec.shape[-1] == RECORD_BYTES
    lead = rec.shape[:-1]
    flat = np.ascontiguousarray(rec.reshape(-1, RECORD_BYTES))
    codes = flat[:, :LATENT]
    scales = np.ascontiguousarray(flat[:, SCALE_OFFSET:ROPE_OFFSET]).view('<f4').astype(np.float32)  # [n, 4]
    rope_bits = np.ascontiguousarray(flat[:, ROPE_OFFSET:]).view('<u2')                               # [n, 64]
    vals = e4m3fn_decode(codes).astype(np.float32)            # exact in float32
    tile_scale = np.repeat(scales, TILE, axis=1)              # [n, 512]
    prod = (vals * tile_scale).astype(np.float32)             # one float32 rounding
    latent = bf16_bits_to_f64(f32_to_bf16_bits_rne(prod))
    rope = bf16_bits_to_f64(rope_bits)
    out = np.concatenate([latent, rope], axis=1)
    return out.reshape(lead + (LATENT + ROPE,))


# --------------------------------------------------------------------------
# The 528-byte record of the newer model (FlashMLA README copy, "FP8 / FP4 KV
# Cache Format"): head_dim 512 with the 64 RoPE dimensions quantised as well;
# per token 512 float8_e4m3 values, then 16 float8_e8m0 scales, one for every
# 32 consecutive values; no bfloat16 part.  K and V are both the 512 values.
#
# Readings: an e8m0 byte e is the power of two 2^(e - 127), with e = 255 NaN
# (the OCP "E8M0" scale format); the dequantised value e4m3(x) * 2^(e - 127)
# is exact in float64, and also in bfloat16 unless it leaves bfloat16's
# exponent range, so it is returned unrounded.

V41_RECORD_BYTES = 528
V41_DIM = 512
V41_GROUP = 32


def e8m0_decode(e):
    """float8_e8m0 bytes -> float64: 2^(e - 127), NaN for 255."""
    e = np.asarray(e, dtype=np.int64)
    out = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, out)


def dequant_records_v41(rec):
    """uint8 records [..., 528] -> float64 K (= V) values [..., 512]."""
    rec = np.asarray(rec, dtype=np.uint8)
    assert rec.shape[-1] == V41_RECORD_BYTES
    lead = rec.shape[:-1]
    flat = np.ascontiguousarray(rec.reshape(-1, V41_RECORD_BYTES))
    vals = e4m3fn_decode(flat[:, :V41_DIM]).astype(np.float64)
    scales = e8m0_decode(flat[:, V41_DIM:])                      # [n, 16]
    out = vals * np.repeat(scales, V41_GROUP, axis=1)
    return out.reshape(lead + (V41_DIM,))


# --------------------------------------------------------------------------
# The 288-byte FP4 record of the same 512-wide head (FlashMLA README copy,
# "FP8 / FP4 KV Cache Format"): per token 256 bytes holding 512 e2m1 values,
# two per byte with the even-indexed value in the low nibble, then 32
# float8_e4m3 scales, one for every 16 consecutive values.  K and V are both
# the 512 values.
#
# Readings: e2m1 is the OCP microscaling FP4 element (1 sign bit, 2 exponent
# bits with bias 1, 1 mantissa bit, no infinities or NaN): magnitudes 0, 0.5,
# 1, 1.5, 2, 3, 4, 6.  The dequantised value e2m1 * e4m3 has at most five
# significant bits and lies in [2^-10, 2688], so it is exact in float64 and in
# bfloat16 and is returned unrounded; an e4m3 NaN scale (0x7F/0xFF) gives NaN.

FP4_RECORD_BYTES = 288
FP4_DIM = 512
FP4_GROUP = 16


def e2m1_decode(codes):
    """4-bit e2m1 codes (0..15) -> float64 values."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    return sign * mag


def dequant_records_fp4(rec):
    """uint8 records [..., 288] -> float64 K (= V) values [..., 512]."""
    rec = np.asarray(rec, dtype=np.uint8)
    assert rec.shape[-1] == FP4_RECORD_BYTES
    lead = rec.shape[:-1]
    flat = np.ascontiguousarray(rec.reshape(-1, FP4_RECORD_BYTES))
    packed = flat[:, :FP4_DIM // 2].astype(np.int64)
    codes = np.empty((flat.shape[0], FP4_DIM), dtype=np.int64)
    codes[:, 0::2] = packed & 0xF          # even index: low nibble
    codes[:, 1::2] = packed >> 4
    scales = e4m3fn_decode(flat[:, FP4_DIM // 2:])                 # [n, 32]
    out = e2m1_decode(codes) * np.repeat(scales, FP4_GROUP, axis=1)
    return out.reshape(lead + (FP4_DIM,))
