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
