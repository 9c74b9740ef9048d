"""Pins of the bfloat16 / e4m3fn decoding and of the 656-byte FP8 record
against closed forms, the pages' figures and torch's own conversions."""

import numpy as np
import torch

from oracle import numerics as Nm
from oracle import fp8cache as F8
from workloads.gen import encode_fp8_records


def test_e4m3_all_codes_closed_form_and_library():
    codes = np.arange(256, dtype=np.uint8)
    got = Nm.e4m3fn_decode(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(got[c]) and np.isnan(lib[c])
            continue
        ref = s * (2.0 ** -6) * (m / 8) if e == 0 else s * 2.0 ** (e - 7) * (1 + m / 8)
        assert got[c] == ref == lib[c]
    finite = got[np.isfinite(got)]
    assert finite.size == 254 and finite.max() == 448.0


def test_bf16_bits_roundtrip_and_rne_against_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # exact ties: bf16 value + half an ulp
    base = torch.from_numpy(x[:2000]).to(torch.bfloat16).to(torch.float32).numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-45], dtype=np.float32)
    allx = np.concatenate([x, ties, special])
    ours = Nm.f32_to_bf16_bits_rne(allx)
    lib = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)
    back = Nm.bf16_bits_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(allx).to(torch.bfloat16).to(torch.float64).numpy())


def test_record_layout_matches_pages(golden):
    g = golden['fp8_record_bytes']
    assert F8.RECORD_BYTES == g['value'] == sum(g['parts'])
    assert list(F8.record_layout()) == g['parts']


def test_dequant_against_torch_conversions():
    gen = torch.Generator().manual_seed(3)
    x = torch.randn(300, 576, generator=gen)
    x[5, :128] = 0.0                       # an all-zero tile (scale 1)
    x[6, 7] = 1e-9                         # subnormal region
    rec = encode_fp8_records(x[:, :512].contiguous(), x[:, 512:].to(torch.bfloat16))
    got = F8.dequant_records(rec.numpy())
    codes = rec[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
    scales = rec[:, 512:528].contiguous().view(torch.float32)
    ref_lat = (codes.view(300, 4, 128) * scales[:, :, None]).view(300, 512).to(torch.bfloat16)
    ref_rope = rec[:, 528:].contiguous().view(torch.bfloat16)
    ref = torch.cat([ref_lat, ref_rope], dim=1).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    # dequantised values approximate the source within e4m3 resolution
    err = np.abs(got[:, :512] - x[:, :512].numpy())
    amax = np.abs(x[:, :512].numpy()).reshape(300, 4, 128).max(axis=2)
    assert np.all(err.reshape(300, 4, 128) <= (amax / 448.0 * 16.0 + amax * 2.0 ** -8 + 1e-6)[:, :, None])


# ------------------------------------------------------------------ the 528-byte record (512-wide head)

def test_e8m0_all_codes_closed_form_and_library():
    e = np.arange(256, dtype=np.uint8)
    got = F8.e8m0_decode(e)
    lib = torch.from_numpy(e.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(255):
        assert got[c] == 2.0 ** (c - 127) == lib[c]
    assert np.isnan(got[255]) and np.isnan(lib[255])


def test_v41_record_layout_matches_pages():
    # 512 e4m3 values, then one e8m0 scale for every 32 values: 512 + 16 bytes
    assert F8.V41_RECORD_BYTES == 512 * 1 + (512 // 32) * 1 == 528


def test_v41_dequant_against_torch_conversions():
    from workloads.gen import encode_v41_records
    g = torch.Generator().manual_seed(5)
    x = torch.randn(300, 512, generator=g) * torch.logspace(-3, 3, 512)[None, :]   # spread of group scales
    x[7, 64:96] = 0.0                                                                # an all-zero group
    rec = encode_v41_records(x).numpy()
    got = F8.dequant_records_v41(rec)
    codes = torch.from_numpy(rec[:, :512].copy()).view(torch.float8_e4m3fn).to(torch.float64)
    scales = torch.from_numpy(rec[:, 512:].copy()).view(torch.float8_e8m0fnu).to(torch.float64)
    ref = (codes.view(300, 16, 32) * scales[..., None]).view(300, 512).numpy()
    assert np.array_equal(got, ref)
    # the encoder's power-of-two scales keep every code finite and within e4m3's precision of x
    xs = x.double().numpy()
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - xs) <= 2.0 ** -4 * np.abs(xs) + np.repeat(F8.e8m0_decode(rec[:, 512:]), 32, 1) * 2.0 ** -9)
    assert np.all(got[7, 64:96] == 0.0)


def test_v41_decode_is_attention_over_the_dequantised_rows():
    """The oracle's decode over 528-byte records equals the plain two-pass
    attention over the dequantised 512-wide rows, with V = K."""
    from oracle import attention as A
    from workloads import make_v41_sparse
    w = make_v41_sparse(2, 1, 4, pool_tokens_per_seq=256, topk=40, invalid_frac=0.1, seed=9)
    q = w.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    kv = w.kv.numpy().reshape(-1, 528)
    idx = w.indices.numpy()
    out, lse = A.decode(q, kv, w.softmax_scale, indices=idx, kv_format='fp8_528')
    for b in range(2):
        rows = idx[b, 0][idx[b, 0] >= 0]
        K = F8.dequant_records_v41(kv[rows])
        qh = Nm.bf16_bits_to_f64(q[b, 0])
        s = w.softmax_scale * qh @ K.T
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        assert np.max(np.abs(out[b, 0] - (p @ K) / p.sum(axis=1, keepdims=True))) < 1e-12
        assert np.max(np.abs(lse[b, :, 0] - (m[:, 0] + np.log(p.sum(axis=1))))) < 1e-12


# ---------------------------------------------------------------- 288-byte FP4 records

def test_e2m1_all_codes_closed_form():
    # the OCP e2m1 element: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, bit 3 the sign
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    got = F8.e2m1_decode(np.arange(16))
    assert np.array_equal(got, np.array(want)) and np.array_equal(np.signbit(got), np.signbit(np.array(want)))


def test_fp4_record_layout_matches_pages():
    # 512 e2m1 values two per byte, then one e4m3 scale for every 16 values: 256 + 32 bytes
    assert F8.FP4_RECORD_BYTES == 512 // 2 + (512 // 16) * 1 == 288


def test_fp4_nibble_order_and_group_scales():
    """Even-indexed values sit in the low nibble; scale byte k covers values 16k..16k+15."""
    rec = np.zeros(288, dtype=np.uint8)
    rec[0] = 0x72                     # values 0, 1 = codes 2, 7 = 1.0, 6.0
    rec[1] = 0xF9                     # values 2, 3 = codes 9, 15 = -0.5, -6.0
    rec[8] = 0x35                     # values 16, 17 = codes 5, 3 = 3.0, 1.5
    rec[256:] = 0x38                  # e4m3 1.0
    rec[257] = 0x40                   # e4m3 2.0 for values 16..31
    rec[258] = 0x7F                   # e4m3 NaN for values 32..47
    v = F8.dequant_records_fp4(rec)
    assert v.shape == (512,)
    assert list(v[:4]) == [1.0, 6.0, -0.5, -6.0]
    assert list(v[16:18]) == [6.0, 3.0]
    assert np.all(np.isnan(v[32:48])) and np.all(v[48:] == 0.0) and np.all(v[4:16] == 0.0)


def test_fp4_dequant_against_torch_scales_and_table():
    """Dequantised values equal a table lookup of each nibble times torch's
    float8_e4m3fn decode of the group scale, and stay within 1.5 scale units
    of the encoded float32 values."""
    from workloads.gen import encode_fp4_records
    g = torch.Generator().manual_seed(5)
    x = torch.randn((64, 512), generator=g) * torch.exp(torch.randn((64, 1), generator=g))
    rec = encode_fp4_records(x).numpy()
    got = F8.dequant_records_fp4(rec)
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])
    lo, hi = rec[:, :256] & 0xF, rec[:, :256] >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(64, 512)
    scales = torch.from_numpy(rec[:, 256:].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = table[codes] * np.repeat(scales, 16, axis=1)
    assert np.array_equal(got, want)
    s = np.repeat(scales, 16, axis=1)
    assert np.all(np.abs(got - x.double().numpy()) <= 1.5 * s)


def test_fp4_decode_is_attention_over_the_dequantised_rows():
    """The oracle's decode over 288-byte records equals the plain two-pass
    attention over the dequantised 512-wide rows, with V = K."""
    from oracle import attention as A
    from workloads import make_fp4_sparse
    w = make_fp4_sparse(2, 1, 4, pool_tokens_per_seq=256, topk=40, invalid_frac=0.1, seed=9)
    q = w.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    kv = w.kv.numpy().reshape(-1, 288)
    idx = w.indices.numpy()
    out, lse = A.decode(q, kv, w.softmax_scale, indices=idx, kv_format='fp4_288')
    for b in range(2):
        rows = idx[b, 0][idx[b, 0] >= 0]
        K = F8.dequant_records_fp4(kv[rows])
        qh = Nm.bf16_bits_to_f64(q[b, 0])
        s = w.softmax_scale * qh @ K.T
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        assert np.max(np.abs(out[b, 0] - (p @ K) / p.sum(axis=1, keepdims=True))) < 1e-12
        assert np.max(np.abs(lse[b, :, 0] - (m[:, 0] + np.log(p.sum(axis=1))))) < 1e-12
