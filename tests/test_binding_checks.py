"""The Python binding checks every tensor against the problem before it calls
the C ABI: dtype, contiguity, element count and last dimension, then that the
tensor is on a GPU.  Runs on the CPU: tensors on the ``meta`` device carry
shapes and dtypes without memory, so a call whose shapes are all right fails
only at the final device check, and a wrong one fails earlier, naming the
argument."""

import pytest
import torch

import mla_decode_amd as mla

M = "meta"
bf16, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


def T(*shape, dtype=f32):
    return torch.empty(shape, dtype=dtype, device=M)


B, S, H, NB, MB = 4, 2, 128, 32, 8


def dense(kv_format="bf16", out_dtype="bf16"):
    return mla.make_problem(B, S, H, NB, MB, kv_format=kv_format, out_dtype=out_dtype)


def dense_args(p, **over):
    rec = {"bf16": (576, bf16), "fp8": (656, u8)}["bf16" if p.kv_format == 0 else "fp8"]
    a = dict(q=T(B, S, H, 576, dtype=bf16), kv_cache=T(NB, 64, 1, rec[0], dtype=rec[1]),
             block_table=T(B, MB, dtype=i32), cache_seqlens=T(B, dtype=i32), workspace=T(1024),
             out=T(B, S, H, 512, dtype=f32 if p.out_dtype == 1 else bf16), lse=T(B, H, S))
    a.update(over)
    return a


def call_dense(p, a):
    m = mla.Metadata()
    mla.decode_fwd(p, a["q"], a["kv_cache"], a["block_table"], a["cache_seqlens"], m, a["workspace"], a["out"],
                   a["lse"])


def test_well_formed_dense_call_reaches_the_device_check():
    for fmt in ("bf16", "fp8"):
        for od in ("bf16", "fp32"):
            p = dense(fmt, od)
            with pytest.raises(ValueError, match="must be a device tensor"):
                call_dense(p, dense_args(p))


@pytest.mark.parametrize("name,bad,msg", [
    ("out", T(B, S, H, 512, dtype=f32), "out must be torch.bfloat16"),          # fp32 out, bf16 problem
    ("out", T(B, S, H, 256, dtype=bf16), "out must have"),
    ("q", T(B, S, H, 512, dtype=bf16), "q must have"),                          # 512-wide q, 576 problem
    ("q", T(B, S, H, 576, dtype=f32), "q must be torch.bfloat16"),
    ("lse", T(B, S, H), None),                                                  # same numel, accepted
    ("lse", T(B, H, S + 1), "lse must have"),
    ("block_table", T(B, MB - 1, dtype=i32), "block_table must have"),
    ("block_table", T(B, MB, dtype=torch.int64), "block_table must be torch.int32"),
    ("cache_seqlens", T(B + 1, dtype=i32), "cache_seqlens must have"),
    ("kv_cache", T(NB, 64, 1, 656, dtype=u8), "kv_cache must be torch.bfloat16"),
    ("kv_cache", T(NB - 1, 64, 1, 576, dtype=bf16), "kv_cache holds"),
    ("kv_cache", T(NB, 64, 1, 512, dtype=bf16), "last dimension of 576"),
    ("q", T(B, S, 576, H, dtype=bf16).transpose(2, 3), "q must be contiguous"),
])
def test_dense_rejections(name, bad, msg):
    p = dense()
    if msg is None:
        with pytest.raises(ValueError, match="must be a device tensor"):
            call_dense(p, dense_args(p, **{name: bad}))
        return
    with pytest.raises(ValueError, match=msg):
        call_dense(p, dense_args(p, **{name: bad}))


def test_fp32_problem_rejects_bf16_out():
    p = dense(out_dtype="fp32")
    with pytest.raises(ValueError, match="out must be torch.float32"):
        call_dense(p, dense_args(p, out=T(B, S, H, 512, dtype=bf16)))


def test_fp8_problem_rejects_short_records():
    p = dense("fp8")
    with pytest.raises(ValueError, match="last dimension of 656"):
        call_dense(p, dense_args(p, kv_cache=T(NB, 64, 1, 528, dtype=u8)))


def _sparse(topk=128, kv_format="bf16"):
    return mla.make_problem(B, S, H, NB, topk=topk, kv_format=kv_format)


def test_sparse_rejections():
    p = _sparse()
    m = mla.Metadata()
    q, kv, out, lse, ws = T(B, S, H, 576, dtype=bf16), T(NB, 64, 1, 576, dtype=bf16), T(B, S, H, 512, dtype=bf16), \
        T(B, H, S), T(64)
    good = T(B, S, 128, dtype=i32)
    with pytest.raises(ValueError, match="must be a device tensor"):
        mla.sparse_decode_fwd(p, q, kv, good, m, ws, out, lse)
    with pytest.raises(ValueError, match="indices must have"):
        mla.sparse_decode_fwd(p, q, kv, T(B, S, 64, dtype=i32), m, ws, out, lse)
    with pytest.raises(ValueError, match="topk_length must have"):
        mla.sparse_decode_fwd(p, q, kv, good, m, ws, out, lse, topk_length=T(B, dtype=i32))
    with pytest.raises(ValueError, match="attn_sink must have"):
        mla.sparse_decode_fwd(p, q, kv, good, m, ws, out, lse, attn_sink=T(H - 1))
    # 512-wide head with 528-byte records
    p = _sparse(kv_format="fp8_528")
    q5 = T(B, S, H, 512, dtype=bf16)
    with pytest.raises(ValueError, match="must be a device tensor"):
        mla.sparse_decode_fwd(p, q5, T(NB, 64, 1, 528, dtype=u8), good, m, ws, out, lse)
    with pytest.raises(ValueError, match="q must have"):
        mla.sparse_decode_fwd(p, q, T(NB, 64, 1, 528, dtype=u8), good, m, ws, out, lse)


def test_prefill_rejections():
    s_q, s_kv, topk = 3, 200, 64
    q, idx = T(s_q, H, 576, dtype=bf16), T(s_q, 1, topk, dtype=i32)
    with pytest.raises(ValueError, match="kv must be bfloat16"):
        mla.sparse_prefill(q, T(s_kv, 1, 576, dtype=f32), idx)
    with pytest.raises(ValueError, match="kv must be bfloat16"):
        mla.sparse_prefill(q, T(s_kv, 1, 600, dtype=u8), idx)
    p = mla.make_problem(1, s_q, H, (s_kv + 63) // 64, topk=topk)
    m = mla.Metadata()
    out, lse, ws = T(s_q, H, 512, dtype=bf16), T(H, s_q), T(64)
    with pytest.raises(ValueError, match="must be a device tensor"):
        mla.sparse_prefill_fwd(p, s_kv, q, T(s_kv, 1, 576, dtype=bf16), idx, m, ws, out, lse)
    with pytest.raises(ValueError, match="kv holds"):
        mla.sparse_prefill_fwd(p, s_kv, q, T(s_kv - 1, 1, 576, dtype=bf16), idx, m, ws, out, lse)


def test_combine_rejections():
    n, h, s = 6, 16, 2
    so = T(n + 1, dtype=i32)
    out, lse = T(n // s, s, h, 512), T(n // s, h, s)
    with pytest.raises(ValueError, match="must be a device tensor"):
        mla.combine(n, h, s, T(10, h, 512), T(10, h), so, out, lse)
    with pytest.raises(ValueError, match="o_part must have"):
        mla.combine(n, h, s, T(10, h, 256), T(10, h), so, out, lse)
    with pytest.raises(ValueError, match="split_offsets must have"):
        mla.combine(n, h, s, T(10, h, 512), T(10, h), T(n, dtype=i32), out, lse)
    with pytest.raises(ValueError, match="out must have"):
        mla.combine(n, h, s, T(10, h, 512), T(10, h), so, T(n, h, 256), lse)
    with pytest.raises(ValueError, match="out must be a bfloat16 or float32"):
        mla.combine(n, h, s, T(10, h, 512), T(10, h), so, T(n, h, 512, dtype=torch.float16), lse)
    with pytest.raises(ValueError, match="lse must have"):
        mla.combine(n, h, s, T(10, h, 512), T(10, h), so, out, T(n))


def test_gather_rows_rejections():
    p = dense()
    with pytest.raises(ValueError, match="rows_out must have"):
        mla.debug_gather_rows(p, T(B, MB, dtype=i32), T(B, dtype=i32), T(B * S, 64, dtype=i32))
    with pytest.raises(ValueError, match="must be a device tensor"):
        mla.debug_gather_rows(p, T(B, MB, dtype=i32), T(B, dtype=i32), T(B * S, 64 * MB, dtype=i32))
