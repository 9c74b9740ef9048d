"""Absorbed-MLA decoding for MI355X (gfx950): thin Python binding.

The functions mirror the C entry points in ``include/mla_decode.h``
(``mla_get_decode_metadata``, ``mla_decode_fwd``, ``mla_sparse_decode_fwd``,
``mla_combine``, ...).  PyTorch only supplies device memory and the current
stream; each call checks tensor placement, dtype and contiguity, passes raw
pointers, and raises ``MlaError`` on a non-OK status.  All compute runs in the
HIP library; if it is not built, importing the binding's functions raises.
"""

import ctypes
import math

import torch

from . import _lib
from ._lib import MlaError, Problem, Metadata  # noqa: F401

__all__ = ["make_problem", "plan", "workspace_bytes", "get_decode_metadata", "decode_fwd",
           "sparse_decode_fwd", "sparse_prefill_fwd", "sparse_prefill", "combine", "debug_gather_rows", "Decoder",
           "MlaError", "abi_version", "check_inputs", "decode_step_noalloc"]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, numel=None, last_dim=None):
    """Check one tensor argument's dtype, contiguity, element count and last
    dimension (where the problem fixes them).  Raises ValueError.  Placement is
    checked afterwards, for all arguments at once, by ``_on_gpu``."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()} (shape {tuple(t.shape)})")
    if last_dim is not None and (t.dim() == 0 or t.shape[-1] != last_dim):
        raise ValueError(f"{name} must have a last dimension of {last_dim}, got shape {tuple(t.shape)}")
    return t


def _on_gpu(**tensors):
    """Every given tensor (None: absent optional argument) lives on a GPU."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")


# bytes of one cached token row per kv_format
_RECORD_BYTES = {_lib.KV_BF16_576: 1152, _lib.KV_FP8_656: 656, _lib.KV_FP8_528: 528, _lib.KV_FP4_288: 288}


def _out_dtype(problem):
    return torch.float32 if problem.out_dtype == _lib.OUT_FP32 else torch.bfloat16


def _check_q_out(problem, q, out, lse):
    """q [batch, s_q, h_q, d_qk] bfloat16, out [batch, s_q, h_q, 512] in the problem's output dtype,
    lse [batch, h_q, s_q] float32 (for prefill, batch = 1 and the leading dimension may be dropped)."""
    B, S, H = problem.batch, problem.s_q, problem.h_q
    _need(q, "q", torch.bfloat16, B * S * H * problem.d_qk, problem.d_qk)
    _need(out, "out", _out_dtype(problem), B * S * H * 512, 512)
    _need(lse, "lse", torch.float32, B * H * S)


def _check_kv(problem, kv, rows, name="kv_cache"):
    """At least ``rows`` cached rows in the problem's format: bfloat16 [..., 576] or uint8 [..., record bytes]."""
    rec = _RECORD_BYTES[problem.kv_format]
    if problem.kv_format == _lib.KV_BF16_576:
        _need(kv, name, torch.bfloat16, None, 576)
    else:
        _need(kv, name, torch.uint8, None, rec)
    if kv.numel() * kv.element_size() < rows * rec:
        raise ValueError(f"{name} holds {kv.numel() * kv.element_size()} bytes, the problem needs {rows} rows of "
                         f"{rec} bytes")


def _check_table(problem, table_or_indices, cache_seqlens):
    if problem.topk > 0:
        _need(table_or_indices, "indices", torch.int32, problem.batch * problem.s_q * problem.topk)
    else:
        _need(table_or_indices, "block_table", torch.int32, problem.batch * problem.max_blocks_per_seq)
        _need(cache_seqlens, "cache_seqlens", torch.int32, problem.batch)


def abi_version():
    return _lib.load().mla_abi_version()


def make_problem(batch, s_q, h_q, num_blocks, max_blocks_per_seq=0, *, topk=0, causal=False, kv_format="bf16",
                 out_dtype="bf16", softmax_scale=None, rescale_threshold=0.0):
    p = Problem()
    d_qk = 512 if kv_format in ("fp8_528", "fp4_288") else 576
    p.batch, p.s_q, p.h_q, p.h_kv, p.d_qk, p.d_v, p.block_size = batch, s_q, h_q, 1, d_qk, 512, 64
    p.num_blocks, p.max_blocks_per_seq, p.topk, p.causal = num_blocks, max_blocks_per_seq, topk, int(bool(causal))
    p.kv_format = {"bf16": _lib.KV_BF16_576, "fp8": _lib.KV_FP8_656, "fp8_528": _lib.KV_FP8_528,
                   "fp4_288": _lib.KV_FP4_288}[kv_format]
    p.out_dtype = {"bf16": _lib.OUT_BF16, "fp32": _lib.OUT_FP32}[out_dtype]
    p.softmax_scale = 1.0 / math.sqrt(576) if softmax_scale is None else float(softmax_scale)
    p.rescale_threshold = float(rescale_threshold)
    return p


def plan(problem, num_cus=0):
    """Host-side plan (mla_plan): partitions, head blocks, metadata and workspace sizes."""
    lib = _lib.load()
    m = Metadata()
    _lib.check("mla_plan", lib.mla_plan(ctypes.byref(problem), int(num_cus), ctypes.byref(m)))
    return m


def workspace_bytes(meta):
    return int(_lib.load().mla_workspace_bytes(ctypes.byref(meta)))


def _optional(t, name, dtype, numel):
    if t is None:
        return None
    return _need(t, name, dtype, numel)


def _topk_length(problem, topk_length):
    """Sparse only: [batch, s_q] int32 or None; ignored (None) for dense problems."""
    if problem.topk == 0:
        return None
    return _optional(topk_length, "topk_length", torch.int32, problem.batch * problem.s_q)


def _attn_sink(h_q, attn_sink):
    return _optional(attn_sink, "attn_sink", torch.float32, h_q)


def get_decode_metadata(problem, cache_seqlens, meta, meta_buf, stream=None, topk_length=None):
    """Split-KV scheduler: fill ``meta_buf`` (device uint8/int32 tensor >= meta.bytes) with the schedule.
    Dense problems read cache_seqlens; sparse ones read topk_length (None: all topk entries)."""
    lib = _lib.load()
    _need(meta_buf, "meta_buf", None)
    if meta_buf.numel() * meta_buf.element_size() < meta.bytes:
        raise ValueError("meta_buf too small")
    if problem.topk > 0:
        cache_seqlens = None
    else:
        _need(cache_seqlens, "cache_seqlens", torch.int32, problem.batch)
    tl = _topk_length(problem, topk_length)
    _on_gpu(meta_buf=meta_buf, cache_seqlens=cache_seqlens, topk_length=tl)
    meta.dev = meta_buf.data_ptr()
    _lib.check("mla_get_decode_metadata", lib.mla_get_decode_metadata(
        ctypes.byref(problem), _ptr(cache_seqlens), _ptr(tl), ctypes.byref(meta), _stream(stream)))
    return meta


def decode_fwd(problem, q, kv_cache, block_table, cache_seqlens, meta, workspace, out, lse, stream=None,
               attn_sink=None):
    """Dense paged decode (mla_decode_fwd)."""
    lib = _lib.load()
    _check_q_out(problem, q, out, lse)
    _check_kv(problem, kv_cache, problem.num_blocks * 64)
    _check_table(problem, block_table, cache_seqlens)
    _need(workspace, "workspace", None)
    sink = _attn_sink(problem.h_q, attn_sink)
    _on_gpu(q=q, kv_cache=kv_cache, block_table=block_table, cache_seqlens=cache_seqlens, workspace=workspace,
            out=out, lse=lse, attn_sink=sink)
    _lib.check("mla_decode_fwd", lib.mla_decode_fwd(
        ctypes.byref(problem), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), _ptr(sink),
        ctypes.byref(meta), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _stream(stream)))


def sparse_decode_fwd(problem, q, kv_cache, indices, meta, workspace, out, lse, stream=None, topk_length=None,
                      attn_sink=None):
    """Top-k sparse decode (mla_sparse_decode_fwd)."""
    lib = _lib.load()
    _check_q_out(problem, q, out, lse)
    _check_kv(problem, kv_cache, problem.num_blocks * 64)
    _check_table(problem, indices, None)
    _need(workspace, "workspace", None)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
    _on_gpu(q=q, kv_cache=kv_cache, indices=indices, workspace=workspace, out=out, lse=lse, topk_length=tl,
            attn_sink=sink)
    _lib.check("mla_sparse_decode_fwd", lib.mla_sparse_decode_fwd(
        ctypes.byref(problem), _ptr(q), _ptr(kv_cache), _ptr(indices), _ptr(tl), _ptr(sink), ctypes.byref(meta),
        _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def sparse_prefill_fwd(problem, s_kv, q, kv, indices, meta, workspace, out, lse, stream=None, topk_length=None,
                       attn_sink=None):
    """Top-k sparse prefill over a flat cache of s_kv rows (mla_sparse_prefill_fwd); ``problem`` has batch 1."""
    lib = _lib.load()
    _check_q_out(problem, q, out, lse)
    _check_kv(problem, kv, int(s_kv), "kv")
    _check_table(problem, indices, None)
    _need(workspace, "workspace", None)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
    _on_gpu(q=q, kv=kv, indices=indices, workspace=workspace, out=out, lse=lse, topk_length=tl, attn_sink=sink)
    _lib.check("mla_sparse_prefill_fwd", lib.mla_sparse_prefill_fwd(
        ctypes.byref(problem), int(s_kv), _ptr(q), _ptr(kv), _ptr(indices), _ptr(tl), _ptr(sink),
        ctypes.byref(meta), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _stream(stream)))


def sparse_prefill(q, kv, indices, sm_scale=None, topk_length=None, attn_sink=None, out_dtype="bf16", num_cus=0,
                   rescale_threshold=0.0, stream=None):
    """DSA sparse prefill in the README's argument order: q [s_q, h_q, 576], kv [s_kv, 1, 576] bfloat16 (or
    [s_kv, 1, 656] FP8 records), indices [s_q, 1, topk] -> (out [s_q, h_q, 512], lse [h_q, s_q]).  Plans,
    schedules and allocates the outputs and workspace with torch on q's device, then runs the library."""
    s_q, h_q = int(q.shape[0]), int(q.shape[1])
    s_kv, topk = int(kv.shape[0]), int(indices.shape[-1])
    if kv.dtype == torch.bfloat16:
        fmt = "bf16"
    elif kv.dtype == torch.uint8 and int(kv.shape[-1]) in (656, 528, 288):
        fmt = {656: "fp8", 528: "fp8_528", 288: "fp4_288"}[int(kv.shape[-1])]
    else:
        raise ValueError(f"kv must be bfloat16 [s_kv, 1, 576] or uint8 records of 656, 528 or 288 bytes, got "
                         f"{kv.dtype} {tuple(kv.shape)}")
    p = make_problem(1, s_q, h_q, (s_kv + 63) // 64, topk=topk, kv_format=fmt, out_dtype=out_dtype,
                     softmax_scale=sm_scale, rescale_threshold=rescale_threshold)
    m = plan(p, num_cus)
    dev = q.device
    meta_buf = torch.zeros((m.bytes + 15) // 16 * 4, dtype=torch.int32, device=dev)
    ws = torch.empty(max(16, (workspace_bytes(m) + 15) // 16 * 4), dtype=torch.float32, device=dev)
    out = torch.empty((s_q, h_q, 512), dtype=torch.float32 if out_dtype == "fp32" else torch.bfloat16, device=dev)
    lse = torch.empty((h_q, s_q), dtype=torch.float32, device=dev)
    get_decode_metadata(p, None, m, meta_buf, stream, topk_length)
    sparse_prefill_fwd(p, s_kv, q, kv, indices, m, ws, out, lse, stream, topk_length, attn_sink)
    return out, lse


def combine(num_items, h_q, s_q, o_part, lse_part, split_offsets, out, lse, stream=None, attn_sink=None):
    """Standalone LSE merge of split partials (mla_combine)."""
    lib = _lib.load()
    n, H = int(num_items), int(h_q)
    if out is None or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be a bfloat16 or float32 tensor")
    _need(lse_part, "lse_part", torch.float32)
    _need(o_part, "o_part", torch.float32, lse_part.numel() * 512)
    if lse_part.numel() % max(H, 1):
        raise ValueError(f"lse_part must hold whole [h_q] rows, got {lse_part.numel()} elements")
    _need(split_offsets, "split_offsets", torch.int32, n + 1)
    _need(out, "out", out.dtype, n * H * 512, 512)
    _need(lse, "lse", torch.float32, n * H)
    od = {torch.bfloat16: _lib.OUT_BF16, torch.float32: _lib.OUT_FP32}[out.dtype]
    sink = _attn_sink(int(h_q), attn_sink)
    _on_gpu(o_part=o_part, lse_part=lse_part, split_offsets=split_offsets, out=out, lse=lse, attn_sink=sink)
    _lib.check("mla_combine", lib.mla_combine(int(num_items), int(h_q), int(s_q), _ptr(o_part), _ptr(lse_part),
                                              _ptr(split_offsets), _ptr(sink), od, _ptr(out), _ptr(lse),
                                              _stream(stream)))


def debug_gather_rows(problem, table_or_indices, cache_seqlens, rows_out, stream=None, topk_length=None):
    lib = _lib.load()
    _check_table(problem, table_or_indices, cache_seqlens)
    stride = 64 * ((problem.topk + 63) // 64) if problem.topk > 0 else 64 * problem.max_blocks_per_seq
    _need(rows_out, "rows_out", torch.int32, problem.batch * problem.s_q * stride)
    tl = _topk_length(problem, topk_length)
    _on_gpu(table_or_indices=table_or_indices, cache_seqlens=None if problem.topk > 0 else cache_seqlens,
            rows_out=rows_out, topk_length=tl)
    _lib.check("mla_debug_gather_rows", lib.mla_debug_gather_rows(
        ctypes.byref(problem), _ptr(table_or_indices), _ptr(cache_seqlens), _ptr(tl), _ptr(rows_out),
        _stream(stream)))


def debug_decode_partial(problem, q, kv_cache, table_or_indices, cache_seqlens, meta, workspace, out, lse,
                         stream=None, topk_length=None, attn_sink=None, production=False):
    """Test hook: the partial-attention kernel alone (mla_debug_decode_partial).  ``production``: False or 0
    for mla_combine's float32 partials, True or 1 for the decode call's own format (the launch mla_decode_fwd
    makes), 2 for the launch mla_decode_step makes (the schedule computed in the kernel where it does that)."""
    fmt = int(production)
    if fmt not in (0, 1, 2):
        raise ValueError("production must be 0, 1 or 2")
    lib = _lib.load()
    _check_q_out(problem, q, out, lse)
    _check_kv(problem, kv_cache, problem.num_blocks * 64)
    _check_table(problem, table_or_indices, cache_seqlens)
    _need(workspace, "workspace", None)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
    _on_gpu(q=q, kv_cache=kv_cache, table_or_indices=table_or_indices,
            cache_seqlens=None if problem.topk > 0 else cache_seqlens, workspace=workspace, out=out, lse=lse,
            topk_length=tl, attn_sink=sink)
    _lib.check("mla_debug_decode_partial", lib.mla_debug_decode_partial(
        ctypes.byref(problem), _ptr(q), _ptr(kv_cache), _ptr(table_or_indices), _ptr(cache_seqlens), _ptr(tl),
        _ptr(sink), ctypes.byref(meta), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        fmt, _stream(stream)))


def decode_step(problem, q, kv_cache, table_or_indices, meta, meta_buf, workspace, out, lse, cache_seqlens=None,
                topk_length=None, attn_sink=None, stream=None):
    """A whole decode step in one call (mla_decode_step): the schedule for the current lengths, written to
    ``meta_buf`` as the metadata call would, then the decode.  Problems with batch * s_q <= 256 (every cache
    format) compute the schedule inside the partial-attention kernel."""
    lib = _lib.load()
    _check_q_out(problem, q, out, lse)
    _check_kv(problem, kv_cache, problem.num_blocks * 64)
    _check_table(problem, table_or_indices, cache_seqlens)
    _need(meta_buf, "meta_buf", None)
    if meta_buf.numel() * meta_buf.element_size() < meta.bytes:
        raise ValueError("meta_buf too small")
    _need(workspace, "workspace", None)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
    dense_len = None if problem.topk > 0 else cache_seqlens
    _on_gpu(q=q, kv_cache=kv_cache, table_or_indices=table_or_indices, cache_seqlens=dense_len, meta_buf=meta_buf,
            workspace=workspace, out=out, lse=lse, topk_length=tl, attn_sink=sink)
    meta.dev = meta_buf.data_ptr()
    _lib.check("mla_decode_step", lib.mla_decode_step(
        ctypes.byref(problem), _ptr(q), _ptr(kv_cache), _ptr(table_or_indices), _ptr(dense_len), _ptr(tl),
        _ptr(sink), ctypes.byref(meta), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _ptr(lse), _stream(stream)))


def decode_step_noalloc(problem, q, kv_cache, table_or_indices, out, lse, cache_seqlens=None, topk_length=None,
                        attn_sink=None, num_cus=0, stream=None):
    """A whole decode step (plan, scheduler, decode, combine) in the library's own device scratch
    (mla_decode_step_noalloc): no metadata buffer or workspace; calls that overlap on one device race."""
    lib = _lib.load()
    _check_q_out(problem, q, out, lse)
    _check_kv(problem, kv_cache, problem.num_blocks * 64)
    _check_table(problem, table_or_indices, cache_seqlens)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
    dense_len = None if problem.topk > 0 else cache_seqlens
    _on_gpu(q=q, kv_cache=kv_cache, table_or_indices=table_or_indices, cache_seqlens=dense_len, out=out, lse=lse,
            topk_length=tl, attn_sink=sink)
    _lib.check("mla_decode_step_noalloc", lib.mla_decode_step_noalloc(
        ctypes.byref(problem), int(num_cus), _ptr(q), _ptr(kv_cache), _ptr(table_or_indices), _ptr(dense_len),
        _ptr(tl), _ptr(sink), _ptr(out), _ptr(lse), _stream(stream)))


def check_inputs(problem, meta=None, meta_words=None, cache_seqlens=None, table_or_indices=None, topk_length=None,
                 num_rows=0):
    """Host-side check of a decode call's arrays (mla_check_inputs): numpy or CPU-tensor int32 arrays, each
    optional as in the C call.  Returns None when they pass; raises MlaError with the first offending entry."""
    import numpy as np
    lib = _lib.load()
    keep = []

    def host(a, name):
        if a is None:
            return None
        a = np.ascontiguousarray(a.cpu().numpy() if isinstance(a, torch.Tensor) else a)
        if a.dtype != np.int32:
            raise ValueError(f"{name} must be int32, got {a.dtype}")
        keep.append(a)
        return ctypes.c_void_p(a.ctypes.data)

    msg = ctypes.create_string_buffer(256)
    st = lib.mla_check_inputs(ctypes.byref(problem), ctypes.byref(meta) if meta is not None else None,
                              host(meta_words, "meta_words"), host(cache_seqlens, "cache_seqlens"),
                              host(table_or_indices, "table_or_indices"), host(topk_length, "topk_length"),
                              int(num_rows), msg, len(msg))
    if st != _lib.MLA_OK:
        raise MlaError("mla_check_inputs", st, msg.value.decode() or lib.mla_status_string(st).decode())


class Decoder:
    """Owns the per-shape plan, metadata buffer, workspace and outputs for one
    decode problem; ``step()`` runs the whole hot path (metadata + decode)."""

    def __init__(self, problem, device="cuda", num_cus=0):
        self.problem = problem
        self.meta = plan(problem, num_cus)
        dev = torch.device(device)
        self.meta_buf = torch.zeros((self.meta.bytes + 15) // 16 * 4, dtype=torch.int32, device=dev)
        self.workspace = torch.empty(max(16, (workspace_bytes(self.meta) + 15) // 16 * 4), dtype=torch.float32,
                                     device=dev)
        B, S, H = problem.batch, problem.s_q, problem.h_q
        odt = torch.float32 if problem.out_dtype == _lib.OUT_FP32 else torch.bfloat16
        self.out = torch.empty((B, S, H, 512), dtype=odt, device=dev)
        self.lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)

    def metadata(self, cache_seqlens=None, stream=None, topk_length=None):
        get_decode_metadata(self.problem, cache_seqlens, self.meta, self.meta_buf, stream, topk_length)

    def decode_partial(self, q, kv_cache, block_table=None, cache_seqlens=None, indices=None, stream=None,
                       topk_length=None, attn_sink=None, production=False, fused=False):
        """The partial-attention kernel alone (test and measurement hook); ``production`` keeps the decode
        call's own partial format, ``fused`` (with production) makes the launch ``step`` makes."""
        toi = indices if self.problem.topk > 0 else block_table
        fmt = (2 if fused else 1) if production else 0
        debug_decode_partial(self.problem, q, kv_cache, toi, cache_seqlens, self.meta, self.workspace, self.out,
                             self.lse, stream, topk_length, attn_sink, fmt)

    def decode(self, q, kv_cache, block_table=None, cache_seqlens=None, indices=None, stream=None,
               topk_length=None, attn_sink=None):
        if self.problem.topk > 0:
            sparse_decode_fwd(self.problem, q, kv_cache, indices, self.meta, self.workspace, self.out, self.lse,
                              stream, topk_length, attn_sink)
        else:
            decode_fwd(self.problem, q, kv_cache, block_table, cache_seqlens, self.meta, self.workspace, self.out,
                       self.lse, stream, attn_sink)
        return self.out, self.lse

    def step(self, q, kv_cache, block_table=None, cache_seqlens=None, indices=None, stream=None,
             topk_length=None, attn_sink=None):
        """Schedule and decode in one call (mla_decode_step); leaves the schedule in ``meta_buf`` for later
        ``decode`` calls with the same lengths."""
        toi = indices if self.problem.topk > 0 else block_table
        decode_step(self.problem, q, kv_cache, toi, self.meta, self.meta_buf, self.workspace, self.out, self.lse,
                    cache_seqlens, topk_length, attn_sink, stream)
        return self.out, self.lse

    def capture(self, q, kv_cache, block_table=None, cache_seqlens=None, indices=None, topk_length=None,
                attn_sink=None):
        """Record one whole step (scheduler, decode kernel, combine) into a HIP graph and return it;
        ``graph.replay()`` reruns the step on the same tensors with a single launch from the host.
        The step records no memset node; the tensors must stay allocated while the graph is used."""
        side = torch.cuda.Stream(device=self.out.device)
        side.wait_stream(torch.cuda.current_stream(self.out.device))
        with torch.cuda.stream(side):          # warm the launch path outside the capture
            self.step(q, kv_cache, block_table, cache_seqlens, indices, side, topk_length, attn_sink)
        torch.cuda.current_stream(self.out.device).wait_stream(side)
        torch.cuda.synchronize(self.out.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(q, kv_cache, block_table, cache_seqlens, indices, None, topk_length, attn_sink)
        return g

    @classmethod
    def for_workload(cls, w, device="cuda", num_cus=0, rescale_threshold=0.0):
        p = make_problem(w.batch, w.s_q, w.h_q, w.num_blocks, w.max_blocks_per_seq, topk=w.topk, causal=w.causal,
                         kv_format=w.kv_format, out_dtype=w.out_dtype, softmax_scale=w.softmax_scale,
                         rescale_threshold=rescale_threshold)
        return cls(p, device, num_cus)

    def run_workload(self, w, stream=None):
        return self.step(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, stream,
                         getattr(w, "topk_length", None), getattr(w, "attn_sink", None))
