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
           "MlaError", "abi_version"]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


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
    _need(t, name, dtype)
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t


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
    elif cache_seqlens is not None:
        _need(cache_seqlens, "cache_seqlens", torch.int32)
    tl = _topk_length(problem, topk_length)
    meta.dev = meta_buf.data_ptr()
    _lib.check("mla_get_decode_metadata", lib.mla_get_decode_metadata(
        ctypes.byref(problem), _ptr(cache_seqlens), _ptr(tl), ctypes.byref(meta), _stream(stream)))
    return meta


def decode_fwd(problem, q, kv_cache, block_table, cache_seqlens, meta, workspace, out, lse, stream=None,
               attn_sink=None):
    """Dense paged decode (mla_decode_fwd)."""
    lib = _lib.load()
    _need(q, "q", torch.bfloat16)
    _need(kv_cache, "kv_cache", None)
    _need(block_table, "block_table", torch.int32)
    _need(cache_seqlens, "cache_seqlens", torch.int32)
    _need(workspace, "workspace", None)
    _need(out, "out", None)
    _need(lse, "lse", torch.float32)
    sink = _attn_sink(problem.h_q, attn_sink)
    _lib.check("mla_decode_fwd", lib.mla_decode_fwd(
        ctypes.byref(problem), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), _ptr(sink),
        ctypes.byref(meta), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _stream(stream)))


def sparse_decode_fwd(problem, q, kv_cache, indices, meta, workspace, out, lse, stream=None, topk_length=None,
                      attn_sink=None):
    """Top-k sparse decode (mla_sparse_decode_fwd)."""
    lib = _lib.load()
    _need(q, "q", torch.bfloat16)
    _need(kv_cache, "kv_cache", None)
    _need(indices, "indices", torch.int32)
    _need(workspace, "workspace", None)
    _need(out, "out", None)
    _need(lse, "lse", torch.float32)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
    _lib.check("mla_sparse_decode_fwd", lib.mla_sparse_decode_fwd(
        ctypes.byref(problem), _ptr(q), _ptr(kv_cache), _ptr(indices), _ptr(tl), _ptr(sink), ctypes.byref(meta),
        _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def sparse_prefill_fwd(problem, s_kv, q, kv, indices, meta, workspace, out, lse, stream=None, topk_length=None,
                       attn_sink=None):
    """Top-k sparse prefill over a flat cache of s_kv rows (mla_sparse_prefill_fwd); ``problem`` has batch 1."""
    lib = _lib.load()
    _need(q, "q", torch.bfloat16)
    _need(kv, "kv", None)
    _need(indices, "indices", torch.int32)
    _need(workspace, "workspace", None)
    _need(out, "out", None)
    _need(lse, "lse", torch.float32)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
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
    fmt = "bf16" if kv.dtype != torch.uint8 else {528: "fp8_528", 288: "fp4_288"}.get(int(kv.shape[-1]), "fp8")
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
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    _need(split_offsets, "split_offsets", torch.int32)
    _need(out, "out", None)
    _need(lse, "lse", torch.float32)
    od = {torch.bfloat16: _lib.OUT_BF16, torch.float32: _lib.OUT_FP32}[out.dtype]
    sink = _attn_sink(int(h_q), attn_sink)
    _lib.check("mla_combine", lib.mla_combine(int(num_items), int(h_q), int(s_q), _ptr(o_part), _ptr(lse_part),
                                              _ptr(split_offsets), _ptr(sink), od, _ptr(out), _ptr(lse),
                                              _stream(stream)))


def debug_gather_rows(problem, table_or_indices, cache_seqlens, rows_out, stream=None, topk_length=None):
    lib = _lib.load()
    _need(table_or_indices, "table_or_indices", torch.int32)
    _need(rows_out, "rows_out", torch.int32)
    tl = _topk_length(problem, topk_length)
    _lib.check("mla_debug_gather_rows", lib.mla_debug_gather_rows(
        ctypes.byref(problem), _ptr(table_or_indices), _ptr(cache_seqlens), _ptr(tl), _ptr(rows_out),
        _stream(stream)))


def debug_decode_partial(problem, q, kv_cache, table_or_indices, cache_seqlens, meta, workspace, out, lse,
                         stream=None, topk_length=None, attn_sink=None, production=False):
    """Test hook: the partial-attention kernel alone (mla_debug_decode_partial).  ``production``: split
    partials in the decode call's own format (the launch a decode step makes) instead of mla_combine's."""
    lib = _lib.load()
    _need(q, "q", torch.bfloat16)
    _need(kv_cache, "kv_cache", None)
    _need(table_or_indices, "table_or_indices", torch.int32)
    _need(workspace, "workspace", None)
    _need(out, "out", None)
    _need(lse, "lse", torch.float32)
    tl, sink = _topk_length(problem, topk_length), _attn_sink(problem.h_q, attn_sink)
    _lib.check("mla_debug_decode_partial", lib.mla_debug_decode_partial(
        ctypes.byref(problem), _ptr(q), _ptr(kv_cache), _ptr(table_or_indices), _ptr(cache_seqlens), _ptr(tl),
        _ptr(sink), ctypes.byref(meta), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        1 if production else 0, _stream(stream)))


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
                       topk_length=None, attn_sink=None, production=False):
        """The partial-attention kernel alone (test and measurement hook); ``production`` keeps the decode
        call's own partial format."""
        toi = indices if self.problem.topk > 0 else block_table
        debug_decode_partial(self.problem, q, kv_cache, toi, cache_seqlens, self.meta, self.workspace, self.out,
                             self.lse, stream, topk_length, attn_sink, production)

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
        self.metadata(cache_seqlens, stream, topk_length)
        return self.decode(q, kv_cache, block_table, cache_seqlens, indices, stream, topk_length, attn_sink)

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
