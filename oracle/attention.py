"""Absorbed-MLA decode: the definition, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (sources, by page title and section):

* "Matrices, attention & GPU" explainer (juejin), section 5 "Attention: two
  GEMMs and a softmax": attention = softmax(Q K^T * scale) V, with the plain
  three-step naive form and the streaming form that keeps a running max m, a
  running sum l and a partial output acc per query.
* Same explainer, section 6 "MLA": after absorbing W^UK into the query and
  W^UV into the output projection, every head scores against the same cached
  latent c_j (512) and the shared RoPE key k_j^R (64), so decode is MQA with
  h_q query heads over one KV head of width 576; values are the 512 latent
  dims (FlashMLA new-kernel deep dive, "Theoretical analysis": d_k = 576,
  d_v = 512, K and V are the same data).
* Same explainer, section 7 "split-KV": partial results over KV segments are
  merged with m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m),
  o = (o1 l1 e^(m1-m) + o2 l2 e^(m2-m)) / l.
* FlashMLA README ("Usage", DSA decoding): paged cache with block_table and
  cache_seqlens; top-k ``indices[b, s_q, topk]`` hold page_block*block_size +
  offset, -1 marks an invalid entry and block_table is not used; the kernel
  returns out [b, s_q, h_q, d_v] and lse [b, h_q, s_q] in float32 (transposed
  with respect to out).
* Same README, sparse attention arguments: an optional per-head
  ``attn_sink`` scales the output by exp(lse) / (exp(lse) + exp(attn_sink)),
  and an optional ``topk_length`` restricts a query token to the first
  topk_length entries of its index row.

Readings where the pages are silent (each also listed in the design notes):
* scores are multiplied by ``softmax_scale``; lse is the natural-log
  log-sum-exp of the scaled scores;
* causal with s_q > 1: query token i of a request with cache length L sees the
  first L - s_q + 1 + i tokens (the cache already holds the new tokens);
* a query that sees no token gets out = 0 and lse = -inf;
* a top-k index < 0 or >= num_blocks*block_size is treated as invalid
  (the pages say only -1 is invalid and that no upper-bound check is made);
* duplicate top-k entries each count (the slot multiset);
* ``topk_length`` is given per decode query token ([b, s_q]; the README's
  prefill call gives it per query row) and clamped to [0, topk]; lse is not
  changed by the sink.

Everything is float64 on the exact values of the bfloat16 (or dequantised
FP8) inputs, so the result is the mathematical value up to float64 rounding.
"""

import math

import numpy as np

from .numerics import bf16_bits_to_f64
from .fp8cache import dequant_records, dequant_records_v41, dequant_records_fp4, RECORD_BYTES, V41_RECORD_BYTES
from .sched import visible_len

D_QK = 576
D_V = 512
BLOCK = 64


# --------------------------------------------------------------------------
# single query group: all heads of one query token against one KV row set

def attend(qh, K, V, scale):
    """Two-pass softmax attention in float64.

    qh [H, 576], K [n, 576], V [n, 512]  ->  out [H, 512], lse [H]
    """
    H = qh.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf)
    s = scale * (qh @ K.T)                       # [H, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ V) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def attend_bruteforce(q, K, V, scale):
    """Loop-only attention for one query vector (lists of floats).

    Follows the naive form: materialise every score, subtract the max,
    exponentiate, normalise, then weight the value rows.  Pure Python math.
    """
    n = len(K)
    if n == 0:
        return [0.0] * len(V[0]) if V else [], -math.inf
    s = []
    for j in range(n):
        acc = 0.0
        for t in range(len(q)):
            acc += q[t] * K[j][t]
        s.append(acc * scale)
    m = max(s)
    e = [math.exp(x - m) for x in s]
    tot = sum(e)
    out = [0.0] * len(V[0])
    for j in range(n):
        w = e[j] / tot
        for t in range(len(out)):
            out[t] += w * V[j][t]
    return out, m + math.log(tot)


def attend_online(q, K, V, scale):
    """Streaming (online-softmax) recurrence for one query vector, float64.

    Running max m, running sum l and accumulator acc, one KV row at a time:
    m_new = max(m, s); alpha = e^(m - m_new); p = e^(s - m_new);
    l = l*alpha + p; acc = acc*alpha + p*v; finally out = acc / l.
    """
    m = -np.inf
    l = 0.0
    acc = np.zeros(V.shape[1])
    for j in range(K.shape[0]):
        s = scale * float(q @ K[j])
        m_new = max(m, s)
        alpha = math.exp(m - m_new) if m != -np.inf else 0.0
        p = math.exp(s - m_new)
        l = l * alpha + p
        acc = acc * alpha + p * V[j]
        m = m_new
    if l == 0.0:
        return np.zeros(V.shape[1]), -np.inf
    return acc / l, m + math.log(l)


def merge_partials(o_parts, lse_parts):
    """Merge split partials (normalised o_k, lse_k) into (o, lse), float64.

    o_parts [n, ..., D], lse_parts [n, ...].  Each partial is written as
    (m_k, l_k) = (lse_k, 1), then folded pairwise with the split-KV merge
    formula.  A partial with lse = -inf weighs nothing; if all are -inf the
    result is o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o = np.zeros(o_parts.shape[1:])
    m = np.full(lse_parts.shape[1:], -np.inf)
    l = np.zeros(lse_parts.shape[1:])
    for k in range(o_parts.shape[0]):
        m2 = lse_parts[k]
        with np.errstate(invalid='ignore'):
            d1 = m - np.maximum(m, m2)
            d2 = m2 - np.maximum(m, m2)
        l2 = np.where(np.isneginf(m2), 0.0, 1.0)
        m_new = np.maximum(m, m2)
        safe = ~np.isneginf(m_new)
        a1 = np.where(safe, np.exp(np.where(safe, d1, 0.0)), 0.0) * l
        a2 = np.where(safe, np.exp(np.where(safe, d2, 0.0)), 0.0) * l2
        l_new = a1 + a2
        den = np.where(l_new > 0, l_new, 1.0)
        o = (o * a1[..., None] + o_parts[k] * a2[..., None]) / den[..., None]
        m, l = m_new, l_new
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    o = np.where((l > 0)[..., None], o, 0.0)
    return o, lse


# --------------------------------------------------------------------------
# cache access

def kv_values(kv, rows, kv_format):
    """Gather physical cache rows and decode them to float64 [n, 576] (or
    [n, 512] for the 528- and 288-byte records of the 512-wide head)."""
    rows = np.asarray(rows, dtype=np.int64)
    if kv_format == 'bf16':
        return bf16_bits_to_f64(kv[rows])
    if kv_format == 'fp8':
        assert kv.shape[-1] == RECORD_BYTES
        return dequant_records(kv[rows])
    if kv_format == 'fp8_528':
        assert kv.shape[-1] == V41_RECORD_BYTES
        return dequant_records_v41(kv[rows])
    if kv_format == 'fp4_288':
        return dequant_records_fp4(kv[rows])
    raise ValueError(kv_format)


def paged_rows(block_table_row, n):
    """Physical rows of logical tokens 0..n-1 through one block-table row."""
    t = np.arange(n, dtype=np.int64)
    return np.asarray(block_table_row, dtype=np.int64)[t // BLOCK] * BLOCK + t % BLOCK


def sparse_rows(index_row, num_rows, length=None):
    """Valid physical rows of one top-k index row (the slot multiset), over
    its first ``length`` entries when a top-k length is given."""
    idx = np.asarray(index_row, dtype=np.int64)
    if length is not None:
        idx = idx[:min(max(int(length), 0), idx.shape[0])]
    return idx[(idx >= 0) & (idx < num_rows)]


def apply_sink(out, lse, sink):
    """Scale one query group's rows by exp(lse) / (exp(lse) + exp(sink)) per
    head; lse unchanged.  A row that sees nothing (lse = -inf) stays 0."""
    sink = np.asarray(sink, dtype=np.float64)
    f = np.zeros_like(lse)
    ok = np.isfinite(lse)
    f[ok] = 1.0 / (1.0 + np.exp(sink[ok] - lse[ok]))
    return out * f[:, None]


def gather_rows_dense(block_table, cache_seqlens, s_q, causal):
    """Resolved rows per item (b, i): list of int64 arrays (row ids)."""
    out = []
    for b, L in enumerate(np.asarray(cache_seqlens).tolist()):
        for i in range(s_q):
            out.append(paged_rows(block_table[b], visible_len(L, s_q, i, causal)))
    return out


# --------------------------------------------------------------------------
# whole-batch decode

def decode(q_bits, kv, softmax_scale, *, block_table=None, cache_seqlens=None,
           indices=None, causal=False, kv_format='bf16', items=None, topk_length=None, attn_sink=None):
    """Absorbed-MLA decode over a batch, float64.

    q_bits   uint16 [B, S, H, 576]   bfloat16 bit patterns of the absorbed q
    kv       uint16 [R, 576] (bf16) or uint8 [R, 656] (fp8), R = num_blocks*64
    dense:   block_table int [B, max_blocks], cache_seqlens int [B]
    sparse:  indices int [B, S, topk]  (block_table unused); topk_length
             optional int [B, S]
    attn_sink optional float [H]
    items    optional list of (b, i) to compute; default all

    Returns out float64 [B, S, H, 512] and lse float64 [B, H, S]; entries not
    in ``items`` are left NaN.
    """
    q_bits = np.asarray(q_bits)
    B, S, H, D = q_bits.shape
    assert D == (512 if kv_format in ('fp8_528', 'fp4_288') else D_QK)
    num_rows = kv.shape[0]
    out = np.full((B, S, H, D_V), np.nan)
    lse = np.full((B, H, S), np.nan)
    if items is None:
        items = [(b, i) for b in range(B) for i in range(S)]
    for (b, i) in items:
        if indices is not None:
            rows = sparse_rows(indices[b, i], num_rows, None if topk_length is None else topk_length[b][i])
        else:
            L = int(cache_seqlens[b])
            rows = paged_rows(block_table[b], visible_len(L, S, i, causal))
        Kf = kv_values(kv, rows, kv_format)
        qh = bf16_bits_to_f64(q_bits[b, i])
        o, ls = attend(qh, Kf, Kf[:, :D_V], softmax_scale)
        if attn_sink is not None:
            o = apply_sink(o, ls, attn_sink)
        out[b, i] = o
        lse[b, :, i] = ls
    return out, lse


def decode_partial(q_bits, kv, softmax_scale, rows, b, i, kv_format='bf16'):
    """(out, lse) of one query group over an explicit list of physical rows."""
    Kf = kv_values(kv, rows, kv_format)
    return attend(bf16_bits_to_f64(q_bits[b, i]), Kf, Kf[:, :D_V], softmax_scale)
