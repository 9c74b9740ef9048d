"""Algorithmic FLOP and byte counts for absorbed-MLA decode.

Counting rules (FlashMLA new-kernel deep dive, "Theoretical analysis"; MLA
cost-analysis page, "FlashMLA" cost model):
* FLOPs = 2 * h_q * (d_k + d_v) per (query token, visible KV token) pair,
  d_k = 576 (512 for the 528-byte records), d_v = 512; top-k decode counts
  valid slots only;
* bytes = every KV row a request needs, read once (1152 B bf16, 656 B or
  528 B FP8), plus q (d_k bf16 per head), out (512 per head, 2 or 4 B), lse
  (4 B per head), and the block table or top-k indices (4 B each).
Split partials and scheduler metadata are implementation overhead and are not
counted here.  ``partial_bytes`` (KV rows, q, table or indices) is what the
partial-attention kernel alone must move; the outputs of split items are
written by the combine.
"""

import math

import torch

D_QK = 576
D_V = 512
BLOCK = 64


def visible(L, s_q, i, causal):
    if not causal:
        return L
    return min(max(L - s_q + 1 + i, 0), L)


def flops_and_bytes(w):
    """Algorithmic FLOPs and HBM bytes of one decode call on workload ``w``."""
    B, S, H = w.batch, w.s_q, w.h_q
    row_bytes = {'bf16': 1152, 'fp8': 656, 'fp8_528': 528, 'fp4_288': 288}[w.kv_format]
    d_qk = 512 if w.kv_format in ('fp8_528', 'fp4_288') else D_QK
    out_elem = 2 if w.out_dtype == 'bf16' else 4
    if w.topk:
        idx = w.indices.to('cpu').to(torch.int64)
        nrows = w.num_blocks * BLOCK
        valid = ((idx >= 0) & (idx < nrows))
        pairs = int(valid.sum())
        kv_rows = 0
        for b in range(B):
            kv_rows += int(torch.unique(idx[b][valid[b]]).numel())
        side = idx.numel() * 4
    else:
        lens = [int(x) for x in w.cache_seqlens.to('cpu').tolist()]
        pairs = sum(visible(L, S, i, w.causal) for L in lens for i in range(S))
        kv_rows = sum(lens)
        side = sum(math.ceil(L / BLOCK) for L in lens) * 4
    flops = 2.0 * H * (d_qk + D_V) * pairs
    kv_bytes = kv_rows * row_bytes
    q_bytes = B * S * H * d_qk * 2
    out_bytes = B * S * H * D_V * out_elem + B * S * H * 4
    total = kv_bytes + q_bytes + out_bytes + side
    return {'flops': flops, 'bytes': float(total), 'kv_bytes': float(kv_bytes),
            'partial_bytes': float(kv_bytes + q_bytes + side), 'pairs': pairs, 'kv_rows': kv_rows}


def cost_model_flashmla(b, h, s, t, k=512, p=64, w=2):
    """FLOPs and bytes of the latent-space cost model: 2bhst(2k+p) FLOPs,
    w*(bhs(2k+p) + bt(k+p)) bytes."""
    flops = 2 * b * h * s * t * (2 * k + p)
    byts = w * (b * h * s * (2 * k + p) + b * t * (k + p))
    return flops, byts


def mma_cycles_per_token(heads, flop_per_clk, d_k=D_QK, d_v=D_V):
    """MMA cycles one compute unit spends per KV token for ``heads`` heads."""
    return heads * (d_k + d_v) * 2 / flop_per_clk


def h800_dequant_cycles_per_token(n=512):
    """Per-token dequant cycles on H800 from the four listed conversion rates:
    e4m3->half, half->float, float->bf16 at 1/64, 1/64, 1/16 cycle per value
    and the scale multiply at 1/256."""
    return (1 / 64 + 1 / 64 + 1 / 16 + 1 / 256) * n
