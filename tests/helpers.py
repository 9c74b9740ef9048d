"""Shared helpers for the GPU parity tests: run the library through its C ABI
on a workload, run the fp64 oracle on the same inputs, compare."""

import numpy as np
import torch

from oracle import attention as A

OUT_REL_L2 = 3e-3      # bf16 output vs fp64, ~1.8x the bf16 rounding floor
OUT_MAX_ABS = 1e-2
# Element bound: OUT_MAX_ABS plus 2^-7 |ref|.  The second term is the bf16
# output half-ulp (2^-8 |ref|) plus a coherent bf16 rounding of P (2^-9) with
# margin; it only matters for rows over a handful of tokens, whose outputs
# approach single V rows of magnitude > 2, where a fixed 1e-2 is below bf16's
# own resolution.  For the long rows of the five workloads it is 1e-2.
MAX_ABS_REL = 2.0 ** -7
LSE_ABS = 1e-3
FP8_REL_L2 = 2e-2


def bits16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def kv_host(w):
    if w.kv_format == 'bf16':
        return bits16(w.kv).reshape(-1, 576)
    return w.kv.detach().contiguous().cpu().numpy().reshape(-1, int(w.kv.shape[-1]))


def kv_host_rows(w, items):
    """Host copy of the cache holding only the rows the sampled top-k query
    tokens gather (the rest stay zero pages of a lazily allocated array), so
    that multi-GB caches need not be copied whole."""
    rows_dev = w.kv.view(-1, w.kv.shape[-1])
    nrows = rows_dev.shape[0]
    idx = w.indices.cpu().numpy()
    need = np.unique(np.concatenate([idx[b, i][(idx[b, i] >= 0) & (idx[b, i] < nrows)] for b, i in items]))
    raw = w.kv_format != 'bf16'                # byte records; bf16 rows otherwise
    host = np.zeros((nrows, rows_dev.shape[1]), dtype=np.uint8 if raw else np.uint16)
    sel = torch.from_numpy(need.astype(np.int64)).to(w.kv.device)
    got = rows_dev[sel].cpu()
    host[need] = got.numpy() if raw else got.view(torch.int16).numpy().view(np.uint16)
    return host


def run_library(w, num_cus=0, stream=None, rescale_threshold=0.0):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, w.q.device, num_cus, rescale_threshold=rescale_threshold)
    out, lse = dec.run_workload(w, stream)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), dec


def oracle(w, items=None, kv=None):
    q = bits16(w.q)
    kv = kv_host(w) if kv is None else kv
    sink = None if getattr(w, "attn_sink", None) is None else w.attn_sink.cpu().double().numpy()
    if w.topk:
        tl = None if getattr(w, "topk_length", None) is None else w.topk_length.cpu().numpy()
        return A.decode(q, kv, w.softmax_scale, indices=w.indices.cpu().numpy(), kv_format=w.kv_format, items=items,
                        topk_length=tl, attn_sink=sink)
    return A.decode(q, kv, w.softmax_scale, block_table=w.block_table.cpu().numpy(),
                    cache_seqlens=w.cache_seqlens.cpu().numpy(), causal=w.causal, kv_format=w.kv_format,
                    items=items, attn_sink=sink)


def compare(got_out, got_lse, ref_out, ref_lse, items=None, rel_l2=OUT_REL_L2, max_abs=OUT_MAX_ABS, lse_abs=LSE_ABS,
            max_abs_rel=MAX_ABS_REL):
    """Element-wise comparison on the selected items (default all); returns stats.

    Every element satisfies |got - ref| <= max_abs + max_abs_rel * |ref|;
    ``max_abs_rel=0`` makes it the literal max-abs bound (the full-size
    workloads, whose outputs stay below 2 in magnitude, use that)."""
    B, S = ref_out.shape[:2]
    if items is None:
        items = [(b, i) for b in range(B) for i in range(S)]
    go = np.stack([got_out[b, i] for b, i in items])
    ro = np.stack([ref_out[b, i] for b, i in items])
    gl = np.stack([got_lse[b, :, i] for b, i in items])
    rl = np.stack([ref_lse[b, :, i] for b, i in items])
    assert np.all(np.isfinite(go)), "non-finite output"
    nrm = np.linalg.norm(ro)
    rel = np.linalg.norm(go - ro) / nrm if nrm > 0 else np.linalg.norm(go)
    mab = float(np.max(np.abs(go - ro))) if go.size else 0.0
    excess = float(np.max(np.abs(go - ro) - max_abs_rel * np.abs(ro))) if go.size else 0.0
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), "-inf lse positions differ"
    lerr = float(np.max(np.abs(gl[fin] - rl[fin]))) if fin.any() else 0.0
    stats = {'rel_l2': float(rel), 'max_abs': mab, 'max_abs_over_rel': excess, 'lse_abs': lerr}
    assert rel <= rel_l2, stats
    assert excess <= max_abs, stats
    assert lerr <= lse_abs, stats
    # rows that see nothing are exactly zero
    empty = np.isneginf(rl)
    if empty.any():
        assert np.all(go[empty] == 0.0)
    return stats


RANDOM_KINDS = ("dense", "fp8", "sparse", "sparse_fp8", "v41", "fp4")
RANDOM_EDGE = (0, 1, 63, 64, 65, 128)


def draw_random_problem(seed, device):
    """A seeded random decode problem: (cache format, workload, description).
    The format cycles over RANDOM_KINDS; batch, s_q, heads, lengths or top-k
    sizes (mixed with the edge values 0, 1, 63, 64, 65, 128), causal masking,
    output type, sink and per-query top-k lengths are drawn."""
    from workloads import make_dense, make_sparse, make_fp8_dense, make_v41_sparse, make_fp4_sparse
    DEV = device
    r = np.random.default_rng(5000 + seed)
    kind = RANDOM_KINDS[seed % len(RANDOM_KINDS)]
    B = int(r.integers(1, 25))
    S = int(r.choice([1, 1, 2, 3]))
    H = int(r.choice([16, 40, 64, 100, 128, 192]))
    out_dtype = str(r.choice(["bf16", "fp32"]))
    if kind in ("dense", "fp8"):
        lens = [int(x) if r.random() < 0.7 else int(r.choice(RANDOM_EDGE)) for x in r.integers(0, 1201, size=B)]
        causal = bool(S > 1 and r.random() < 0.7)
        make = make_dense if kind == "dense" else make_fp8_dense
        w = make(B, S, H, lens, causal=causal, seed=seed, device=DEV, out_dtype=out_dtype)
        desc = f"{kind} B={B} S={S} H={H} out={out_dtype} causal={causal} lens={lens[:6]}"
    else:
        pool = int(r.choice([256, 512, 1024]))
        topk = int(r.choice(RANDOM_EDGE[1:]) if r.random() < 0.3 else r.integers(1, min(pool, 700) + 1))
        inv = float(r.choice([0.0, 0.05, 0.2]))
        if kind in ("sparse", "sparse_fp8"):
            w = make_sparse(B, S, H, pool_tokens_per_seq=pool, topk=topk, invalid_frac=inv, seed=seed, device=DEV,
                            out_dtype=out_dtype, kv_format="fp8" if kind == "sparse_fp8" else "bf16")
        else:
            make = make_v41_sparse if kind == "v41" else make_fp4_sparse
            w = make(B, S, H, pool_tokens_per_seq=pool, topk=topk, invalid_frac=inv, seed=seed, device=DEV)
            w.out_dtype = out_dtype
        if r.random() < 0.4:
            tl = torch.as_tensor(r.integers(0, topk + 1, size=(B, S)), dtype=torch.int32)
            w.topk_length = tl.to(DEV)
        desc = f"{kind} B={B} S={S} H={H} out={out_dtype} pool={pool} topk={topk} invalid={inv}"
    if r.random() < 0.3:
        s = torch.as_tensor(r.normal(8.0, 4.0, size=H), dtype=torch.float32)
        s[0] = -float("inf")
        w.attn_sink = s.to(DEV)
        desc += " sink"
    return kind, w, desc
