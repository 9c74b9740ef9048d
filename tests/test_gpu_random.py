"""Seeded random problems through both call patterns, on every cache format.

Each case draws a cache format (dense bf16, dense FP8, sparse bf16, sparse
FP8, the 528- and 288-byte records), a batch, s_q, a head count (including
counts that are not a multiple of 32 and two head blocks), cache lengths or
top-k sizes mixed with the edge values 0, 1, 63, 64, 65 and 128, causal
masking, the output type, an attention sink and per-query top-k lengths.  The
one-call step (schedule in the kernel where the batch allows it) and the
metadata call followed by the decode call must give the same outputs bit for
bit, and both must match the fp64 oracle within the tolerances the other
parity tests use."""

import numpy as np
import pytest
import torch

from workloads import make_dense, make_sparse, make_fp8_dense, make_v41_sparse, make_fp4_sparse
from helpers import oracle, compare, FP8_REL_L2

pytestmark = pytest.mark.gpu

DEV = "cuda"
KINDS = ("dense", "fp8", "sparse", "sparse_fp8", "v41", "fp4")
EDGE = (0, 1, 63, 64, 65, 128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _draw(seed):
    """The case of ``seed``: (workload, description)."""
    r = np.random.default_rng(5000 + seed)
    kind = KINDS[seed % len(KINDS)]
    B = int(r.integers(1, 25))
    S = int(r.choice([1, 1, 2, 3]))
    H = int(r.choice([16, 40, 64, 100, 128, 192]))
    out_dtype = str(r.choice(["bf16", "fp32"]))
    if kind in ("dense", "fp8"):
        lens = [int(x) if r.random() < 0.7 else int(r.choice(EDGE)) for x in r.integers(0, 1201, size=B)]
        causal = bool(S > 1 and r.random() < 0.7)
        make = make_dense if kind == "dense" else make_fp8_dense
        w = make(B, S, H, lens, causal=causal, seed=seed, device=DEV, out_dtype=out_dtype)
        desc = f"{kind} B={B} S={S} H={H} out={out_dtype} causal={causal} lens={lens[:6]}"
    else:
        pool = int(r.choice([256, 512, 1024]))
        topk = int(r.choice(EDGE[1:]) if r.random() < 0.3 else r.integers(1, min(pool, 700) + 1))
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


def _run(w, num_cus, step):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV, num_cus)
    tl, sink = getattr(w, "topk_length", None), getattr(w, "attn_sink", None)
    if step:
        out, lse = dec.step(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, None, tl, sink)
    else:
        dec.metadata(None if w.topk else w.cache_seqlens, None, tl)
        out, lse = dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, None, tl, sink)
    torch.cuda.synchronize()
    return out.clone(), lse.clone()


@pytest.mark.parametrize("seed", range(64))
def test_random_problem(seed):
    kind, w, desc = _draw(seed)
    print(desc, flush=True)
    num_cus = (0, 7, 64)[seed % 3]
    so, sl = _run(w, num_cus, step=True)
    do, dl = _run(w, num_cus, step=False)
    as_bits = torch.int16 if so.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(so.view(as_bits), do.view(as_bits)), "step and metadata + decode outputs differ"
    assert torch.equal(sl.view(torch.int32), dl.view(torch.int32)), "step and metadata + decode lse differ"
    kv = w.kv.cpu().numpy().reshape(-1, int(w.kv.shape[-1])) if kind in ("v41", "fp4") else None
    ro, rl = oracle(w, kv=kv)
    kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kind in ("fp8", "sparse_fp8") else {}
    go = so.float().cpu().numpy().astype(np.float64)
    gl = sl.cpu().numpy().astype(np.float64)
    print(compare(go, gl, ro, rl, **kw), flush=True)
