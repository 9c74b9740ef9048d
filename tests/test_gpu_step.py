"""The one-call decode step (mla_decode_step).  For problems of up to 256
query tokens (every cache format) the schedule is computed inside the
partial-attention kernel; the metadata buffer it leaves must hold word for
word what the scheduler kernel writes for the same lengths, and out/lse must
equal, bit for bit, those of the metadata call followed by the decode call.
The cases cover one, two and four items per lane of the in-kernel scan, empty
and one-token requests, partitions spanning many short requests, three head
blocks, sparse calls with and without per-token top-k lengths and with FP8 and
FP4 records, the FP8 dense cache (causal, ragged) and batches past the fused
limit (scheduler kernel first)."""

import numpy as np
import pytest
import torch

from workloads import make_dense, make_sparse, make_fp8_dense, make_fp4_sparse

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _lens(n, lo, hi, seed):
    r = np.random.default_rng(seed)
    return [int(x) for x in r.integers(lo, hi + 1, size=n)]


CASES = {
    "b2_h16": lambda: make_dense(2, 1, 16, [200, 256], seed=1, device=DEV),
    "b64_equal": lambda: make_dense(64, 1, 128, [1024] * 64, seed=2, device=DEV),
    "b65_varlen_with_empty": lambda: make_dense(65, 1, 128, [0, 1] + _lens(63, 0, 900, 3), seed=3, device=DEV),
    "b100_s2_causal": lambda: make_dense(100, 2, 128, _lens(100, 1, 700, 4), causal=True, seed=4, device=DEV),
    "b128_s2_causal": lambda: make_dense(128, 2, 128, _lens(128, 64, 600, 5), causal=True, seed=5, device=DEV),
    "b200_short": lambda: make_dense(200, 1, 64, _lens(200, 0, 130, 6), seed=6, device=DEV),
    "b3_h192_causal": lambda: make_dense(3, 2, 192, [1, 300, 777], causal=True, seed=7, device=DEV),
    "b300_not_fused": lambda: make_dense(300, 1, 32, _lens(300, 1, 200, 8), seed=8, device=DEV),
    "sparse_b64": lambda: make_sparse(64, 1, 128, pool_tokens_per_seq=512, topk=200, invalid_frac=0.05, seed=10,
                                      device=DEV),
    "sparse_b128_s2_fp8": lambda: make_sparse(128, 2, 64, pool_tokens_per_seq=256, topk=128, seed=11, device=DEV,
                                              kv_format="fp8"),
    "sparse_b3_fp4": lambda: make_fp4_sparse(3, 2, 128, pool_tokens_per_seq=1024, topk=333, invalid_frac=0.1,
                                             seed=12, device=DEV),
    "sparse_b150_not_fused": lambda: make_sparse(150, 2, 16, pool_tokens_per_seq=128, topk=64, seed=13,
                                                 device=DEV),
    "fp8_dense_b4": lambda: make_fp8_dense(4, 1, 128, [1, 500, 1000, 64], seed=14, device=DEV),
    "fp8_dense_b70_s2_causal": lambda: make_fp8_dense(70, 2, 128, _lens(70, 1, 900, 17), causal=True, seed=17,
                                                      device=DEV),
    "fp8_dense_b300_not_fused": lambda: make_fp8_dense(300, 1, 16, _lens(300, 1, 200, 18), seed=18, device=DEV),
}


def _with_topk_length(w, seed):
    """A copy of sparse workload w with per-token top-k lengths in [0, topk], some 0."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    tl = torch.randint(0, w.topk + 1, (w.batch, w.s_q), generator=g, dtype=torch.int32)
    tl.view(-1)[::7] = 0
    w.topk_length = tl.to(DEV)
    return w


CASES["sparse_b64_topk_length"] = lambda: _with_topk_length(
    make_sparse(64, 2, 128, pool_tokens_per_seq=512, topk=300, seed=15, device=DEV), 16)


@pytest.mark.parametrize("name", list(CASES))
def test_step_matches_metadata_then_decode(name):
    import mla_decode_amd as mla
    print(f"decode step: {name}", flush=True)
    w = CASES[name]()
    dec = mla.Decoder.for_workload(w, DEV)
    words = dec.meta.bytes // 4
    tl = getattr(w, "topk_length", None)
    sl = None if w.topk else w.cache_seqlens
    dec.metadata(sl, topk_length=tl)
    ref_meta = dec.meta_buf.view(torch.int32)[:words].clone()
    o1, l1 = dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, topk_length=tl)
    o1, l1 = o1.clone(), l1.clone()
    dec.meta_buf.fill_(-7)
    dec.out.fill_(float("nan"))
    dec.lse.fill_(float("nan"))
    o2, l2 = dec.step(w.q, w.kv, w.block_table, sl, w.indices, topk_length=tl)
    torch.cuda.synchronize()
    got_meta = dec.meta_buf.view(torch.int32)[:words]
    assert torch.equal(got_meta, ref_meta), (got_meta - ref_meta).nonzero()[:8].tolist()
    assert torch.equal(o1.view(torch.int16 if o1.dtype == torch.bfloat16 else torch.int32),
                       o2.view(torch.int16 if o2.dtype == torch.bfloat16 else torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    # the schedule left behind serves a later decode call with the same lengths
    o3, l3 = dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, topk_length=tl)
    assert torch.equal(o1, o3) and torch.equal(l1.view(torch.int32), l3.view(torch.int32))


def test_step_follows_new_lengths():
    import mla_decode_amd as mla
    print("decode step: lengths change between calls", flush=True)
    w = make_dense(64, 1, 128, _lens(64, 100, 2000, 9), seed=9, device=DEV, max_blocks=40)
    dec = mla.Decoder.for_workload(w, DEV)
    dec.step(w.q, w.kv, w.block_table, w.cache_seqlens)
    shorter = (w.cache_seqlens // 2).contiguous()
    o2, l2 = dec.step(w.q, w.kv, w.block_table, shorter)
    o2, l2 = o2.clone(), l2.clone()
    m2 = dec.meta_buf.clone()
    dec.metadata(shorter)
    assert torch.equal(dec.meta_buf, m2)
    o3, l3 = dec.decode(w.q, w.kv, w.block_table, shorter)
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
