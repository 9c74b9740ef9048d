"""The largest batches the library accepts: batch * s_q = 16384 query groups.

At the limit the scheduler kernel writes 16384 item entries; its metadata
must equal the oracle scheduler's word for word, the one-call step must equal
the metadata call followed by the decode call bit for bit, sampled query
groups (the first, the last, empty rows and random ones) must match the fp64
oracle, and over every query group the rows that see no key must come out
with lse -inf and an output of exact zeros while every other output is finite.
One group more is refused on the host (covered by the ABI tests)."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import sched as S
from workloads import make_dense, make_fp8_dense, make_sparse
from helpers import oracle, compare, kv_host_rows, FP8_REL_L2

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_ITEMS = 16384


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _lengths(r, B):
    lens = r.integers(0, 131, size=B)
    edge = np.array([0, 1, 63, 64, 65, 128])
    pick = r.random(B) < 0.2
    lens[pick] = r.choice(edge, size=int(pick.sum()))
    return lens.tolist()


def _make(kind):
    r = np.random.default_rng({"dense": 11, "fp8": 12, "sparse": 13}[kind])
    if kind == "dense":      # 64 heads per workgroup, two query tokens per row, causal
        B, s_q, H = MAX_ITEMS // 2, 2, 16
        return make_dense(B, s_q, H, _lengths(r, B), causal=True, seed=21, device=DEV, max_blocks=3)
    if kind == "fp8":
        B, H = MAX_ITEMS, 32
        return make_fp8_dense(B, 1, H, _lengths(r, B), seed=22, device=DEV, max_blocks=3)
    return make_sparse(MAX_ITEMS, 1, 16, pool_tokens_per_seq=128, topk=64, seed=23, device=DEV)


def _run(w, step):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV)
    if step:
        out, lse = dec.step(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices)
    else:
        dec.metadata(None if w.topk else w.cache_seqlens)
        out, lse = dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices)
    torch.cuda.synchronize()
    return dec, out.clone(), lse.clone()


@pytest.mark.parametrize("kind", ["dense", "fp8", "sparse"])
def test_max_items(kind):
    w = _make(kind)
    assert w.batch * w.s_q == MAX_ITEMS
    print(f"{kind}: B={w.batch} s_q={w.s_q} H={w.h_q} pages={w.num_blocks}", flush=True)

    dec, do, dl = _run(w, step=False)
    got = dec.meta_buf.cpu().numpy()[: dec.meta.bytes // 4]
    if w.topk:
        n = S.item_tiles_sparse(w.batch, w.s_q, w.topk)
    else:
        n = S.item_tiles_dense(w.cache_seqlens.cpu().numpy(), w.s_q, w.causal)
    ref = S.metadata_words(S.schedule(n, dec.meta.num_partitions, dec.meta.fixed_overhead), w.s_q)
    assert np.array_equal(got, ref), "scheduler metadata differs from the oracle scheduler"

    _, so, sl = _run(w, step=True)
    as_bits = torch.int16 if so.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(so.view(as_bits), do.view(as_bits)), "step and metadata + decode outputs differ"
    assert torch.equal(sl.view(torch.int32), dl.view(torch.int32)), "step and metadata + decode lse differ"

    # every query group: empty rows are lse -inf with zero output, the rest finite
    lse = sl.cpu().numpy()                       # [B, H, S]
    out = so.float()
    if w.topk:
        idx = w.indices.cpu().numpy()
        visible = ((idx >= 0) & (idx < w.num_blocks * 64)).sum(axis=-1)
    else:
        L = w.cache_seqlens.cpu().numpy()
        visible = np.array([[A.visible_len(int(L[b]), w.s_q, i, w.causal) for i in range(w.s_q)]
                            for b in range(w.batch)])
    empty = visible == 0                         # [B, S]
    assert np.array_equal(np.isneginf(lse).all(axis=1), empty)
    assert np.isfinite(lse.transpose(0, 2, 1)[~empty]).all()
    assert bool(torch.isfinite(out).all())
    e = torch.from_numpy(empty).to(out.device)
    assert bool((out[e] == 0).all())

    # sampled query groups against the oracle
    r = np.random.default_rng(99)
    items = {(0, 0), (w.batch - 1, w.s_q - 1)}
    items |= {(int(b), int(i)) for b, i in list(zip(*np.nonzero(empty)))[:4]}
    items |= {(int(r.integers(w.batch)), int(r.integers(w.s_q))) for _ in range(40)}
    items = sorted(items)
    kv = kv_host_rows(w, items) if w.topk else None
    ro, rl = oracle(w, items=items, kv=kv)
    kw = dict(rel_l2=FP8_REL_L2) if kind == "fp8" else {}
    go = so.float().cpu().numpy().astype(np.float64)
    print(compare(go, lse.astype(np.float64), ro, rl, items=items, **kw), flush=True)
