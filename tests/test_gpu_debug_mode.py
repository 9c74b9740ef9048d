"""MLA_DEBUG=1 on the GPU: valid calls give the same bytes as without the
mode, and calls whose device arrays fail the host checks (a stale schedule, a
page id or top-k index out of range, broken split offsets) are refused with
INVALID_ARG before any launch."""

import pytest
import torch

from workloads import make_dense, make_sparse

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _run(w):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV)
    out, lse = dec.run_workload(w)
    torch.cuda.synchronize()
    return dec, out.clone(), lse.clone()


def test_debug_mode_valid_calls_match(monkeypatch):
    print("debug mode: dense b=3 s_q=2 causal and sparse b=2 topk=200", flush=True)
    wd = make_dense(3, 2, 128, [70, 300, 1], causal=True, seed=3, device=DEV)
    ws = make_sparse(2, 1, 128, pool_tokens_per_seq=1024, topk=200, seed=4, device=DEV)
    ref = [_run(w)[1:] for w in (wd, ws)]
    monkeypatch.setenv("MLA_DEBUG", "1")
    got = [_run(w)[1:] for w in (wd, ws)]
    for (o0, l0), (o1, l1) in zip(ref, got):
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_debug_mode_refuses_bad_arrays(monkeypatch):
    import mla_decode_amd as mla
    print("debug mode: refusals", flush=True)
    monkeypatch.setenv("MLA_DEBUG", "1")
    w = make_dense(2, 1, 128, [200, 256], seed=5, device=DEV)
    dec = mla.Decoder.for_workload(w, DEV)
    dec.metadata(w.cache_seqlens)
    # stale schedule: the lengths changed after the metadata call
    shorter = w.cache_seqlens.clone()
    shorter[0] -= 64
    with pytest.raises(mla.MlaError) as e:
        dec.decode(w.q, w.kv, w.block_table, shorter)
    assert e.value.status == 1
    # a page in use outside the pool
    table = w.block_table.clone()
    table[1, 0] = w.kv.shape[0]
    with pytest.raises(mla.MlaError) as e:
        dec.decode(w.q, w.kv, table, w.cache_seqlens)
    assert e.value.status == 1
    # a length beyond the block table
    with pytest.raises(mla.MlaError) as e:
        dec.metadata(torch.full_like(w.cache_seqlens, 64 * w.block_table.shape[1] + 1))
    assert e.value.status == 1
    # top-k index past the cache
    s = make_sparse(2, 1, 128, pool_tokens_per_seq=1024, topk=128, seed=6, device=DEV)
    sdec = mla.Decoder.for_workload(s, DEV)
    sdec.metadata()
    idx = s.indices.clone()
    idx[1, 0, 5] = s.kv.shape[0] * 64
    with pytest.raises(mla.MlaError) as e:
        sdec.decode(s.q, s.kv, indices=idx)
    assert e.value.status == 1
    # split offsets that are not a prefix sum
    H = 16
    so = torch.tensor([0, 2, 1, 3], dtype=torch.int32, device=DEV)
    o = torch.zeros(3, H, 512, device=DEV)
    lse = torch.zeros(3, H, device=DEV)
    with pytest.raises(mla.MlaError) as e:
        mla.combine(3, H, 1, o, lse, so, torch.empty(3, 1, H, 512, device=DEV), torch.empty(3, H, 1, device=DEV))
    assert e.value.status == 1
    torch.cuda.synchronize()
