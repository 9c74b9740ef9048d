"""GPU parity of the optional arguments of the FlashMLA README's sparse
attention call: a per-head ``attn_sink`` (out scaled by exp(lse) / (exp(lse) +
exp(sink)), lse unchanged) and a per-query ``topk_length`` (only the first
topk_length entries of an index row are used).  Items that lie in one
partition take the sink in the decode kernel's epilogue, split items in the
combine; the schedule with top-k lengths is checked bit-exactly."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import sched as S
from workloads import make_dense, make_sparse, make_fp8_dense
from helpers import run_library, oracle, compare, FP8_REL_L2

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _say(*a):
    print(*a, flush=True)


def _sink(h, seed):
    g = torch.Generator().manual_seed(seed)
    s = torch.randn(h, generator=g) * 4 + 8      # around typical lse values (ln of a few thousand)
    s[0] = -float("inf")                         # no sink for head 0
    s[1] = 40.0                                  # a sink that swamps the row
    return s.to(torch.float32).to(DEV)


@pytest.mark.parametrize("num_cus", [0, 8])
def test_dense_with_sink(num_cus):
    """num_cus = 8 splits every long item (combine path); 0 keeps most whole."""
    _say(f"dense sink num_cus={num_cus}")
    w = make_dense(4, 2, 128, [0, 70, 1500, 3000], causal=True, seed=41, device=DEV)
    w.attn_sink = _sink(128, 1)
    go, gl, dec = run_library(w, num_cus=num_cus)
    ro, rl = oracle(w)
    _say(compare(go, gl, ro, rl))


def test_fp32_out_with_sink():
    w = make_dense(2, 1, 16, [200, 256], seed=42, device=DEV, out_dtype='fp32', max_blocks=4, pool_blocks=8)
    w.attn_sink = _sink(16, 2)
    go, gl, _ = run_library(w, num_cus=3)
    ro, rl = oracle(w)
    _say(compare(go, gl, ro, rl))


def _meta_sparse(w, num_cus):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV, num_cus)
    dec.metadata(None, topk_length=w.topk_length)
    torch.cuda.synchronize()
    got = dec.meta_buf.cpu().numpy()[: dec.meta.bytes // 4]
    n = S.item_tiles_sparse(w.batch, w.s_q, w.topk, w.topk_length.cpu().numpy())
    ref = S.metadata_words(S.schedule(n, dec.meta.num_partitions, dec.meta.fixed_overhead), w.s_q)
    assert np.array_equal(got, ref)


def _lengths(batch, s_q, topk, seed):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, topk + 1, size=(batch, s_q))
    L.flat[0] = 0            # sees nothing
    L.flat[1] = topk + 500   # clamped to topk
    L.flat[2] = -3           # clamped to 0
    L.flat[3] = 1
    return torch.from_numpy(L.astype(np.int32)).to(DEV)


@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
def test_sparse_topk_length_and_sink(kv_format):
    _say(f"sparse topk_length + sink {kv_format}")
    w = make_sparse(5, 2, 128, pool_tokens_per_seq=4096, topk=1000, invalid_frac=0.05, seed=43, device=DEV,
                    kv_format=kv_format)
    w.topk_length = _lengths(5, 2, 1000, 7)
    w.attn_sink = _sink(128, 3)
    for num_cus in (1, 5, 64, 256):
        _meta_sparse(w, num_cus)
    for num_cus in (0, 16):
        go, gl, _ = run_library(w, num_cus=num_cus)
        ro, rl = oracle(w)
        assert np.all(np.isneginf(rl[0, :, 0])) and np.all(np.isneginf(gl[0, :, 0]))
        kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kv_format == "fp8" else {}
        _say(num_cus, compare(go, gl, ro, rl, **kw))


@pytest.mark.parametrize("num_cus", [12, 48])
def test_sparse_rows_seeing_nothing_with_sink(num_cus):
    """Rows whose top-k entries are all -1 see nothing: out stays 0 and lse is
    -inf with a sink too, also for a head whose sink is -inf (where the sink
    factor exp(lse) / (exp(lse) + exp(sink)) itself would be 0 / 0).  The 12
    items have four 64-token tiles each: with 12 partitions every item is
    whole (the decode kernel writes the output), with 48 every tile is a
    split (the combine does)."""
    _say(f"sparse rows seeing nothing, sink, num_cus={num_cus}")
    w = make_sparse(6, 2, 128, pool_tokens_per_seq=256, topk=200, seed=43, device=DEV)
    w.indices[0, 0, :] = -1
    w.indices[3, 1, :] = -1
    w.indices[5, :, :] = -1
    w.attn_sink = _sink(128, 4)
    go, gl, _ = run_library(w, num_cus=num_cus)
    ro, rl = oracle(w)
    for b, i in ((0, 0), (3, 1), (5, 0), (5, 1)):
        assert np.all(go[b, i] == 0.0) and np.all(np.isneginf(gl[b, :, i]))
    _say(compare(go, gl, ro, rl))


def test_gather_rows_with_topk_length():
    import mla_decode_amd as mla
    w = make_sparse(3, 2, 16, pool_tokens_per_seq=512, topk=100, invalid_frac=0.2, seed=44, device=DEV)
    w.topk_length = _lengths(3, 2, 100, 8)
    dec = mla.Decoder.for_workload(w, DEV)
    stride = 64 * ((w.topk + 63) // 64)
    rows = torch.full((6, stride), -7, dtype=torch.int32, device=DEV)
    mla.debug_gather_rows(dec.problem, w.indices, None, rows, topk_length=w.topk_length)
    torch.cuda.synchronize()
    got = rows.cpu().numpy()
    idx = w.indices.cpu().numpy().astype(np.int64)
    L = w.topk_length.cpu().numpy()
    nrows = w.num_blocks * 64
    for j in range(6):
        b, i = divmod(j, 2)
        n = min(max(int(L[b, i]), 0), 100)
        ntile = (n + 63) // 64
        exp = -np.ones(ntile * 64, dtype=np.int64)
        exp[:n] = np.where((idx[b, i, :n] >= 0) & (idx[b, i, :n] < nrows), idx[b, i, :n], -1)
        assert np.array_equal(got[j, : exp.size], exp), j
        assert np.all(got[j, exp.size:] == -7)


def test_combine_standalone_with_sink():
    import mla_decode_amd as mla
    g = torch.Generator().manual_seed(5)
    H, S_, B = 8, 1, 4
    ns = [0, 1, 3, 6]
    so = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    T = int(so[-1])
    o = torch.randn(T, H, 512, generator=g)
    lse = torch.randn(T, H, generator=g) * 3
    sink = torch.randn(H, generator=g) * 2
    sink[3] = -float("inf")
    out = torch.empty(B, S_, H, 512, dtype=torch.float32, device=DEV)
    lo = torch.empty(B, H, S_, dtype=torch.float32, device=DEV)
    mla.combine(B * S_, H, S_, o.to(DEV), lse.to(DEV), torch.from_numpy(so).to(DEV), out, lo,
                attn_sink=sink.to(DEV))
    torch.cuda.synchronize()
    for j in range(B):
        ro, rl = A.merge_partials(o[so[j]:so[j + 1]].double().numpy(), lse[so[j]:so[j + 1]].double().numpy())
        if ns[j] == 0:
            ro, rl = np.zeros((H, 512)), np.full(H, -np.inf)
        else:
            ro = A.apply_sink(ro, rl, sink.double().numpy())
        assert np.max(np.abs(out[j, 0].cpu().numpy() - ro)) < 1e-5
        gl = lo[j, :, 0].cpu().numpy()
        fin = np.isfinite(rl)
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
        assert np.all(np.abs(gl[fin] - rl[fin]) < 1e-5)
