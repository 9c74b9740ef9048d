"""GPU parity of the top-k sparse prefill (README copy, "DSA Prefill"): many
query rows over a flat, unpaged cache of s_kv rows, each row attending to its
own index list.  Entries < 0 or >= s_kv are invalid, including those that
fall inside the last partial 64-row page; the optional topk_length and
attn_sink apply as in decode."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from workloads import make_sparse_prefill
from helpers import bits16, compare, FP8_REL_L2

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _oracle(w, rows=None):
    q = bits16(w.q)[None]                                    # [1, s_q, h_q, 576]
    kv = w.kv.cpu().numpy().reshape(w.s_kv, -1) if w.kv_format == 'fp8' else bits16(w.kv).reshape(w.s_kv, 576)
    idx = w.indices.cpu().numpy()[None, :, 0, :]             # [1, s_q, topk]
    tl = None if w.topk_length is None else w.topk_length.cpu().numpy()[None]
    sink = None if w.attn_sink is None else w.attn_sink.cpu().double().numpy()
    items = None if rows is None else [(0, s) for s in rows]
    return A.decode(q, kv, w.softmax_scale, indices=idx, kv_format=w.kv_format, items=items, topk_length=tl,
                    attn_sink=sink)


def _run(w, **kw):
    import mla_decode_amd as mla
    out, lse = mla.sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, topk_length=w.topk_length,
                                  attn_sink=w.attn_sink, **kw)
    torch.cuda.synchronize()
    go = out.float().cpu().numpy().astype(np.float64)[None]            # [1, s_q, h_q, 512]
    gl = lse.cpu().numpy().astype(np.float64)[None]                    # [1, h_q, s_q]
    return go, gl


@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
def test_prefill_small_edge_cases(kv_format):
    print(f"prefill small {kv_format}", flush=True)
    w = make_sparse_prefill(300, 1000, 128, 600, invalid_frac=0.05, seed=51, device=DEV, kv_format=kv_format)
    idx = w.indices.clone()
    idx[0, 0, :] = -1                      # a row that sees nothing
    idx[1, 0, :40] = 1000 + torch.arange(24, device=DEV).repeat(2)[:40].int()   # in the last page, past s_kv
    idx[2, 0, 5] = 1 << 20                 # far out of range
    w.indices = idx
    kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kv_format == "fp8" else {}
    for num_cus in (0, 7):
        go, gl = _run(w, num_cus=num_cus)
        ro, rl = _oracle(w)
        assert np.all(np.isneginf(gl[0, :, 0]))
        print(num_cus, compare(go, gl, ro, rl, **kw), flush=True)


def test_prefill_topk_length_and_sink():
    w = make_sparse_prefill(257, 777, 64, 300, invalid_frac=0.05, seed=52, device=DEV)
    rng = np.random.default_rng(3)
    L = rng.integers(-2, 340, size=257).astype(np.int32)
    w.topk_length = torch.from_numpy(L).to(DEV)
    g = torch.Generator().manual_seed(4)
    w.attn_sink = (torch.randn(64, generator=g) * 3 + 6).to(DEV)
    go, gl = _run(w)
    ro, rl = _oracle(w)
    print(compare(go, gl, ro, rl), flush=True)


def test_prefill_bench_shape_sampled():
    """The shape ``bench.py --workload sparse_prefill`` times: 4096 query rows
    at the end of a 32768-row cache, top-k 2048, 128 heads."""
    w = make_sparse_prefill(4096, 32768, 128, 2048, seed=53, device=DEV)
    rows = [0, 1, 777, 2048, 4095]
    go, gl = _run(w)
    ro, rl = _oracle(w, rows)
    print(compare(go, gl, ro, rl, items=[(0, s) for s in rows]), flush=True)
