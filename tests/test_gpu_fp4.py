"""GPU parity of top-k decode over the 288-byte FP4 records of the 512-wide
head (FlashMLA README copy, "FP8 / FP4 KV Cache Format": 512 e2m1 values two
per byte, the even-indexed one in the low nibble, with one e4m3 scale per 16
values; K = V = the 512 values).  The dequantised values are exact in bfloat16,
so the bfloat16 tolerances apply."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from workloads import make_fp4_sparse, make_sparse_prefill, encode_fp4_records
from helpers import run_library, oracle, compare, bits16, kv_host_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _kv_host(w):
    return w.kv.cpu().numpy().reshape(-1, 288)


def test_fp4_small_edge_cases():
    print("fp4 small", flush=True)
    w = make_fp4_sparse(4, 2, 64, pool_tokens_per_seq=640, topk=100, invalid_frac=0.1, seed=191, device=DEV)
    idx = w.indices.clone()
    idx[1, 0, :] = -1                                   # a row that sees nothing
    idx[2, 1, 3] = w.num_blocks * 64 + 9                # out of range: masked
    idx[3, 0, 10] = idx[3, 0, 11]                       # duplicate entry counts twice
    w.indices = idx
    for num_cus in (0, 5):
        go, gl, _ = run_library(w, num_cus=num_cus)
        ro, rl = oracle(w, kv=_kv_host(w))
        assert np.isneginf(rl[1, :, 0]).all() and np.isneginf(gl[1, :, 0]).all()
        print(num_cus, compare(go, gl, ro, rl), flush=True)


def test_fp4_topk_length_and_sink():
    w = make_fp4_sparse(3, 2, 128, pool_tokens_per_seq=4096, topk=1000, invalid_frac=0.05, seed=192, device=DEV)
    rng = np.random.default_rng(4)
    w.topk_length = torch.from_numpy(rng.integers(0, 1100, size=(3, 2)).astype(np.int32)).to(DEV)
    w.attn_sink = (torch.randn(128, generator=torch.Generator().manual_seed(6)) * 2 + 5).to(DEV)
    go, gl, _ = run_library(w)
    ro, rl = oracle(w, kv=_kv_host(w))
    print(compare(go, gl, ro, rl), flush=True)


def test_fp4_headline_shape_sampled():
    """b=128, s_q=2, h_q=128, top-k 2048: the shape ``bench.py --workload fp4_sparse_topk2048`` times."""
    w = make_fp4_sparse(128, 2, 128, pool_tokens_per_seq=32768, topk=2048, seed=193, device=DEV)
    items = [(0, 0), (64, 1), (127, 0)]
    go, gl, _ = run_library(w)
    ro, rl = oracle(w, items=items, kv=kv_host_rows(w, items))
    print(compare(go, gl, ro, rl, items=items), flush=True)


def test_fp4_sparse_prefill():
    import mla_decode_amd as mla
    p = make_sparse_prefill(200, 900, 64, 300, invalid_frac=0.05, seed=194, device=DEV)
    x = torch.randn(900, 512, generator=torch.Generator(device=DEV).manual_seed(17), device=DEV)
    kv = encode_fp4_records(x).view(900, 1, 288)
    q = torch.randn(200, 64, 512, generator=torch.Generator(device=DEV).manual_seed(18), device=DEV).to(torch.bfloat16)
    scale = 1.0 / 512 ** 0.5
    out, lse = mla.sparse_prefill(q, kv, p.indices, scale)
    torch.cuda.synchronize()
    ro, rl = A.decode(bits16(q)[None], kv.cpu().numpy().reshape(900, 288), scale,
                      indices=p.indices.cpu().numpy()[None, :, 0, :], kv_format='fp4_288')
    go = out.float().cpu().numpy().astype(np.float64)[None]
    gl = lse.cpu().numpy().astype(np.float64)[None]
    print(compare(go, gl, ro, rl), flush=True)
