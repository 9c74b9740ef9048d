"""GPU parity of FP8 sparse decode at the shape the FlashMLA deep dive quotes
for its H800 kernel ("Performance", part 2): 128 requests, 2 query tokens,
128 heads, top-k 2048 and 32768 over 656-byte records.  Full-size inputs in
the launch configuration ``bench.py --workload fp8_sparse_topk*`` times;
every head and dim of sampled query tokens is checked against the fp64
oracle fed the same dequantised values."""

import numpy as np
import pytest
import torch

from workloads import make_fp8_sparse
from helpers import run_library, oracle, compare, kv_host_rows, FP8_REL_L2

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


@pytest.mark.parametrize("topk,items", [
    (2048, [(0, 0), (0, 1), (45, 1), (77, 0), (127, 1)]),
    (32768, [(0, 0), (63, 1), (127, 0)]),
])
def test_fp8_sparse_headline_sampled(topk, items):
    print(f"fp8 sparse b=128 s_q=2 h_q=128 topk={topk}", flush=True)
    w = make_fp8_sparse(topk, device=DEV)
    go, gl, dec = run_library(w)
    print(f"partitions {dec.meta.num_partitions}, split slots {dec.meta.max_splits}", flush=True)
    ro, rl = oracle(w, items=items, kv=kv_host_rows(w, items))
    print(compare(go, gl, ro, rl, items=items, rel_l2=FP8_REL_L2, max_abs=1e-2), flush=True)
    # every query token produced finite output and lse
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
