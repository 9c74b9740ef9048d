"""GPU parity of the float16 split partials (bf16 output): each lane stores its
partial output values scaled by a power of two taken from their largest
magnitude, so values far outside float16's range (and far below its smallest
normal) survive the round trip through the combine.  The latent dims of the
cache are scaled by 2^k and those of q by 2^-k, which leaves every score
unchanged and scales the output by exactly 2^k (bf16 keeps power-of-two
scalings exact)."""

import numpy as np
import pytest
import torch

from workloads import make_dense, make_sparse
from helpers import run_library, oracle, compare

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _scale(w, k):
    w.kv[..., :512] *= 2.0 ** k
    w.q[..., :512] *= 2.0 ** -k
    return w


@pytest.mark.parametrize("k", [0, 40, 100, -40, -100])
def test_dense_partial_magnitudes(k):
    print(f"dense 2^{k}", flush=True)
    w = _scale(make_dense(2, 1, 128, [3000, 2500], seed=300 + k, device=DEV), k)
    ref_out, ref_lse = oracle(w)
    for num_cus in (0, 24):   # many splits per item, and a few
        go, gl, _ = run_library(w, num_cus=num_cus)
        assert np.all(np.isfinite(go))
        st = compare(go / 2.0 ** k, gl, ref_out / 2.0 ** k, ref_lse)
        print(num_cus, st, flush=True)


@pytest.mark.parametrize("k", [60, -60])
def test_sparse_partial_magnitudes(k):
    print(f"sparse 2^{k}", flush=True)
    w = _scale(make_sparse(2, 2, 128, pool_tokens_per_seq=4096, topk=2048, invalid_frac=0.05, seed=400 + k,
                           device=DEV), k)
    ref_out, ref_lse = oracle(w)
    go, gl, _ = run_library(w, num_cus=0)
    print(compare(go / 2.0 ** k, gl, ref_out / 2.0 ** k, ref_lse), flush=True)
