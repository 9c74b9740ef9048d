"""GPU parity over head counts and output types on every cache format: head
counts that are not a multiple of 32 (masked lanes), two head blocks
(h_q = 192), fp32 output, and s_q > 1, for dense bf16, dense FP8, sparse
bf16, sparse FP8, and the 528- and 288-byte records."""

import numpy as np
import pytest
import torch

from workloads import make_dense, make_sparse, make_fp8_dense, make_v41_sparse, make_fp4_sparse
from helpers import run_library, oracle, compare, FP8_REL_L2

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _make(kind, H, out_dtype, seed):
    if kind == "dense":
        return make_dense(3, 2, H, [1, 300, 777], causal=True, seed=seed, device=DEV, out_dtype=out_dtype)
    if kind == "fp8":
        return make_fp8_dense(3, 1, H, [1, 300, 777], seed=seed, device=DEV, out_dtype=out_dtype)
    if kind == "sparse":
        return make_sparse(3, 2, H, pool_tokens_per_seq=1024, topk=333, invalid_frac=0.1, seed=seed, device=DEV,
                           out_dtype=out_dtype)
    if kind == "sparse_fp8":
        return make_sparse(3, 2, H, pool_tokens_per_seq=1024, topk=333, invalid_frac=0.1, seed=seed, device=DEV,
                           out_dtype=out_dtype, kv_format="fp8")
    make = make_fp4_sparse if kind == "fp4" else make_v41_sparse
    w = make(3, 2, H, pool_tokens_per_seq=1024, topk=333, invalid_frac=0.1, seed=seed, device=DEV)
    w.out_dtype = out_dtype
    return w


@pytest.mark.parametrize("kind", ["dense", "fp8", "sparse", "sparse_fp8", "v41", "fp4"])
@pytest.mark.parametrize("H,out_dtype", [(40, "bf16"), (192, "fp32"), (128, "fp32")])
def test_heads_and_out_dtype(kind, H, out_dtype):
    print(f"{kind} H={H} out={out_dtype}", flush=True)
    w = _make(kind, H, out_dtype, seed=7 * H + len(kind))
    kv = w.kv.cpu().numpy().reshape(-1, int(w.kv.shape[-1])) if kind in ("v41", "fp4") else None
    for num_cus in (0, 9):
        go, gl, _ = run_library(w, num_cus=num_cus)
        ro, rl = oracle(w, kv=kv)
        kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kind in ("fp8", "sparse_fp8") else {}
        print(num_cus, compare(go, gl, ro, rl, **kw), flush=True)
