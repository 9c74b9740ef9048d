"""GPU: a NaN in the cache reaches the output of every query row that attends
the token holding it, as in the fp64 oracle, also when that row is split over
several partitions (the partition's lse is NaN, not the -inf of an empty
split, so the merge keeps it).  Rows that do not see the token are unaffected."""

import numpy as np
import pytest
import torch

from workloads import make_dense, make_fp4_sparse
from helpers import run_library, oracle, compare

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _check(w, nan_items, num_cus, kv=None):
    go, gl, _ = run_library(w, num_cus=num_cus)
    ro, rl = oracle(w, kv=kv)
    for b, i in nan_items:
        assert np.isnan(ro[b, i]).all() and np.isnan(rl[b, :, i]).all()
        assert np.isnan(go[b, i]).all(), (b, i)
        assert np.isnan(gl[b, :, i]).all(), (b, i)
    rest = [(b, i) for b in range(w.batch) for i in range(w.s_q) if (b, i) not in nan_items]
    return compare(go, gl, ro, rl, items=rest)


def test_dense_nan_token_in_a_split_item():
    print("dense nan", flush=True)
    w = make_dense(3, 1, 128, [3000, 1500, 900], seed=71, device=DEV)
    page = int(w.block_table[1, 7])
    w.kv[page, 13, 0, 100] = float("nan")          # token 7*64+13 of request 1, a latent dim
    for num_cus in (0, 3):                          # request 1 split over many partitions, and over few
        print(num_cus, _check(w, [(1, 0)], num_cus), flush=True)


def test_fp4_nan_scale():
    print("fp4 nan scale", flush=True)
    w = make_fp4_sparse(3, 1, 64, pool_tokens_per_seq=1024, topk=300, seed=72, device=DEV)
    row = int(w.indices[2, 0, 17])
    assert row >= 0 and not bool((w.indices[:2] == row).any())
    rec = w.kv.view(-1, 288)
    rec[row, 256 + 3] = 0x7F                        # e4m3 NaN scale of values 48..63
    rec[int(w.indices[0, 0, 5]), 256 + 9] = 0x00    # a zero scale: that group reads as zeros
    kv = w.kv.cpu().numpy().reshape(-1, 288)
    for num_cus in (0, 7):
        print(num_cus, _check(w, [(2, 0)], num_cus, kv=kv), flush=True)


def test_nan_in_one_head_of_q():
    """Every partition of the item sees the NaN (it is in q), so all its
    splits report a NaN lse; only that head of that query token is NaN."""
    print("q nan", flush=True)
    w = make_dense(3, 1, 128, [3000, 1500, 900], seed=73, device=DEV)
    w.q[1, 0, 5, 7] = float("nan")
    ro0, rl0 = oracle(w)
    for num_cus in (0, 3):
        go, gl, _ = run_library(w, num_cus=num_cus)
        ro, rl = ro0.copy(), rl0.copy()
        assert np.isnan(ro[1, 0, 5]).all() and np.isnan(rl[1, 5, 0])
        assert np.isnan(go[1, 0, 5]).all() and np.isnan(gl[1, 5, 0]), num_cus
        go[1, 0, 5] = ro[1, 0, 5] = 0.0
        gl[1, 5, 0] = rl[1, 5, 0] = 0.0
        print(num_cus, compare(go, gl, ro, rl), flush=True)
