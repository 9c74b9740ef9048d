"""mla_decode_step_noalloc, called through the C ABI, against the step of the
existing entry points (mla_get_decode_metadata + mla_decode_fwd /
mla_sparse_decode_fwd with a caller-owned metadata buffer and workspace):
bit-identical outputs on two calls in a row, the second with a smaller
problem, so it runs over the scratch the first call left behind; the smaller
call is also checked against the oracle."""

import numpy as np
import pytest
import torch

from workloads import make_dense, make_sparse
from helpers import draw_random_problem, oracle, compare

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _both(w):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV)
    ref_out, ref_lse = dec.run_workload(w)
    ref_out, ref_lse = ref_out.clone(), ref_lse.clone()
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    toi = w.indices if w.topk else w.block_table
    mla.decode_step_noalloc(dec.problem, w.q, w.kv, toi, out, lse, cache_seqlens=None if w.topk else w.cache_seqlens,
                            topk_length=getattr(w, "topk_length", None), attn_sink=getattr(w, "attn_sink", None))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), float((out.float() - ref_out.float()).abs().max())
    assert torch.equal(lse, ref_lse)
    return out, lse


@pytest.mark.parametrize("kind", ["dense", "sparse"])
def test_noalloc_matches_the_step_on_two_calls(kind):
    if kind == "dense":
        big = make_dense(16, 1, 128, [4096] * 16, seed=31, device=DEV)
        small = make_dense(3, 2, 128, [200, 77, 1], causal=True, seed=32, device=DEV)
    else:
        big = make_sparse(16, 2, 128, pool_tokens_per_seq=8192, topk=2048, seed=33, device=DEV)
        small = make_sparse(2, 1, 128, pool_tokens_per_seq=1024, topk=200, seed=34, device=DEV)
    print(f"noalloc {kind}: big", flush=True)
    _both(big)
    print(f"noalloc {kind}: small", flush=True)
    out, lse = _both(small)
    ro, rl = oracle(small)
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl)


@pytest.mark.parametrize("seed", range(12))
def test_noalloc_matches_the_step_on_random_problems(seed):
    """Seeded random problems of every cache format (the generator the other
    random tests use): the call that allocates nothing equals the step."""
    kind, w, desc = draw_random_problem(seed, DEV)
    print(f"noalloc random {desc}", flush=True)
    _both(w)
