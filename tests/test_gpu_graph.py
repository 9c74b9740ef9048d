"""A whole decode step (scheduler, decode kernel, combine) recorded into a HIP
graph: every replay, with eager work and synchronisations in between, gives
bitwise the eager step's output."""

import numpy as np
import pytest
import torch

from workloads import make_config, make_sparse
from helpers import oracle, compare

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


@pytest.mark.parametrize("which", ["config3", "sparse"])
def test_graph_replays_match_eager(which):
    import mla_decode_amd as mla
    print(f"graph {which}", flush=True)
    if which == "config3":
        w = make_config(3, device=DEV)
    else:
        w = make_sparse(8, 2, 128, pool_tokens_per_seq=8192, topk=2048, invalid_frac=0.05, seed=81, device=DEV)
    dec = mla.Decoder.for_workload(w, DEV)
    seqlens = None if w.topk else w.cache_seqlens
    out, lse = dec.step(w.q, w.kv, w.block_table, seqlens, w.indices)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = dec.capture(w.q, w.kv, w.block_table, seqlens, w.indices)
    for r in range(4):
        dec.out.fill_(3.0)
        dec.lse.fill_(3.0)
        dec.meta_buf.fill_(0)                       # the replay rebuilds the schedule
        scratch = torch.randn(1 << 20, device=DEV)  # unrelated eager work between replays
        (scratch * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.out.view(torch.int16), ref_out.view(torch.int16)), r
        assert torch.equal(dec.lse, ref_lse), r
    if which == "sparse":
        go = ref_out.float().cpu().numpy().astype(np.float64)
        gl = ref_lse.cpu().numpy().astype(np.float64)
        ro, rl = oracle(w)
        print(compare(go, gl, ro, rl), flush=True)
