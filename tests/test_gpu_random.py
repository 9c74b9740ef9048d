"""Seeded random problems through both call patterns, on every cache format.

Each case draws a cache format (dense bf16, dense FP8, sparse bf16, sparse
FP8, the 528- and 288-byte records), a batch, s_q, a head count (including
counts that are not a multiple of 32 and two head blocks), cache lengths or
top-k sizes mixed with the edge values 0, 1, 63, 64, 65 and 128, causal
masking, the output type, an attention sink and per-query top-k lengths.  The
one-call step (schedule in the kernel where the batch allows it) and the
metadata call followed by the decode call must give the same outputs bit for
bit, and both must match the fp64 oracle within the tolerances the other
parity tests use.  Further cases take batches past the in-kernel schedule's
256 items (the step runs the scheduler kernel first), the sparse prefill
(rows that see nothing, top-k lengths of zero or below, sinks of -inf) and
the standalone combine (items of 0 to 6 splits, partials of lse -inf)."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from workloads import make_dense, make_sparse, make_fp8_dense, make_sparse_prefill
from helpers import oracle, compare, bits16, draw_random_problem, FP8_REL_L2

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


def _run(w, num_cus, step):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV, num_cus)
    tl, sink = getattr(w, "topk_length", None), getattr(w, "attn_sink", None)
    if step:
        out, lse = dec.step(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, None, tl, sink)
    else:
        dec.metadata(None if w.topk else w.cache_seqlens, None, tl)
        out, lse = dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, None, tl, sink)
    torch.cuda.synchronize()
    return out.clone(), lse.clone()


@pytest.mark.parametrize("seed", range(64))
def test_random_problem(seed):
    kind, w, desc = draw_random_problem(seed, DEV)
    print(desc, flush=True)
    num_cus = (0, 7, 64)[seed % 3]
    so, sl = _run(w, num_cus, step=True)
    do, dl = _run(w, num_cus, step=False)
    as_bits = torch.int16 if so.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(so.view(as_bits), do.view(as_bits)), "step and metadata + decode outputs differ"
    assert torch.equal(sl.view(torch.int32), dl.view(torch.int32)), "step and metadata + decode lse differ"
    kv = w.kv.cpu().numpy().reshape(-1, int(w.kv.shape[-1])) if kind in ("v41", "fp4") else None
    ro, rl = oracle(w, kv=kv)
    kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kind in ("fp8", "sparse_fp8") else {}
    go = so.float().cpu().numpy().astype(np.float64)
    gl = sl.cpu().numpy().astype(np.float64)
    print(compare(go, gl, ro, rl, **kw), flush=True)


def _sink(r, H):
    s = torch.as_tensor(r.normal(8.0, 4.0, size=H), dtype=torch.float32)
    s[0] = -float("inf")
    return s.to(DEV)


@pytest.mark.parametrize("seed", range(12))
def test_random_large_batch(seed):
    r = np.random.default_rng(7000 + seed)
    kind = ("dense", "fp8", "sparse")[seed % 3]
    S = int(r.choice([1, 2, 3]))
    B = int(r.integers(257 // S + 1, 301))
    H = int(r.choice([16, 32]))
    if kind == "sparse":
        topk = int(r.integers(1, 129))
        w = make_sparse(B, S, H, pool_tokens_per_seq=128, topk=topk, invalid_frac=0.1, seed=seed, device=DEV)
        desc = f"large {kind} B={B} S={S} H={H} topk={topk}"
    else:
        lens = [int(x) for x in r.integers(0, 301, size=B)]
        make = make_dense if kind == "dense" else make_fp8_dense
        w = make(B, S, H, lens, causal=bool(S > 1), seed=seed, device=DEV)
        desc = f"large {kind} B={B} S={S} H={H}"
    if r.random() < 0.5:
        w.attn_sink = _sink(r, H)
        desc += " sink"
    print(desc, flush=True)
    num_cus = (0, 33)[seed % 2]
    so, sl = _run(w, num_cus, step=True)
    do, dl = _run(w, num_cus, step=False)
    assert torch.equal(so.view(torch.int16), do.view(torch.int16)), "step and metadata + decode outputs differ"
    assert torch.equal(sl.view(torch.int32), dl.view(torch.int32)), "step and metadata + decode lse differ"
    ro, rl = oracle(w)
    kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kind == "fp8" else {}
    print(compare(so.float().cpu().numpy().astype(np.float64), sl.cpu().numpy().astype(np.float64), ro, rl, **kw),
          flush=True)


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill(seed):
    import mla_decode_amd as mla
    r = np.random.default_rng(8000 + seed)
    kv_format = ("bf16", "fp8")[seed % 2]
    s_q = int(r.integers(1, 201))
    s_kv = int(r.integers(s_q, 3001))
    H = int(r.choice([16, 64, 128]))
    topk = int(r.integers(1, min(s_kv, 500) + 1))
    w = make_sparse_prefill(s_q, s_kv, H, topk, invalid_frac=float(r.choice([0.0, 0.1])), seed=seed, device=DEV,
                            kv_format=kv_format)
    idx = w.indices.clone()
    idx[int(r.integers(0, s_q)), 0, :] = -1               # a row that sees nothing
    w.indices = idx
    if r.random() < 0.5:
        w.topk_length = torch.as_tensor(r.integers(-2, topk + 3, size=s_q), dtype=torch.int32).to(DEV)
    if r.random() < 0.5:
        w.attn_sink = _sink(r, H)
    print(f"prefill {kv_format} s_q={s_q} s_kv={s_kv} H={H} topk={topk} "
          f"topk_length={w.topk_length is not None} sink={w.attn_sink is not None}", flush=True)
    out, lse = mla.sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, topk_length=w.topk_length,
                                  attn_sink=w.attn_sink, num_cus=(0, 19)[seed % 2])
    torch.cuda.synchronize()
    q = bits16(w.q)[None]
    kv = w.kv.cpu().numpy().reshape(s_kv, -1) if kv_format == "fp8" else bits16(w.kv).reshape(s_kv, 576)
    tl = None if w.topk_length is None else w.topk_length.cpu().numpy()[None]
    sink = None if w.attn_sink is None else w.attn_sink.cpu().double().numpy()
    ro, rl = A.decode(q, kv, w.softmax_scale, indices=w.indices.cpu().numpy()[None, :, 0, :], kv_format=kv_format,
                      topk_length=tl, attn_sink=sink)
    kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kv_format == "fp8" else {}
    print(compare(out.float().cpu().numpy().astype(np.float64)[None], lse.cpu().numpy().astype(np.float64)[None],
                  ro, rl, **kw), flush=True)


@pytest.mark.parametrize("seed", range(12))
def test_random_combine(seed):
    import mla_decode_amd as mla
    r = np.random.default_rng(9000 + seed)
    B, S = int(r.integers(1, 31)), int(r.choice([1, 2]))
    H = int(r.choice([8, 16, 64, 128]))
    out_dtype = (torch.bfloat16, torch.float32)[seed % 2]
    ns = r.integers(0, 7, size=B * S)
    so = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    T = max(int(so[-1]), 1)
    o = r.normal(size=(T, H, 512))
    lse = r.normal(size=(T, H)) * 3
    lse[r.random(size=(T, H)) < 0.15] = -np.inf          # partials that saw nothing
    sink = _sink(r, H) if seed % 3 == 0 else None
    out = torch.empty(B, S, H, 512, dtype=out_dtype, device=DEV)
    lo = torch.empty(B, H, S, dtype=torch.float32, device=DEV)
    mla.combine(B * S, H, S, torch.as_tensor(o, dtype=torch.float32).to(DEV),
                torch.as_tensor(lse, dtype=torch.float32).to(DEV), torch.from_numpy(so).to(DEV), out, lo,
                attn_sink=sink)
    torch.cuda.synchronize()
    o32 = o.astype(np.float32).astype(np.float64)
    l32 = lse.astype(np.float32).astype(np.float64)
    go, gl = out.float().cpu().numpy(), lo.cpu().numpy()
    tol = 1e-5 if out_dtype == torch.float32 else 2.0 ** -7
    for j in range(B * S):
        b, i = divmod(j, S)
        ro, rl = A.merge_partials(o32[so[j]:so[j + 1]], l32[so[j]:so[j + 1]])
        if ns[j] == 0:
            ro, rl = np.zeros((H, 512)), np.full(H, -np.inf)
        elif sink is not None:
            ro = A.apply_sink(ro, rl, sink.cpu().double().numpy())
        assert np.all(np.abs(go[b, i] - ro) <= tol * (1.0 + np.abs(ro))), f"item {j}: out"
        assert np.array_equal(np.isneginf(gl[b, :, i]), np.isneginf(rl)), f"item {j}: lse -inf"
        fin = np.isfinite(rl)
        assert np.all(np.abs(gl[b, fin, i] - rl[fin]) < 1e-4), f"item {j}: lse"


@pytest.mark.parametrize("seed", range(12))
def test_random_problem_debug_mode(seed, monkeypatch):
    """MLA_DEBUG=1 validates every call's inputs on the host first; valid
    random problems must pass those checks and give the same outputs, bit for
    bit, as without them."""
    kind, w, desc = draw_random_problem(seed, DEV)
    print(desc, flush=True)
    ref = [_run(w, 0, step) for step in (True, False)]
    monkeypatch.setenv("MLA_DEBUG", "1")
    got = [_run(w, 0, step) for step in (True, False)]
    monkeypatch.delenv("MLA_DEBUG")
    for (ro, rl), (go, gl) in zip(ref, got):
        as_bits = torch.int16 if ro.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(go.view(as_bits), ro.view(as_bits)) and torch.equal(gl.view(torch.int32), rl.view(torch.int32))


@pytest.mark.parametrize("seed", range(12))
def test_random_problem_nan_in_q(seed):
    """A NaN planted in one head of one query token of a random problem: that
    head's output and lse are NaN exactly where the oracle's are (all of them
    when the token sees anything, out 0 and lse -inf when it sees nothing), with
    or without a sink, and every other value matches as before."""
    kind, w, desc = draw_random_problem(seed, DEV)
    r = np.random.default_rng(6000 + seed)
    b, i, h = int(r.integers(0, w.batch)), int(r.integers(0, w.s_q)), int(r.integers(0, w.h_q))
    w.q[b, i, h, int(r.integers(0, w.q.shape[-1]))] = float("nan")
    print(f"{desc}; NaN in q[{b}, {i}, {h}]", flush=True)
    kv = w.kv.cpu().numpy().reshape(-1, int(w.kv.shape[-1])) if kind in ("v41", "fp4") else None
    ro, rl = oracle(w, kv=kv)
    kw = dict(rel_l2=FP8_REL_L2, max_abs=1e-2) if kind in ("fp8", "sparse_fp8") else {}
    for step in (True, False):
        go, gl = _run(w, (0, 7)[seed % 2], step)
        go = go.float().cpu().numpy().astype(np.float64)
        gl = gl.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(go), np.isnan(ro)), "NaN positions of out differ"
        assert np.array_equal(np.isnan(gl), np.isnan(rl)), "NaN positions of lse differ"
        go2, ro2, gl2, rl2 = go.copy(), ro.copy(), gl.copy(), rl.copy()
        go2[np.isnan(go2)] = ro2[np.isnan(ro2)] = 0.0
        gl2[np.isnan(gl2)] = rl2[np.isnan(rl2)] = 0.0
        print(step, compare(go2, gl2, ro2, rl2, **kw), flush=True)
