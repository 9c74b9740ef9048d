"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Sizes: small cases span several 64-token tiles, ragged tails and several
splits so the oracle checks every output; the five full-size workloads are
checked whole (every output element and lse) in the launch configuration the
benchmark times.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import sched as S
from workloads import make_config, make_dense, make_sparse, make_fp8_dense
from helpers import run_library, oracle, compare, kv_host, bits16, FP8_REL_L2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_amd._lib as L
    L.load()   # fails loudly if the HIP library is missing


DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ scheduler metadata

def _meta_case(w, num_cus):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV, num_cus)
    dec.metadata(None if w.topk else w.cache_seqlens)
    torch.cuda.synchronize()
    got = dec.meta_buf.cpu().numpy()[: dec.meta.bytes // 4]
    if w.topk:
        n = S.item_tiles_sparse(w.batch, w.s_q, w.topk)
    else:
        n = S.item_tiles_dense(w.cache_seqlens.cpu().numpy(), w.s_q, w.causal)
    ref = S.metadata_words(S.schedule(n, dec.meta.num_partitions, dec.meta.fixed_overhead), w.s_q)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_metadata_bit_exact_configs(cfg):
    _say(f"metadata config{cfg}")
    w = make_config(cfg, device=DEV)
    for num_cus in (0, 7, 1000):
        _meta_case(w, num_cus)


@pytest.mark.parametrize("seed", range(4))
def test_metadata_bit_exact_random(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    s_q = int(rng.integers(1, 4))
    lens = rng.integers(0, 700, size=B).tolist()
    w = make_dense(B, s_q, 16, lens, causal=bool(seed % 2), seed=seed, device=DEV, max_blocks=11)
    for num_cus in (1, 3, 64, 256):
        _meta_case(w, num_cus)


# ------------------------------------------------------------------ gather rows

def _gather_case(w, table):
    import mla_decode_amd as mla
    dec = mla.Decoder.for_workload(w, DEV)
    stride = 64 * ((w.topk + 63) // 64) if w.topk else 64 * w.max_blocks_per_seq
    rows = torch.full((w.batch * w.s_q, stride), -7, dtype=torch.int32, device=DEV)
    mla.debug_gather_rows(dec.problem, table, None if w.topk else w.cache_seqlens, rows)
    torch.cuda.synchronize()
    got = rows.cpu().numpy()
    nrows = w.num_blocks * 64
    for j in range(w.batch * w.s_q):
        b, i = divmod(j, w.s_q)
        if w.topk:
            idx = w.indices.cpu().numpy()[b, i].astype(np.int64)
            exp = np.where((idx >= 0) & (idx < nrows), idx, -1)
            ntile = (w.topk + 63) // 64
            exp = np.concatenate([exp, -np.ones(ntile * 64 - w.topk, dtype=np.int64)])
        else:
            vis = S.visible_len(int(w.cache_seqlens[b]), w.s_q, i, w.causal)
            ntile = (vis + 63) // 64
            exp = -np.ones(ntile * 64, dtype=np.int64)
            exp[:vis] = A.paged_rows(w.block_table.cpu().numpy()[b], vis)
        assert np.array_equal(got[j, : exp.size], exp), j
        assert np.all(got[j, exp.size:] == -7)


def test_gather_rows_dense():
    _say("gather dense")
    w = make_dense(4, 2, 16, [0, 1, 130, 257], causal=True, seed=3, device=DEV, max_blocks=5)
    _gather_case(w, w.block_table)


def test_gather_rows_sparse():
    _say("gather sparse")
    w = make_sparse(3, 2, 16, pool_tokens_per_seq=512, topk=100, invalid_frac=0.2, seed=4, device=DEV)
    idx = w.indices.clone()
    idx[0, 0, 5] = w.num_blocks * 64          # out of range -> masked
    idx[0, 1, 7] = -3
    w.indices = idx
    _gather_case(w, w.indices)


# ------------------------------------------------------------------ decode: small, all outputs

def test_config1_tiny_full():
    _say("config1")
    w = make_config(1, device=DEV)
    go, gl, _ = run_library(w)
    ro, rl = oracle(w)
    _say(compare(go, gl, ro, rl))


@pytest.mark.parametrize("B,S_,H,lens,causal", [
    (3, 1, 128, [1, 63, 200], False),
    (2, 1, 64, [64, 65], False),
    (3, 2, 128, [1, 64, 129], True),
    (2, 3, 100, [5, 190], True),
    (4, 1, 16, [700, 3, 0, 128], False),
    (1, 1, 192, [333], False),
])
def test_dense_small_shapes(B, S_, H, lens, causal):
    _say(f"dense B={B} S={S_} H={H} lens={lens} causal={causal}")
    w = make_dense(B, S_, H, lens, causal=causal, seed=B * 100 + H, device=DEV)
    go, gl, _ = run_library(w)
    ro, rl = oracle(w)
    _say(compare(go, gl, ro, rl))


def test_split_count_invariance():
    """Different partition counts (no split .. many splits) all match the
    oracle and each other within tolerance."""
    w = make_dense(3, 2, 128, [1000, 77, 520], causal=True, seed=11, device=DEV)
    ro, rl = oracle(w)
    outs = []
    for num_cus in (2, 16, 256, 1024):
        _say(f"split invariance num_cus={num_cus}")
        go, gl, dec = run_library(w, num_cus=num_cus)
        compare(go, gl, ro, rl)
        outs.append(go)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-2


@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
def test_long_partition_crosses_page_window(kv_format):
    """A partition that walks more than 64 pages reloads its window of page
    ids on the way (the kernel holds 64 page ids at a time); with two CUs the
    partitions also start mid-item and span item boundaries."""
    _say(f"long partition {kv_format}")
    make = make_dense if kv_format == "bf16" else make_fp8_dense
    w = make(3, 1, 32, [64 * 150 + 17, 64 * 70, 300], seed=12, device=DEV)
    ro, rl = oracle(w)
    for num_cus in (1, 2):
        go, gl, _ = run_library(w, num_cus=num_cus)
        if kv_format == "bf16":
            _say(compare(go, gl, ro, rl))
        else:
            _say(compare(go, gl, ro, rl, rel_l2=FP8_REL_L2, max_abs=1e-2))


def test_block_table_reshuffle_is_bitwise_invariant():
    _say("reshuffle")
    w = make_dense(2, 1, 128, [300, 190], seed=5, device=DEV, max_blocks=5, pool_blocks=12)
    go, gl, _ = run_library(w)
    perm = torch.randperm(12, generator=torch.Generator().manual_seed(1))
    kv2 = torch.empty_like(w.kv)
    kv2[perm.to(DEV)] = w.kv
    w.kv = kv2
    w.block_table = perm.to(torch.int32).to(DEV)[w.block_table.long()]
    go2, gl2, _ = run_library(w)
    assert np.array_equal(go, go2) and np.array_equal(gl, gl2)


def test_sparse_small_edge_cases():
    _say("sparse small")
    w = make_sparse(4, 2, 64, pool_tokens_per_seq=640, topk=100, invalid_frac=0.1, seed=6, device=DEV)
    idx = w.indices.clone()
    idx[1, 0, :] = -1                                   # a row that sees nothing
    idx[2, 1, 3] = w.num_blocks * 64 + 9                # out of range: masked
    idx[3, 0, 10] = idx[3, 0, 11]                       # duplicate entry counts twice
    w.indices = idx
    go, gl, _ = run_library(w)
    ro, rl = oracle(w)
    assert np.isneginf(rl[1, :, 0]).all()
    _say(compare(go, gl, ro, rl))


def test_sparse_bf16_cache_past_4gib():
    """A 4.8 GB bf16 cache (2 requests x 2^21 tokens): gathered rows past the
    first 4 GiB are read through 64-bit addresses, not 32-bit buffer offsets."""
    from helpers import kv_host_rows
    _say("sparse bf16 > 4 GiB")
    w = make_sparse(2, 1, 128, pool_tokens_per_seq=1 << 21, topk=2048, invalid_frac=0.05, seed=71, device=DEV)
    idx = w.indices.cpu().numpy()
    assert int((idx.astype(np.int64) * 1152 >= (1 << 32)).sum()) > 100
    items = [(0, 0), (1, 0)]
    go, gl, _ = run_library(w)
    ro, rl = oracle(w, items=items, kv=kv_host_rows(w, items))
    _say(compare(go, gl, ro, rl, items=items))


def test_fp8_small():
    _say("fp8 small")
    w = make_fp8_dense(3, 1, 128, [70, 300, 1], seed=7, device=DEV)
    go, gl, _ = run_library(w)
    ro, rl = oracle(w)
    _say(compare(go, gl, ro, rl, rel_l2=FP8_REL_L2, max_abs=1e-2))


def test_fp8_sparse_small():
    _say("fp8 sparse small")
    w = make_sparse(2, 1, 128, pool_tokens_per_seq=1024, topk=300, invalid_frac=0.05, seed=8, device=DEV,
                    kv_format='fp8')
    go, gl, _ = run_library(w)
    ro, rl = oracle(w)
    _say(compare(go, gl, ro, rl, rel_l2=FP8_REL_L2, max_abs=1e-2))


# ------------------------------------------------------------------ combine entry point

def test_combine_standalone():
    import mla_decode_amd as mla
    _say("combine")
    g = torch.Generator().manual_seed(2)
    H, S_, B = 8, 2, 5
    # split counts include items with more splits than the kernel merges per
    # chunk (4), so that the running-maximum merge across chunks is exercised
    ns = [0, 1, 3, 2, 4, 1, 7, 9, 5, 12]
    so = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    T = int(so[-1])
    o = torch.randn(T, H, 512, generator=g)
    lse = torch.randn(T, H, generator=g) * 3
    lse[2, 1] = -float("inf")            # one empty split of item 2, one head
    lse[7, :] = -float("inf")            # one empty split of item 4
    lse[10, :] = -float("inf")           # item 5: its only split is empty
    lse[11:15, :] = -float("inf")        # item 6: the whole first chunk is empty
    lse[22:26, :] = -float("inf")        # item 7: the whole second chunk is empty
    lse[41, :] += 40.0                   # item 9: the maximum sits in its third chunk
    out = torch.empty(B, S_, H, 512, dtype=torch.float32, device=DEV)
    lo = torch.empty(B, H, S_, dtype=torch.float32, device=DEV)
    mla.combine(B * S_, H, S_, o.to(DEV), lse.to(DEV), torch.from_numpy(so).to(DEV), out, lo)
    torch.cuda.synchronize()
    for j in range(B * S_):
        b, i = divmod(j, S_)
        ro, rl = A.merge_partials(o[so[j]:so[j + 1]].double().numpy(), lse[so[j]:so[j + 1]].double().numpy())
        if ns[j] == 0:
            ro, rl = np.zeros((H, 512)), np.full(H, -np.inf)
        assert np.max(np.abs(out[b, i].cpu().numpy() - ro)) < 1e-5
        gl = lo[b, :, i].cpu().numpy()
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
        fin = np.isfinite(rl)
        assert np.all(np.abs(gl[fin] - rl[fin]) < 1e-5)


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_partial_hook_plus_combine_equals_decode(out_dtype):
    """mla_debug_decode_partial followed by mla_combine over its workspace
    gives what mla_decode_fwd gives, for a shape where every item is split (and
    for a sparse one).  With an fp32 output both paths merge the same float32
    partials, so the results are bit-identical.  With a bf16 output the decode
    call merges float16 partials (scaled per lane by a power of two) while the
    test hook leaves float32 ones: the lse is still identical (float32 in both),
    and each output differs by at most one bf16 step plus 2^-11 of the largest
    magnitude among the item's partials of that head (the float16 rounding of a
    partial scaled into [-1, 1))."""
    import mla_decode_amd as mla
    _say(f"partial hook {out_dtype}")
    for w in (make_dense(4, 1, 128, [4096, 4000, 3001, 2048], pool_blocks=300, seed=31, device=DEV,
                         out_dtype=out_dtype),
              make_sparse(3, 1, 128, pool_tokens_per_seq=8192, topk=2048, seed=32, device=DEV,
                          out_dtype=out_dtype)):
        dec = mla.Decoder.for_workload(w, DEV)
        dec.metadata(None if w.topk else w.cache_seqlens)
        out1, lse1 = dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices)
        out1, lse1 = out1.clone(), lse1.clone()
        dec.out.zero_()
        dec.lse.zero_()
        dec.decode_partial(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices)
        m = dec.meta
        items = w.batch * w.s_q
        slots = m.max_splits
        ws = dec.workspace.view(torch.float32)
        o_part = ws[:slots * w.h_q * 512]
        lse_part = ws[slots * w.h_q * 512: slots * w.h_q * 513]
        so_off = 8 + 5 * m.num_partitions
        split_offsets = dec.meta_buf.view(torch.int32)[so_off: so_off + items + 1]
        nsplit = (split_offsets[1:] - split_offsets[:-1]).cpu()
        assert bool((nsplit > 1).all()), nsplit
        out2 = torch.empty_like(out1)
        lse2 = torch.empty_like(lse1)
        mla.combine(items, w.h_q, w.s_q, o_part, lse_part, split_offsets, out2, lse2)
        torch.cuda.synchronize()
        assert torch.equal(lse1, lse2)
        if out_dtype == "fp32":
            assert torch.equal(out1, out2)
        else:
            # |float16 error| <= 2^-12 2^E <= 2^-11 of the largest magnitude among the
            # item's partials (per head); the two bf16 roundings then land at most
            # one bf16 step (2^-7 |x|) apart
            a, b = out1.float(), out2.float()
            parts = o_part.view(slots, w.h_q, 512).abs().amax(dim=-1)      # [slots, H]
            so = split_offsets.cpu().tolist()
            pmax = torch.stack([parts[so[j]:so[j + 1]].amax(dim=0) for j in range(items)])   # [items, H]
            pmax = pmax.view(w.batch, w.s_q, w.h_q, 1)
            bound = 2.0 ** -7 * b.abs() + 2.0 ** -11 * pmax + 1e-7
            assert bool(((a - b).abs() <= bound).all()), float(((a - b).abs() - bound).max())
            _say(f"bf16 outputs differing: {float((a != b).float().mean()):.4f}")


# ------------------------------------------------------------------ full-size workloads (whole tensors)

def _whole(w, **kw):
    """Every output element and lse of a full-size workload against the
    oracle, with the literal max-abs bound (no magnitude-relative slack)."""
    go, gl, dec = run_library(w)
    ro, rl = oracle(w)
    stats = compare(go, gl, ro, rl, max_abs_rel=0.0, **kw)
    assert float(np.max(np.abs(go - ro))) <= kw.get("max_abs", 1e-2)
    assert np.all(np.isfinite(gl))
    return stats


def test_config2_whole():
    _say("config2 b=64 s_q=1 h_q=128 seqlen=4096 bf16")
    _say(_whole(make_config(2, device=DEV)))


def test_config3_whole():
    _say("config3 b=128 s_q=2 causal h_q=128 seqlen U[1,8192] bf16")
    w = make_config(3, device=DEV)
    lens = w.cache_seqlens.cpu().numpy()
    _say("lens min/median/max", int(lens.min()), int(np.median(lens)), int(lens.max()))
    _say(_whole(w))


def test_config4_full():
    _say("config4")
    w = make_config(4, device=DEV)
    go, gl, _ = run_library(w)
    ro, rl = oracle(w)
    _say(compare(go, gl, ro, rl, max_abs_rel=0.0))


def test_config5_whole():
    _say("config5 b=32 s_q=1 h_q=128 seqlen=16384 fp8 cache")
    _say(_whole(make_config(5, device=DEV), rel_l2=FP8_REL_L2, max_abs=1e-2))


# ------------------------------------------------------------------ peaked rows: top-k order invariance

def _row_gain(x, ref):
    num = np.sum((x - ref) * ref, axis=-1)
    den = np.sum(ref * ref, axis=-1)
    return num / den


def test_peaked_topk_order_invariance():
    """Self token in slot 0 vs moved last (the Exact-max note's order test).

    The note's criterion -- the difference of the two orders' outputs is no
    more coherent than rounding noise (<= 2x) and each order's row gain stays
    within 2x of the ideal bf16 output floor -- concerns a forward pass whose
    rows are computed whole.  It is checked here with one partition per
    request, so that no split merge adds rounding of its own.  At the default
    launch every request of this 8-request workload is split over many
    partitions; the merge of the float16 partials then rounds differently for
    the two orders (which tokens share a partition changes), so there both
    orders are held to element-wise parity and to the per-order row-gain bound.
    """
    outs = {"whole": {}, "default": {}}
    ref = None
    for order in ("asis", "self_last"):
        _say(f"peaked order={order}")
        w = make_sparse(8, 1, 128, pool_tokens_per_seq=8192, topk=2048, invalid_frac=0.05, seed=21, device=DEV,
                        peaked=True, order=order)
        ro, rl = oracle(w)
        go, gl, dec = run_library(w)
        compare(go, gl, ro, rl)
        outs["default"][order] = go[:, 0]
        # one partition per request: as many compute units as requests times head blocks
        go, gl, dec = run_library(w, num_cus=8 * dec.meta.num_head_blocks)
        assert dec.meta.num_partitions == 8
        compare(go, gl, ro, rl)
        outs["whole"][order] = go[:, 0]
        if ref is None:
            ref = ro[:, 0]
        else:
            assert np.max(np.abs(ro[:, 0] - ref)) < 1e-9
    ideal = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    floor = np.sqrt(np.mean(_row_gain(ideal, ref) ** 2))
    for launch, o2 in outs.items():
        for order, o in o2.items():
            g = np.sqrt(np.mean(_row_gain(o, ref) ** 2))
            _say(f"{launch} {order}: row-gain rms {g:.3e} vs ideal floor {floor:.3e}")
            assert g <= 2.0 * floor
        d = o2["asis"] - o2["self_last"]
        coh = np.sqrt(np.mean(_row_gain(ref + d, ref) ** 2))
        noise = np.sqrt(np.mean((np.linalg.norm(d, axis=-1) / np.linalg.norm(ref, axis=-1) / np.sqrt(512)) ** 2))
        _say(f"{launch}: difference coherence {coh:.3e} vs noise {noise:.3e}")
        if launch == "whole":
            assert coh <= 2.0 * max(noise, 1e-12)
