"""mla_check_inputs: the host-side checks behind MLA_DEBUG=1.  The schedule
words come from the oracle's scheduler (the bit-exact target of the metadata
kernel), so a valid call passes; each planted fault (a stale schedule, a
broken record, a page or index out of range, a length out of range) is
reported with the offending entry."""

import numpy as np
import pytest

import mla_decode_amd as mla
from oracle import sched as S

P_CUS = 64


def _dense(seed=0, B=6, s_q=2, causal=True, NB=64, MB=8, num_cus=P_CUS):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, MB * 64 + 1, size=B).astype(np.int32)
    table = rng.integers(0, NB, size=(B, MB)).astype(np.int32)
    p = mla.make_problem(B, s_q, 128, NB, MB, causal=causal)
    m = mla.plan(p, num_cus=num_cus)
    n = S.item_tiles_dense(lens, s_q, causal)
    words = S.metadata_words(S.schedule(n, m.num_partitions, m.fixed_overhead), s_q).astype(np.int32)
    return p, m, words, lens, table


def _sparse(seed=0, B=4, s_q=2, topk=300, NB=16, with_len=True):
    rng = np.random.default_rng(seed)
    rows = NB * 64
    idx = rng.integers(-1, rows, size=(B, s_q, topk)).astype(np.int32)
    tl = rng.integers(0, topk + 1, size=(B, s_q)).astype(np.int32) if with_len else None
    p = mla.make_problem(B, s_q, 128, NB, topk=topk)
    m = mla.plan(p, num_cus=P_CUS)
    n = S.item_tiles_sparse(B, s_q, topk, tl)
    words = S.metadata_words(S.schedule(n, m.num_partitions, m.fixed_overhead), s_q).astype(np.int32)
    return p, m, words, idx, tl


def _fails(match, *a, **k):
    with pytest.raises(mla.MlaError, match=match) as e:
        mla.check_inputs(*a, **k)
    assert e.value.status == 1


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("causal", [False, True])
def test_valid_dense_passes(seed, causal):
    p, m, w, lens, table = _dense(seed, causal=causal)
    mla.check_inputs(p, m, w, lens, table)
    mla.check_inputs(p, None, None, lens, None)     # lengths only


@pytest.mark.parametrize("seed", range(3))
def test_valid_sparse_passes(seed):
    for with_len in (True, False):
        p, m, w, idx, tl = _sparse(seed, with_len=with_len)
        mla.check_inputs(p, m, w, None, idx, tl)


def test_stale_schedule_is_reported():
    p, m, w, lens, table = _dense(1)
    lens2 = lens.copy()
    lens2[0] = max(1, lens2[0] - 64)                  # one tile fewer than the schedule was made for
    _fails("stale metadata", p, m, w, lens2, table)


@pytest.mark.parametrize("fault,match", [
    ("magic", "magic"),
    ("header_P", "metadata header"),
    ("so_start", r"split_offsets\[0\]"),
    ("so_decrease", "split_offsets decrease"),
    ("rec_range", "outside the items' tiles"),
    ("rec_gap", "starts at tile|cover"),
    ("slot", "split slot"),
    ("splits", "splits"),
])
def test_broken_schedule_is_reported(fault, match):
    p, m, w, lens, table = _dense(2, B=8, s_q=1, causal=False, num_cus=16)   # 8 partitions of ~4 tiles
    P, N = m.num_partitions, p.batch * p.s_q
    recs = w[8:8 + 5 * P].reshape(P, 5)
    so = w[8 + 5 * P:8 + 5 * P + N + 1]
    full = [k for k in range(P) if recs[k, 0] < N and (recs[k, 0] < recs[k, 2] or recs[k, 1] < recs[k, 3])]
    k = full[len(full) // 2]
    if fault == "magic":
        w[0] ^= 1
    elif fault == "header_P":
        w[1] += 1
    elif fault == "so_start":
        so[0] = 1
    elif fault == "so_decrease":
        so[N // 2] = so[N // 2 + 1] + 1
    elif fault == "rec_range":
        recs[k, 3] = 10 ** 6
    elif fault == "rec_gap":                          # end one tile early: the next partition leaves a gap
        k = [k for k in full if recs[k, 3] >= 1 and (recs[k, 0] < recs[k, 2] or recs[k, 3] - 1 > recs[k, 1])][0]
        recs[k, 3] -= 1
    elif fault == "slot":
        recs[k, 4] += 1
    elif fault == "splits":
        so[N] += 1                                    # the last item claims a split no partition holds
    _fails(match, p, m, w, lens, table)


def test_dense_ranges():
    p, m, w, lens, table = _dense(3, causal=False)
    bad = lens.copy()
    bad[2] = p.max_blocks_per_seq * 64 + 1
    _fails(r"cache_seqlens\[2\]", p, None, None, bad, None)
    bad[2] = -1
    _fails(r"cache_seqlens\[2\]", p, None, None, bad, None)
    t = table.copy()
    t[1, 0] = p.num_blocks                            # first page of a row in use
    _fails(r"block_table\[1, 0\]", p, m, w, lens, t)
    t = table.copy()
    t[1, 0] = -3
    _fails(r"block_table\[1, 0\]", p, m, w, lens, t)
    # a page past the row's length is not read, so it is not checked
    short = lens.copy()
    short[4] = 64
    t = table.copy()
    t[4, 1:] = 10 ** 6
    mla.check_inputs(p, None, None, short, t)


def test_sparse_ranges():
    p, m, w, idx, tl = _sparse(4)
    b, i = 1, 1
    tl2 = tl.copy()
    tl2[b, i] = p.topk + 1
    _fails(r"topk_length\[3\]", p, None, None, None, None, tl2)
    j = tl[b, i] - 1 if tl[b, i] > 0 else 0
    bad = idx.copy()
    tl3 = tl.copy()
    tl3[b, i] = max(tl[b, i], 1)
    bad[b, i, max(j, 0)] = p.num_blocks * 64        # one past the last row
    _fails(r"indices\[3, ", p, None, None, None, bad, tl3)
    bad[b, i, max(j, 0)] = -2
    _fails(r"indices\[3, ", p, None, None, None, bad, tl3)
    # entries past the token's top-k length are not read
    bad = idx.copy()
    tl4 = tl.copy()
    tl4[b, i] = 0
    bad[b, i, :] = 10 ** 6
    mla.check_inputs(p, None, None, None, bad, tl4)
    # prefill: the rows are the flat cache's s_kv
    _fails("indices", p, None, None, None, np.full_like(idx, 100), None, num_rows=50)


def test_plan_mismatch():
    p, m, w, lens, table = _dense(5)
    p2 = mla.make_problem(p.batch, p.s_q, 64, p.num_blocks, p.max_blocks_per_seq, causal=True)
    with pytest.raises(mla.MlaError) as e:
        mla.check_inputs(p2, m, w, lens, table)
    assert e.value.status == 4
