"""The scheduler specification has no worked example on the pages (parity
unpinned by the pages); it is pinned here by an enumeration brute force of the
cost positions and by invariants every valid split must satisfy."""

import itertools

import numpy as np
import pytest

from oracle import sched as S


def brute(n, P, F):
    """Lay out every cost position explicitly and slice it into P parts."""
    pos = []
    for j, nj in enumerate(n):
        pos += [(j, None)] * F + [(j, t) for t in range(nj)]
    T = len(pos)
    q = max(1, -(-T // P))
    parts = [pos[p * q:(p + 1) * q] for p in range(P)]
    tiles = [[x for x in part if x[1] is not None] for part in parts]
    num_splits = [sum(1 for tp in tiles if any(x[0] == j for x in tp)) for j in range(len(n))]
    return q, T, tiles, num_splits


def check(n, P, F):
    sch = S.schedule(n, P, F)
    q, T, tiles, ns = brute(n, P, F)
    assert sch['q'] == q and sch['T'] == T
    assert sch['num_splits'].tolist() == ns
    segs = S.segments(sch, n)
    # per partition: the segments expand to exactly the brute-force tile list
    for p in range(P):
        got = [(j, t) for (pp, j, t0, t1, _) in segs if pp == p for t in range(t0, t1)]
        assert got == tiles[p], (n, P, F, p)
    # slots: each item's partitions, in order, take consecutive slots
    so = sch['split_offsets']
    for j in range(len(n)):
        mine = [(p, slot) for (p, jj, _, _, slot) in segs if jj == j]
        assert [s for _, s in mine] == list(range(so[j], so[j + 1]))
        assert [p for p, _ in mine] == sorted(p for p, _ in mine)
    # invariants
    covered = [(j, t) for (_, j, t0, t1, _) in segs for t in range(t0, t1)]
    assert sorted(covered) == [(j, t) for j in range(len(n)) for t in range(n[j])]
    nonempty = sum(1 for x in n if x > 0)
    assert so[-1] <= nonempty + P - 1 or so[-1] == 0
    words = S.metadata_words(sch, 1)
    assert words[0] == S.MAGIC and words.shape[0] == S.HEADER + S.REC * P + len(n) + 1


def test_exhaustive_tiny():
    for N in (1, 2, 3):
        for n in itertools.product(range(0, 4), repeat=N):
            for P in (1, 2, 3, 5, 8):
                for F in (0, 1, 2):
                    if sum(n) + N * F == 0:
                        continue
                    check(list(n), P, F)


@pytest.mark.parametrize("seed", range(20))
def test_random_lengths(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 9))
    L = rng.integers(0, 301, size=N)       # cache lengths up to 300 -> 0..5 tiles
    s_q = int(rng.integers(1, 3))
    n = S.item_tiles_dense(L, s_q, causal=bool(rng.integers(0, 2)))
    check(n.tolist(), int(rng.integers(1, 9)), int(rng.integers(0, 3)))


def test_balance_on_config_shapes():
    """Every partition's cost is at most q, and q is the smallest equal share."""
    for n, P in [([64] * 64, 128), ([32] * 64, 256), ([256] * 32, 256)]:
        sch = S.schedule(n, P, 1)
        per = np.zeros(P, dtype=np.int64)
        for (p, j, t0, t1, _) in S.segments(sch, n):
            per[p] += t1 - t0
        assert per.max() <= sch['q'] and per.sum() == sum(n)


def test_causal_tiles():
    assert S.item_tiles_dense([1], 2, True).tolist() == [0, 1]
    assert S.item_tiles_dense([65], 2, True).tolist() == [1, 2]
    assert S.item_tiles_dense([64], 2, False).tolist() == [1, 1]
    assert S.item_tiles_sparse(2, 1, 2048).tolist() == [32, 32]
    assert S.item_tiles_sparse(1, 2, 100).tolist() == [2, 2]


def test_sparse_whole_item_rule():
    """The decode call skips the combine launch for a top-k problem when the
    partition size q is a multiple of the per-item cost.  Checked against the
    scheduler: the rule never fires when some item is split, and it does fire
    on the pages' FP8 sparse shapes (b=128, s_q=2, top-k 2048 and 32768, 256
    partitions), where every item is whole."""
    fired = 0
    for batch in (1, 2, 3, 5, 8, 64, 128):
        for s_q in (1, 2):
            for topk in (1, 63, 64, 100, 2048, 5000):
                for P in (1, 3, 8, 64, 256):
                    n = S.item_tiles_sparse(batch, s_q, topk)
                    sch = S.schedule(n, P, 0)
                    cost = int(n[0])
                    if sch['q'] % cost == 0:
                        fired += 1
                        assert (sch['num_splits'] == 1).all(), (batch, s_q, topk, P)
    assert fired > 50
    for topk in (2048, 32768):
        n = S.item_tiles_sparse(128, 2, topk)
        sch = S.schedule(n, 256, 0)
        assert sch['q'] % int(n[0]) == 0 and (sch['num_splits'] == 1).all()


@pytest.mark.parametrize("seed", range(8))
def test_sparse_topk_lengths(seed):
    """Per-query top-k lengths (clamped to [0, topk]) through the same
    brute-force check as dense lengths."""
    rng = np.random.default_rng(100 + seed)
    batch, s_q, topk = int(rng.integers(1, 5)), int(rng.integers(1, 3)), int(rng.integers(1, 300))
    lengths = rng.integers(-5, topk + 80, size=(batch, s_q))
    n = S.item_tiles_sparse(batch, s_q, topk, lengths)
    assert n.tolist() == [(min(max(int(x), 0), topk) + 63) // 64 for x in lengths.reshape(-1)]
    check(n.tolist(), int(rng.integers(1, 9)), int(rng.integers(0, 3)))
