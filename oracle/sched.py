"""Split-KV tile-scheduler specification (reference implementation).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages state only what the scheduler is for: FlashMLA's tile scheduler
hands requests and KV blocks to SMs so that every SM gets an equal load (new
kernel deep dive, "Other performance improvements"), its metadata is computed
once per decode step and reused by every layer, and reusing it after the shapes
change silently produces a wrong split ("matrices, attention & GPU" explainer,
section on split-KV; FlashMLA README, "Usage").  No algorithm is given, so the
algorithm below is ours; its parity is *unpinned by the pages* and is pinned
by invariants and by an enumeration brute force in the tests instead.

Specification (all integer arithmetic, no floating point):

S0  A work item is one query token of one request: item j = b*s_q + i.  It
    owns h_q query rows and n_j KV tiles of 64 tokens: dense
    n_j = ceil(visible_j / 64) with visible_j the causal-visible length;
    sparse n_j = ceil(topk / 64).
S1  cost_j = n_j + F, where F >= 0 is a fixed per-item overhead.
S2  C_j = exclusive prefix sum of cost, T = sum(cost), q = ceil(T / P)
    (q = 1 if T = 0).
S3  Partition p covers the cost interval [p*q, min((p+1)*q, T)).  A cost
    position x inside item j (C_j <= x < C_j + cost_j) stands for KV tile
    max(0, x - C_j - F) of item j; the first F positions of an item are
    overhead and carry no tile of their own.
S4  Partition p's record is (begin_item, begin_tile, end_item, end_tile,
    first_split_slot).  (begin_item, begin_tile) is the position lo = p*q
    mapped by S3; (end_item, end_tile) is j(hi-1) and
    clamp(hi - C_end - F, 0, n_end) with hi = min((p+1)*q, T).  The partition
    processes, for each item j from begin_item to end_item, the tiles
    [j == begin_item ? begin_tile : 0, j == end_item ? end_tile : n_j).
    An empty partition (lo >= hi) has the record (N, 0, N, 0, 0).
S5  num_splits[j] = number of partitions holding a non-empty tile range of
    item j = floor((C_j+F+n_j-1)/q) - floor((C_j+F)/q) + 1 if n_j > 0 else 0;
    split_offsets is its exclusive prefix sum (length N+1).  The split slot
    of partition p in item j is split_offsets[j] + p - floor((C_j+F)/q);
    first_split_slot is that slot for begin_item (0 when the partition holds
    no tile of begin_item); every later item of the partition starts at its
    tile 0, so its slot is split_offsets[j].
S6  Only integer arithmetic; every (item, tile) pair lands in exactly one
    partition, so there are no ties to break.

Metadata buffer (int32), the exact layout the device writes:
    [0..7]   header: MAGIC, P, N, F, q, T, s_q, total_tiles
    [8 .. 8+5P)           P records of 5 int32
    [8+5P .. 8+5P+N+1)    split_offsets
"""

import numpy as np

MAGIC = 0x4D4C4131          # 'MLA1'
HEADER = 8
REC = 5
BLOCK = 64


def visible_len(L, s_q, i, causal):
    """KV tokens visible to query token i of a request with cache length L.

    Reading (the pages give no causal rule for s_q > 1): the cache already holds
    the s_q new tokens, and query i sees the first L - s_q + 1 + i of them.
    """
    if not causal:
        return int(L)
    return int(min(max(int(L) - s_q + 1 + i, 0), int(L)))


def item_tiles_dense(cache_seqlens, s_q, causal):
    out = []
    for L in np.asarray(cache_seqlens).tolist():
        for i in range(s_q):
            v = visible_len(L, s_q, i, causal)
            out.append((v + BLOCK - 1) // BLOCK)
    return np.asarray(out, dtype=np.int64)


def item_tiles_sparse(batch, s_q, topk, topk_length=None):
    """Tiles per item of a top-k problem: all topk entries, or each query
    token's top-k length clamped to [0, topk]."""
    if topk_length is None:
        return np.full(batch * s_q, (int(topk) + BLOCK - 1) // BLOCK, dtype=np.int64)
    n = np.clip(np.asarray(topk_length, dtype=np.int64).reshape(-1), 0, int(topk))
    assert n.shape[0] == batch * s_q
    return (n + BLOCK - 1) // BLOCK


def schedule(n, P, F):
    """Apply S1-S6 to per-item tile counts ``n`` with P partitions."""
    n = np.asarray(n, dtype=np.int64)
    N = int(n.shape[0])
    P = int(P)
    F = int(F)
    assert N >= 1 and P >= 1 and F >= 0
    cost = n + F
    C = np.zeros(N + 1, dtype=np.int64)
    C[1:] = np.cumsum(cost)
    T = int(C[N])
    q = max(1, -(-T // P))

    def item_of(x):  # last j with C_j <= x, for 0 <= x < T
        return int(np.searchsorted(C[:N], x, side='right') - 1)

    num_splits = np.zeros(N, dtype=np.int64)
    first_part = np.zeros(N, dtype=np.int64)
    for j in range(N):
        first_real = int(C[j]) + F
        first_part[j] = first_real // q
        if n[j] > 0:
            num_splits[j] = (first_real + int(n[j]) - 1) // q - first_real // q + 1
    split_offsets = np.zeros(N + 1, dtype=np.int64)
    split_offsets[1:] = np.cumsum(num_splits)

    records = np.zeros((P, REC), dtype=np.int64)
    for p in range(P):
        lo = p * q
        hi = min((p + 1) * q, T)
        if lo >= hi:
            records[p] = (N, 0, N, 0, 0)
            continue
        jb = item_of(lo)
        tb = max(0, lo - int(C[jb]) - F)
        je = item_of(hi - 1)
        te = min(max(0, hi - int(C[je]) - F), int(n[je]))
        first_end = te if je == jb else int(n[jb])
        slot0 = int(split_offsets[jb] + p - first_part[jb]) if tb < first_end else 0
        records[p] = (jb, tb, je, te, slot0)

    header = np.array([MAGIC, P, N, F, q, T, 0, int(n.sum())], dtype=np.int64)
    return {
        'header': header, 'records': records, 'split_offsets': split_offsets,
        'num_splits': num_splits, 'q': q, 'T': T, 'C': C,
    }


def segments(sched, n):
    """Expand records into the list of (partition, item, t0, t1, slot) segments."""
    n = np.asarray(n, dtype=np.int64)
    N = n.shape[0]
    so = sched['split_offsets']
    out = []
    for p, (jb, tb, je, te, slot0) in enumerate(sched['records'].tolist()):
        for j in range(jb, min(je, N - 1) + 1):
            t0 = tb if j == jb else 0
            t1 = te if j == je else int(n[j])
            if t0 >= t1:
                continue
            slot = slot0 if j == jb else int(so[j])
            out.append((p, j, t0, t1, slot))
    return out


def metadata_words(sched, s_q):
    """The int32 metadata buffer the device is expected to write."""
    h = sched['header'].copy()
    h[6] = s_q
    words = np.concatenate([h, sched['records'].reshape(-1), sched['split_offsets']])
    assert words.max() < 2 ** 31 and words.min() >= -(2 ** 31)
    return words.astype(np.int32)
