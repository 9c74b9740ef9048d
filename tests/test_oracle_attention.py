"""Pins of the fp64 decode oracle against facts that do not come from the
oracle itself: a second (loop-only) implementation, the streaming recurrence,
the split merge, the seesaw schedule, closed forms, the absorption identity
and invariances of the definition."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.numerics import bf16_bits_to_f64
from workloads import make_dense, make_sparse


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_numpy_matches_loop_bruteforce():
    rng = np.random.default_rng(1)
    for n in (1, 2, 7, 33):
        q = _rand(rng, 3, 10)
        K = _rand(rng, n, 10)
        V = K[:, :6]
        out, lse = A.attend(q, K, V, 0.37)
        for h in range(3):
            ob, lb = A.attend_bruteforce(q[h].tolist(), K.tolist(), V.tolist(), 0.37)
            assert np.max(np.abs(out[h] - np.array(ob))) < 1e-12
            assert abs(lse[h] - lb) < 1e-12


def test_online_recurrence_equals_two_pass():
    rng = np.random.default_rng(2)
    q = _rand(rng, 4, 12) * 3
    K = _rand(rng, 50, 12)
    V = _rand(rng, 50, 8)
    out, lse = A.attend(q, K, V, 0.5)
    for h in range(4):
        o2, l2 = A.attend_online(q[h], K, V, 0.5)
        assert np.max(np.abs(out[h] - o2)) < 1e-12
        assert abs(lse[h] - l2) < 1e-12


def _seesaw(q, K, V, scale, blk):
    """Two warpgroup-halves schedule: O split into O_L / O_R, two KV blocks
    per step, cross-scaled so that both halves end equal to online softmax."""
    D = V.shape[1]
    half = D // 2
    m = -np.inf
    oL = np.zeros(half)
    oR = np.zeros(D - half)
    l = 0.0
    n = K.shape[0]
    j = 0
    while j < n:
        K0, V0 = K[j:j + blk], V[j:j + blk]
        K1, V1 = K[j + blk:j + 2 * blk], V[j + blk:j + 2 * blk]
        p0 = scale * (K0 @ q)
        p1 = scale * (K1 @ q) if K1.shape[0] else np.zeros(0)
        mp0 = p0.max()
        mn0 = max(m, mp0)
        s0 = math.exp(m - mn0) if m != -np.inf else 0.0
        m = mn0
        p0 = np.exp(p0 - mn0)
        oL = oL * s0 + p0 @ V0[:, :half]
        mp1 = p1.max() if p1.size else -np.inf
        mn1 = max(m, mp1)
        s1 = math.exp(m - mn1)
        m = mn1
        p1 = np.exp(p1 - mn1)
        oR = oR * (s0 * s1) + (p1 @ V1[:, half:] if p1.size else 0.0)
        p0 = p0 * s1
        oR = oR + p0 @ V0[:, half:]
        oL = oL * s1 + (p1 @ V1[:, :half] if p1.size else 0.0)
        l = l * s0 * s1 + p0.sum() + p1.sum()
        j += 2 * blk
    return np.concatenate([oL, oR]) / l, m + math.log(l)


def test_seesaw_schedule_equals_two_pass():
    rng = np.random.default_rng(3)
    q = _rand(rng, 16) * 2
    K = _rand(rng, 8 * 13, 16)
    V = _rand(rng, 8 * 13, 10)
    out, lse = A.attend(q[None], K, V, 0.8)
    o2, l2 = _seesaw(q, K, V, 0.8, 8)
    assert np.max(np.abs(out[0] - o2)) < 1e-12
    assert abs(lse[0] - l2) < 1e-12


@pytest.mark.parametrize("cuts", [[0, 5, 40], [0, 1, 2, 3, 40], [0, 20, 20, 40], [0, 40]])
def test_merge_of_partials_equals_unsplit(cuts):
    rng = np.random.default_rng(4)
    q = _rand(rng, 5, 9)
    K = _rand(rng, 40, 9)
    V = _rand(rng, 40, 7)
    out, lse = A.attend(q, K, V, 0.6)
    os_, ls_ = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = A.attend(q, K[a:b], V[a:b], 0.6)
        os_.append(o)
        ls_.append(l)
    om, lm = A.merge_partials(np.stack(os_), np.stack(ls_))
    assert np.max(np.abs(om - out)) < 1e-12
    assert np.max(np.abs(lm - lse)) < 1e-12


def test_merge_all_empty_partials():
    o = np.zeros((3, 2, 4))
    lse = np.full((3, 2), -np.inf)
    om, lm = A.merge_partials(o, lse)
    assert np.all(om == 0) and np.all(np.isneginf(lm))


def test_closed_forms():
    rng = np.random.default_rng(5)
    K = _rand(rng, 9, 6)
    V = _rand(rng, 9, 4)
    # zero query: uniform weights -> mean of V, lse = ln n
    out, lse = A.attend(np.zeros((1, 6)), K, V, 1.0)
    assert np.max(np.abs(out[0] - V.mean(axis=0))) < 1e-14
    assert abs(lse[0] - math.log(9)) < 1e-14
    # single token: out = V0, lse = s0
    q = _rand(rng, 1, 6)
    out, lse = A.attend(q, K[:1], V[:1], 0.3)
    assert np.max(np.abs(out[0] - V[0])) < 1e-15
    assert abs(lse[0] - 0.3 * float(q[0] @ K[0])) < 1e-14
    # two tokens: logistic weights
    out, lse = A.attend(q, K[:2], V[:2], 0.3)
    s0, s1 = 0.3 * float(q[0] @ K[0]), 0.3 * float(q[0] @ K[1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.max(np.abs(out[0] - (w0 * V[0] + (1 - w0) * V[1]))) < 1e-14
    # a dominant score (gap >= 50) selects its value row
    K2 = np.zeros((5, 6))
    K2[3, 0] = 1.0
    q2 = np.zeros((1, 6))
    q2[0, 0] = 60.0
    out, lse = A.attend(q2, K2, V[:5], 1.0)
    assert np.max(np.abs(out[0] - V[3])) < 1e-20
    # no tokens: out 0, lse -inf
    out, lse = A.attend(q, K[:0], V[:0], 1.0)
    assert np.all(out == 0) and np.isneginf(lse[0])


def test_decode_closed_forms_through_the_page_table():
    """Worked example through ``decode``: one request whose two pages are 3 and
    1 of a 4-page pool, with 65 visible tokens, is rows 192..255 then row 64.
    A zero query then gives the mean of those rows' first 512 values and
    lse = ln 65.  With one visible token (row 192) the output is that row's
    first 512 values and lse is the scaled dot product over all 576 dims."""
    rng = np.random.default_rng(11)
    kv = torch.randn(4 * 64, 576, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    kv_bits = _bits(kv)
    kv64 = kv.double().numpy()
    table = np.array([[3, 1]])
    q = torch.zeros(1, 1, 2, 576, dtype=torch.bfloat16)
    out, lse = A.decode(_bits(q), kv_bits, 0.05, block_table=table, cache_seqlens=np.array([65]))
    rows = list(range(192, 256)) + [64]
    want = kv64[rows, :512].mean(axis=0)
    assert np.max(np.abs(out[0, 0, 0] - want)) < 1e-12
    assert np.max(np.abs(out[0, 0, 1] - want)) < 1e-12
    assert np.all(np.abs(lse[0, :, 0] - math.log(65)) < 1e-12)
    qr = torch.from_numpy(rng.standard_normal((1, 1, 2, 576))).to(torch.bfloat16)
    out, lse = A.decode(_bits(qr), kv_bits, 0.05, block_table=table, cache_seqlens=np.array([1]))
    q64 = qr.double().numpy()[0, 0]
    for h in range(2):
        assert np.max(np.abs(out[0, 0, h] - kv64[192, :512])) < 1e-15
        assert abs(lse[0, h, 0] - 0.05 * float(q64[h] @ kv64[192])) < 1e-12


def test_absorption_identity():
    """Non-absorbed MHA with per-head up-projections equals W^UV applied to the
    oracle run on the latent cache with the absorbed query."""
    rng = np.random.default_rng(6)
    H, dh, dc, dR, n = 4, 5, 16, 4, 6
    W_uk = _rand(rng, H, dh, dc)
    W_uv = _rand(rng, H, dh, dc)
    c = _rand(rng, n, dc)
    kR = _rand(rng, n, dR)
    qC = _rand(rng, H, dh)
    qR = _rand(rng, H, dR)
    scale = 1.0 / math.sqrt(dh + dR)
    lat = np.concatenate([c, kR], axis=1)                      # [n, dc+dR]
    for h in range(H):
        k = np.concatenate([c @ W_uk[h].T, kR], axis=1)        # [n, dh+dR]
        v = c @ W_uv[h].T                                      # [n, dh]
        qh = np.concatenate([qC[h], qR[h]])
        s = scale * (k @ qh)
        w = np.exp(s - s.max())
        ref = (w / w.sum()) @ v
        q_abs = np.concatenate([W_uk[h].T @ qC[h], qR[h]])     # absorbed query
        o_lat, _ = A.attend(q_abs[None], lat, lat[:, :dc], scale)
        got = W_uv[h] @ o_lat[0]
        assert np.max(np.abs(got - ref)) < 1e-12


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _dense_args(w):
    return dict(block_table=w.block_table.numpy(), cache_seqlens=w.cache_seqlens.numpy(), causal=w.causal)


def test_block_table_reshuffle_is_bitwise_invariant():
    w = make_dense(2, 1, 4, [150, 70], seed=3, max_blocks=3, pool_blocks=9)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    out, lse = A.decode(q, kv, w.softmax_scale, **_dense_args(w))
    # move every page to a new physical slot and remap the table
    perm = np.random.default_rng(0).permutation(9)
    kv_blocks = kv.reshape(9, 64, 576)
    new = np.empty_like(kv_blocks)
    new[perm] = kv_blocks
    table = perm[w.block_table.numpy()]
    out2, lse2 = A.decode(q, new.reshape(-1, 576), w.softmax_scale, block_table=table,
                          cache_seqlens=w.cache_seqlens.numpy())
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_sparse_slot_permutation_and_invalid_insertion():
    w = make_sparse(2, 1, 4, pool_tokens_per_seq=256, topk=40, invalid_frac=0.1, seed=5)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    idx = w.indices.numpy()
    out, lse = A.decode(q, kv, w.softmax_scale, indices=idx)
    perm = np.random.default_rng(1).permutation(40)
    out2, lse2 = A.decode(q, kv, w.softmax_scale, indices=idx[:, :, perm])
    assert np.max(np.abs(out2 - out)) <= 1e-12 * np.max(np.abs(out))
    assert np.max(np.abs(lse2 - lse)) < 1e-12
    # inserting invalid slots (-1 and out-of-range) anywhere changes nothing
    ins = np.insert(idx, [0, 7, 40], [-1, kv.shape[0] + 5, -7], axis=2)
    out3, lse3 = A.decode(q, kv, w.softmax_scale, indices=ins)
    assert np.array_equal(out3, out) and np.array_equal(lse3, lse)


def test_causal_row_equals_dense_with_shorter_length():
    w = make_dense(1, 3, 2, [130], causal=True, seed=9, max_blocks=3)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    out, lse = A.decode(q, kv, w.softmax_scale, **_dense_args(w))
    for i in range(3):
        Lp = 130 - 3 + 1 + i
        o2, l2 = A.decode(q[:, i:i + 1], kv, w.softmax_scale, block_table=w.block_table.numpy(),
                          cache_seqlens=np.array([Lp]))
        assert np.array_equal(out[:, i], o2[:, 0]) and np.array_equal(lse[:, :, i], l2[:, :, 0])


def test_causal_empty_row():
    w = make_dense(1, 2, 2, [1], causal=True, seed=2, max_blocks=1)
    out, lse = A.decode(_bits(w.q), _bits(w.kv).reshape(-1, 576), w.softmax_scale, **_dense_args(w))
    assert np.all(out[0, 0] == 0) and np.all(np.isneginf(lse[0, :, 0]))
    assert np.all(np.isfinite(out[0, 1])) and np.all(np.isfinite(lse[0, :, 1]))


def test_batch_independence():
    w = make_dense(3, 1, 2, [64, 100, 5], seed=4, max_blocks=2)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    out, lse = A.decode(q, kv, w.softmax_scale, **_dense_args(w))
    o1, l1 = A.decode(q[1:2], kv, w.softmax_scale, block_table=w.block_table.numpy()[1:2],
                      cache_seqlens=w.cache_seqlens.numpy()[1:2])
    assert np.array_equal(out[1:2], o1) and np.array_equal(lse[1:2], l1)


def test_peaked_rows_are_self_dominated():
    """The peaked construction gives the self token a median weight near the
    0.17 the sparse-MLA precision note reports for q = 0.25 k_self."""
    w = make_sparse(4, 1, 8, pool_tokens_per_seq=4096, topk=2048, invalid_frac=0.05, seed=11, peaked=True)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    weights = []
    for b in range(4):
        rows = A.sparse_rows(w.indices.numpy()[b, 0], kv.shape[0])
        K = bf16_bits_to_f64(kv[rows])
        s = w.softmax_scale * (bf16_bits_to_f64(q[b, 0]) @ K.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        weights.extend(p[:, 0].tolist())
    med = float(np.median(weights))
    assert 0.08 < med < 0.3


# ------------------------------------------------------------------ optional arguments: attn_sink, topk_length

def test_sink_is_a_zero_value_token():
    """The sink scaling exp(lse) / (exp(lse) + exp(sink)) equals attention with
    one extra key whose scaled score is the sink and whose value is 0 (an
    independent form of the same softmax); lse stays the sink-free one, and
    the extra-key lse is logaddexp(lse, sink)."""
    w = make_dense(2, 1, 6, [70, 9], seed=31, max_blocks=2)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    bt, sl = w.block_table.numpy(), w.cache_seqlens.numpy()
    sink = np.array([-3.0, 0.0, 1.5, 4.0, 9.0, -np.inf])
    out, lse = A.decode(q, kv, w.softmax_scale, block_table=bt, cache_seqlens=sl)
    outs, lses = A.decode(q, kv, w.softmax_scale, block_table=bt, cache_seqlens=sl, attn_sink=sink)
    assert np.array_equal(lses, lse)
    fin = np.isfinite(sink)
    for b in range(2):
        qh = bf16_bits_to_f64(q[b, 0])
        K = A.kv_values(kv, A.paged_rows(bt[b], int(sl[b])), 'bf16')
        # extra key k with scale * qh[h] . k = sink[h] for the finite sinks (least-norm solution)
        Qf = qh[fin]
        k = Qf.T @ np.linalg.solve(Qf @ Qf.T, sink[fin] / w.softmax_scale)
        assert np.max(np.abs(w.softmax_scale * Qf @ k - sink[fin])) < 1e-9
        o2, l2 = A.attend(qh, np.vstack([K, k]), np.vstack([K[:, :512], np.zeros((1, 512))]), w.softmax_scale)
        assert np.max(np.abs(outs[b, 0][fin] - o2[fin])) < 1e-10
        assert np.max(np.abs(l2[fin] - np.logaddexp(lse[b, fin, 0], sink[fin]))) < 1e-9
        # sink = -inf leaves the row exactly as without a sink
        assert np.array_equal(outs[b, 0][~fin], out[b, 0][~fin])


def test_sink_equal_to_lse_halves_the_output():
    w = make_dense(1, 1, 4, [100], seed=32, max_blocks=2)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    args = dict(block_table=w.block_table.numpy(), cache_seqlens=w.cache_seqlens.numpy())
    out, lse = A.decode(q, kv, w.softmax_scale, **args)
    outs, _ = A.decode(q, kv, w.softmax_scale, attn_sink=lse[0, :, 0], **args)
    assert np.max(np.abs(outs - 0.5 * out)) <= 1e-15 * np.max(np.abs(out))


def test_sink_on_an_empty_row():
    w = make_dense(1, 1, 4, [0], seed=33, max_blocks=1)
    out, lse = A.decode(_bits(w.q), _bits(w.kv).reshape(-1, 576), w.softmax_scale,
                        block_table=w.block_table.numpy(), cache_seqlens=w.cache_seqlens.numpy(),
                        attn_sink=np.array([0.0, 5.0, -5.0, -np.inf]))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_topk_length_equals_masking_the_tail():
    """A query token's top-k length L gives the same result as marking its
    entries from L on invalid (-1); L >= topk is the whole row, L <= 0 sees
    nothing."""
    w = make_sparse(2, 2, 4, pool_tokens_per_seq=256, topk=50, invalid_frac=0.1, seed=34)
    q = _bits(w.q)
    kv = _bits(w.kv).reshape(-1, 576)
    idx = w.indices.numpy()
    lengths = np.array([[17, 0], [50, 99]])
    out, lse = A.decode(q, kv, w.softmax_scale, indices=idx, topk_length=lengths)
    masked = idx.copy()
    for b in range(2):
        for i in range(2):
            masked[b, i, max(lengths[b, i], 0):] = -1
    out2, lse2 = A.decode(q, kv, w.softmax_scale, indices=masked)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    full, lfull = A.decode(q, kv, w.softmax_scale, indices=idx)
    assert np.array_equal(out[1, 0], full[1, 0]) and np.array_equal(out[1, 1], full[1, 1])
    assert np.all(out[0, 1] == 0) and np.all(np.isneginf(lse[0, :, 1]))
