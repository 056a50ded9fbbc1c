"""Pins of the oracle's hierarchical selection (pool of blocks, final top-k, Reindex,
prefill) against independent brute force written here in Python.

* Invariant A: when the pool can hold every block, the hierarchy equals a flat top-k.
* Invariant B: with block-max reduction and the (score desc, index asc) order,
  K_blk >= k makes Full's in-pool top-k equal the flat top-k at any context length.
* Special cases: all-equal scores pick the lowest positions; L <= k picks everything;
  L = 0 is empty.  Tie-heavy inputs exercise the lower-index tie-break.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from harness import OracleState, flat_topk, hierarchical_topk, make_table


def _state(wl, seed=0, permute=True):
    table, nblk = make_table(wl.ctx, seed=seed, permute=permute)
    return OracleState(wl, table, nblk, with_latent=False)


def _full(st, layer=0, mixed=False):
    qc, qs, w = st.layer_q(layer, mixed)
    pool, pl, topk, tl, bs = oracle.index_full(st.cfg, qc, qs, w, st.idx, st.table, st.ctx,
                                               want_block_scores=True)
    return (qc, qs, w), pool, pl, topk, tl, bs


def _scores(st, b, q):
    qc, qs, w = q
    return oracle.index_scores(st.cfg, qc[b], qs[b], w[b], st.idx, st.table[b], st.wl.ctx[b])


def _valid(arr, n):
    assert np.all(arr[n:] == -1)
    return arr[:n]


@pytest.mark.parametrize("ctx,K_blk,k", [([1], 4, 8), ([7], 4, 8), ([64], 8, 16),
                                         ([61], 8, 16), ([100, 3, 57], 16, 20)])
def test_pool_covering_all_blocks_equals_flat_topk(ctx, K_blk, k):
    wl = si.small("A", 21, ctx, H_I=2, d_I=64, K_blk=K_blk, k=k)
    st = _state(wl)
    q, pool, pl, topk, tl, bs = _full(st)
    for b, L in enumerate(ctx):
        nb = (L + 7) // 8
        assert nb <= K_blk
        assert list(_valid(pool[b], pl[b])) == list(range(nb))
        s = _scores(st, b, q)
        assert np.array_equal(_valid(topk[b], tl[b]), flat_topk(s, k))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("K_blk,k", [(4, 16), (6, 48), (3, 40)])
def test_hierarchy_matches_bruteforce(seed, K_blk, k):
    ctx = [int(v) for v in np.random.default_rng(seed).integers(1, 200, 3)]
    wl = si.small("H", 100 + seed, ctx, H_I=4, d_I=64, K_blk=K_blk, k=k)
    st = _state(wl, seed)
    q, pool, pl, topk, tl, bs = _full(st, mixed=(seed % 2 == 1))
    for b, L in enumerate(ctx):
        s = _scores(st, b, q)
        blocks, best = hierarchical_topk(s, K_blk, k)
        assert np.array_equal(_valid(pool[b], pl[b]), blocks)
        assert np.array_equal(_valid(topk[b], tl[b]), best)
        # block scores are the per-block maxima of the position scores
        nb = (L + 7) // 8
        for j in range(nb):
            assert bs[b, j] == s[8 * j:min(L, 8 * j + 8)].max()
        if K_blk >= k:  # invariant B
            assert np.array_equal(best, flat_topk(s, k))


def _tied_keys(wl):
    """Keys drawn from a 3-value alphabet so that many positions tie exactly."""
    rng = np.random.default_rng(wl.seed)
    L = wl.ctx[0]
    x = rng.choice([0.0, 1.0, -1.0], (L, wl.H_I, wl.d_I)).astype(np.float32)
    x[:, :, ::32] = 6.0  # pins every group's exponent so equal codes give equal scores
    return x


@pytest.mark.parametrize("seed", range(20))
def test_invariant_b_with_heavy_ties(seed):
    rng = np.random.default_rng(1000 + seed)
    L = int(rng.integers(30, 400))
    k = int(rng.integers(1, 60))
    K_blk = int(rng.integers((k + 7) // 8, k + 4))
    K_blk = max(K_blk, 1)
    wl = si.small("B", 1000 + seed, [L], H_I=2, d_I=32, K_blk=K_blk, k=k)
    table, nblk = make_table([L], seed)
    c = oracle.cfg_of(wl)
    kv, idx = oracle.alloc_caches(c, table, nblk)
    oracle.append_global(c, None, _tied_keys(wl)[None], table, np.array([0], np.int32), None, idx)
    qc, qs = oracle.quantize_mxfp4(_tied_keys(si.small("q", seed, [1], H_I=2, d_I=32)).reshape(1, -1))
    w = np.ones((1, 2), np.float32)
    pool, pl, topk, tl = oracle.index_full(c, qc, qs, w, idx, table, np.array([L], np.int32))
    s = oracle.index_scores(c, qc[0], qs[0], w[0], idx, table[0], L)
    assert len(np.unique(s)) < L // 2  # the input really is tie-heavy
    blocks, best = hierarchical_topk(s, K_blk, k)
    assert np.array_equal(_valid(pool[0], pl[0]), blocks)
    assert np.array_equal(_valid(topk[0], tl[0]), best)
    if K_blk >= k:
        assert np.array_equal(best, flat_topk(s, k))


def test_invariant_b_fails_without_its_premise():
    # with K_blk < k the pool can exclude flat winners: the hierarchy is a real restriction
    hits = 0
    for seed in range(30):
        wl = si.small("nB", 500 + seed, [256], H_I=2, d_I=64, K_blk=2, k=24)
        st = _state(wl, seed)
        q, pool, pl, topk, tl, bs = _full(st)
        s = _scores(st, 0, q)
        hits += not np.array_equal(_valid(topk[0], tl[0]), flat_topk(s, 24))
    assert hits > 0


def test_all_equal_scores_pick_lowest_indices():
    L, K_blk, k = 203, 5, 13
    wl = si.small("eq", 9, [L], H_I=2, d_I=32, K_blk=K_blk, k=k)
    c = oracle.cfg_of(wl)
    table, nblk = make_table([L], 9)
    kv, idx = oracle.alloc_caches(c, table, nblk)
    keys = np.ones((1, L, 2, 32), np.float32)
    oracle.append_global(c, None, keys, table, np.array([0], np.int32), None, idx)
    qc, qs = oracle.quantize_mxfp4(np.ones((1, 64), np.float32))
    pool, pl, topk, tl = oracle.index_full(c, qc, qs, np.ones((1, 2), np.float32), idx, table,
                                           np.array([L], np.int32))
    assert list(_valid(pool[0], pl[0])) == list(range(K_blk))
    assert list(_valid(topk[0], tl[0])) == list(range(k))


def test_short_and_empty_contexts():
    wl = si.small("short", 4, [0, 5, 130], H_I=2, d_I=64, K_blk=16, k=200)
    st = _state(wl)
    q, pool, pl, topk, tl, bs = _full(st)
    assert pl[0] == 0 and tl[0] == 0 and np.all(pool[0] == -1) and np.all(topk[0] == -1)
    assert list(_valid(topk[1], tl[1])) == list(range(5))
    assert list(_valid(topk[2], tl[2])) == list(range(128))  # pool of 16 blocks, k > 128


@pytest.mark.parametrize("seed", range(4))
def test_reindex_is_topk_inside_the_stored_pool(seed):
    ctx = [300, 77, 1000]
    wl = si.small("R", 40 + seed, ctx, H_I=4, d_I=64, K_blk=12, k=30)
    st = _state(wl, seed)
    q0, pool, pl, topk, tl, bs = _full(st, 0)
    qc, qs, w = st.layer_q(1, mixed_sign=(seed == 3))
    rk, rl = oracle.index_reindex(st.cfg, qc, qs, w, st.idx, st.table, st.ctx, pool, pl)
    for b, L in enumerate(ctx):
        s = _scores(st, b, (qc, qs, w))
        cand = [p for j in _valid(pool[b], pl[b]) for p in range(8 * j, min(L, 8 * j + 8))]
        best = sorted(sorted(cand, key=lambda p: (-float(s[p]), p))[:30])
        assert list(_valid(rk[b], rl[b])) == best
    # Reindex with the Full layer's own query reproduces Full's final selection
    rk0, rl0 = oracle.index_reindex(st.cfg, *q0, st.idx, st.table, st.ctx, pool, pl)
    assert np.array_equal(rk0, topk) and np.array_equal(rl0, tl)


def test_prefill_query_equals_decode_on_its_prefix():
    L = 400
    wl = si.small("P", 8, [L], H_I=2, d_I=64, K_blk=6, k=20)
    st = _state(wl)
    n_q, pos0 = 12, L - 12
    q = si.normal(8, 999, (n_q, 2 * 64))
    qc, qs = oracle.quantize_mxfp4(q)
    w = si.uniform(8, 998, (n_q, 2), 0.5, 1.5)
    pool, pl, topk, tl = oracle.index_prefill(st.cfg, qc, qs, w, pos0, st.idx, st.table[0])
    for i in range(n_q):
        t = pos0 + i
        s = oracle.index_scores(st.cfg, qc[i], qs[i], w[i], st.idx, st.table[0], t + 1)
        blocks, best = hierarchical_topk(s, 6, 20)
        assert np.array_equal(_valid(pool[i], pl[i]), blocks)
        assert np.array_equal(_valid(topk[i], tl[i]), best)


def test_planted_blocks_are_found():
    wl = si.small("plant", 3, [8192], H_I=4, d_I=64, K_blk=32, k=64, planted=8)
    st = _state(wl)
    q, pool, pl, topk, tl, bs = _full(st)
    planted = si.planted_blocks(wl, 0)
    assert set(planted) <= set(_valid(pool[0], pl[0]))
    want = sorted(int(j) * 8 + s for j in planted for s in range(8))
    assert list(_valid(topk[0], tl[0])) == want
