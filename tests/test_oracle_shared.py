"""Pins of the oracle's shared-key indexer reading (one d_I key per position, scored by
all H_I query heads: s(p) = sum_h w_h ReLU(q_h . k_p) in the fixed fp32 order of the
per-head score, query head h's group j meeting the key's group j).

* exact rational arithmetic (fractions.Fraction) on dequantised values: equal where every
  fp32 step is exact, within the fp32 rounding bound on N(0,1) data;
* the shared key is the per-head reading with the key replicated into every head: both
  oracle paths give the same bits (a wrong key-group index, or a key read per head from a
  cache that holds one key, fails this);
* the cache layout, byte by byte, from offsets computed by hand;
* the hierarchical selection over shared-key scores equals brute force of its definition.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth_inputs as si
from harness import hierarchical_topk, make_table

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _cfg(H, d, shared=True, K_blk=4, k=8):
    return oracle.cfg(H, d, 512, 16, 128, K_blk, k, 1.0 / np.sqrt(512), shared_key=shared)


def _pack(c, keys):
    """keys fp32 [L, KH, d] -> (table, idx cache) over a permuted block table."""
    L = keys.shape[0]
    table, n_blocks = make_table([L], seed=L + 3)
    _, idx = oracle.alloc_caches(c, table, n_blocks)
    oracle.append_global(c, None, keys[None], table, np.array([0], np.int32), None, idx)
    return table, idx


def _grid_vectors(rng, shape, e_choices):
    """Values on the E2M1 grid times 2^e with one 6 * 2^e element per 32-group, so that the
    quantiser keeps exponent e and every value exactly."""
    v = rng.choice(GRID, shape) * rng.choice([-1.0, 1.0], shape)
    flat = v.reshape(-1, 32)
    e = rng.choice(e_choices, flat.shape[0])
    flat[:, 0] = 6.0 * rng.choice([-1.0, 1.0], flat.shape[0])
    flat *= (2.0 ** e)[:, None]
    return flat.reshape(shape).astype(np.float32)


def _exact(qv, kv, w):
    """qv [H, d], kv [L, d] exact values, w [H] -> exact rational shared-key scores."""
    out = []
    for p in range(kv.shape[0]):
        s = Fraction(0)
        for h in range(qv.shape[0]):
            dot = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv[h], kv[p]))
            s += Fraction(float(w[h])) * max(dot, Fraction(0))
        out.append(s)
    return out


@pytest.mark.parametrize("H,d", [(1, 32), (4, 64), (8, 128), (2, 96)])
def test_shared_score_exact_when_every_step_is_exact(H, d):
    rng = np.random.default_rng(7000 + H * 100 + d)
    c = _cfg(H, d)
    L = 19
    q = _grid_vectors(rng, (H, d), [-1])
    keys = _grid_vectors(rng, (L, 1, d), [-2])
    w = rng.choice([0.25, 0.5, 1.0, 2.0], H).astype(np.float32)
    qc, qs = oracle.quantize_mxfp4(q.reshape(1, -1))
    table, idx = _pack(c, keys)
    s = oracle.index_scores(c, qc[0], qs[0], w, idx, table[0], L)
    ex = _exact(q.astype(np.float64), keys[:, 0].astype(np.float64), w)
    for p in range(L):
        assert Fraction(float(s[p])) == ex[p], p


@pytest.mark.parametrize("H,d,mixed", [(8, 128, False), (4, 64, True)])
def test_shared_score_within_fp32_bound_on_normal_data(H, d, mixed):
    wl = si.small("shs", 71 + H, [37], H_I=H, d_I=d, shared_key=True)
    c = oracle.cfg_of(wl)
    keys = si.idx_keys(wl, 0)
    assert keys.shape == (37, 1, d)
    q = si.layer_idx_q(wl, 0)[0]
    w = si.layer_idx_w(wl, 0, mixed_sign=mixed)[0]
    qc, qs = oracle.quantize_mxfp4(q.reshape(1, -1))
    kc, ks = oracle.quantize_mxfp4(keys.reshape(37, -1))
    qv = oracle.dequant_mxfp4(qc, qs)[0].reshape(H, d)
    kv = oracle.dequant_mxfp4(kc, ks)
    table, idx = _pack(c, keys)
    s = oracle.index_scores(c, qc[0], qs[0], w, idx, table[0], 37)
    ex = _exact(qv, kv, w)
    for p in range(37):
        mag = sum(abs(float(w[h])) * max(0.0, float(np.dot(qv[h], kv[p]))) for h in range(H))
        dmax = max(abs(float(np.dot(qv[h], kv[p]))) for h in range(H))
        bound = (H + d // 32) * 2.0 ** -23 * (mag + sum(abs(w)) * dmax) + 1e-30
        assert abs(float(s[p]) - float(ex[p])) <= bound, p


@pytest.mark.parametrize("H,d", [(8, 128), (4, 64), (2, 32)])
def test_shared_key_equals_per_head_reading_with_replicated_key(H, d):
    """Storing the shared key once, or the same key once per head in a per-head cache, gives
    bit-identical scores, pools and top-k (mixed-sign weights, ragged tail)."""
    wl = si.small("shrep", 81 + H, [333], H_I=H, d_I=d, K_blk=8, k=20, shared_key=True)
    keys = si.idx_keys(wl, 0)                                  # [L, 1, d]
    q = si.layer_idx_q(wl, 0).reshape(1, -1)
    w = si.layer_idx_w(wl, 0, mixed_sign=True)
    qc, qs = oracle.quantize_mxfp4(q)
    c_sh, c_ph = _cfg(H, d, True, 8, 20), _cfg(H, d, False, 8, 20)
    t_sh, idx_sh = _pack(c_sh, keys)
    t_ph, idx_ph = _pack(c_ph, np.repeat(keys, H, axis=1))     # [L, H, d]
    assert idx_sh.shape[1] * H == idx_ph.shape[1]
    s_sh = oracle.index_scores(c_sh, qc[0], qs[0], w[0], idx_sh, t_sh[0], 333)
    s_ph = oracle.index_scores(c_ph, qc[0], qs[0], w[0], idx_ph, t_ph[0], 333)
    assert np.array_equal(s_sh.view(np.uint32), s_ph.view(np.uint32))
    ctx = np.array([333], np.int32)
    r_sh = oracle.index_full(c_sh, qc, qs, w, idx_sh, t_sh, ctx)
    r_ph = oracle.index_full(c_ph, qc, qs, w, idx_ph, t_ph, ctx)
    for a, b in zip(r_sh, r_ph):
        assert np.array_equal(a, b)


def test_shared_layout_by_hand():
    """d_I = 64 (two 32-groups), one key per position: a block is 8 x (32 + 2) = 272 bytes;
    the 16 code bytes of group g of the key in slot s sit at 16 * (g*8 + s) and its scale
    at 8*32 + s*2 + g."""
    c = _cfg(4, 64)
    assert oracle.idx_block_bytes(c) == 272
    rng = np.random.default_rng(9)
    keys = rng.standard_normal((21, 1, 64)).astype(np.float32)
    table, idx = _pack(c, keys)
    kc, ks = oracle.quantize_mxfp4(keys.reshape(21, 64))
    for p in range(21):
        blk = idx[table[0, p // 8]]
        s = p % 8
        for g in range(2):
            assert np.array_equal(blk[16 * (g * 8 + s):16 * (g * 8 + s) + 16], kc[p, 16 * g:16 * g + 16])
            assert blk[8 * 32 + s * 2 + g] == ks[p, g]


def test_shared_selection_equals_brute_force():
    wl = si.small("shsel", 91, [300, 1, 97], H_I=8, d_I=128, K_blk=6, k=17, shared_key=True)
    c = oracle.cfg_of(wl)
    table, n_blocks = make_table(wl.ctx, seed=91)
    _, idx = oracle.alloc_caches(c, table, n_blocks)
    for b in range(wl.B):
        oracle.append_global(c, None, si.idx_keys(wl, b)[None], table[b:b + 1],
                             np.array([0], np.int32), None, idx)
    q = si.layer_idx_q(wl, 0).reshape(wl.B, -1)
    qc, qs = oracle.quantize_mxfp4(q)
    w = si.layer_idx_w(wl, 0)
    pool, pl, topk, tl = oracle.index_full(c, qc, qs, w, idx, table, np.asarray(wl.ctx, np.int32))
    for b, L in enumerate(wl.ctx):
        sc = oracle.index_scores(c, qc[b], qs[b], w[b], idx, table[b], L)
        blocks, best = hierarchical_topk(sc, wl.K_blk, wl.k)
        assert np.array_equal(pool[b, :pl[b]], blocks), b
        assert np.array_equal(topk[b, :tl[b]], best), b
