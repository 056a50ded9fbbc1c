"""GPU parity of the prefill indexer (csa2_index_prefill) against the CPU oracle.

Each prefill query i at position t = q_pos0 + i runs the Full-mode steps on its causal
prefix; pools and top-k sets must be bit-identical to the oracle's.  The shapes span
several query tiles (128 queries) and position chunks (2048 positions) with ragged tails,
queries starting at position 0, and head layouts with fewer than four 32-groups per head.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_harness import GpuState, index_prefill, prefill_q
from harness import OracleState, make_table

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _first_diff(a, b, n=5):
    idx = np.argwhere(a != b)[:n]
    return [(tuple(i), a[tuple(i)], b[tuple(i)]) for i in idx]


def _oracle_q(wl, n_q, scale_fn=None, w=None):
    q = si.prefill_idx_q(wl, 0, n_q)
    if scale_fn is not None:
        scale_fn(q)
    qc, qs = oracle.quantize_mxfp4(q.reshape(n_q, -1))
    return qc, qs, si.prefill_idx_w(wl, 0, n_q) if w is None else w


def _check(wl, n_q, permute=True, scale_fn=None, w=None):
    L = wl.ctx[0]
    q_pos0 = L - n_q
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=permute)
    o = OracleState(wl, table, nblk, with_latent=False)
    g = GpuState(wl, table, nblk, with_latent=False)
    qo = _oracle_q(wl, n_q, scale_fn, w)
    po, plo, to, tlo = oracle.index_prefill(o.cfg, *qo, q_pos0, o.idx, o.table[0])
    qc, qs, wg = prefill_q(wl, 0, n_q, scale_fn)
    if w is not None:
        wg = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    assert np.array_equal(_np(qc), qo[0]) and np.array_equal(_np(qs), qo[1])
    pg, plg, tg, tlg = index_prefill(g, qc, qs, wg, q_pos0)
    torch.cuda.synchronize()
    assert np.array_equal(_np(plg), plo), _first_diff(_np(plg), plo)
    assert np.array_equal(_np(pg), po), _first_diff(_np(pg), po)
    assert np.array_equal(_np(tlg), tlo), _first_diff(_np(tlg), tlo)
    assert np.array_equal(_np(tg), to), _first_diff(_np(tg), to)
    return po, plo, to, tlo


@pytest.mark.parametrize("H,d,L,n_q", [
    (8, 128, 2800, 300),   # 3 query tiles (ragged), 2 position chunks, partial last stage
    (8, 128, 4500, 129),   # one query past a tile boundary
    (4, 64, 700, 200),     # two groups per head
    (2, 32, 130, 130),     # one group per head; queries from position 0 (prefix of 1)
    (1, 128, 2100, 70),
])
def test_prefill_index_bit_exact(H, d, L, n_q):
    wl = si.small("pf", 100 + H + d + L, [L], H_I=H, d_I=d, K_blk=64, k=128, W=16)
    _check(wl, n_q)


def test_prefill_pool_covers_everything():
    # most prefixes have at most K_blk blocks: the pool is every visible block
    wl = si.small("pfcov", 120, [900], H_I=4, d_I=128, K_blk=128, k=300, W=16)
    _check(wl, 400, permute=False)


def test_prefill_wide_exponent_spans_take_the_exact_path():
    """Scales that spread more than 9 binades within a head vector force the per-group
    path of the matrix kernel; mixed-sign head weights exercise the fma chain's signs."""
    wl = si.small("pfspan", 121, [3000], H_I=8, d_I=128, K_blk=64, k=128, W=16)
    n_q = 260

    def keys_wide(x):
        blk = np.arange(x.shape[0]) // 8
        x[blk % 25 == 3, :, 0:32] *= np.float32(2.0 ** 11)   # group 0 of every head
        x[blk % 31 == 7, 2, 96:128] *= np.float32(2.0 ** -8)  # group 3 of head 2

    def q_wide(q):
        q[::5, :, 32:64] *= np.float32(2.0 ** 10)

    orig = si.idx_keys
    try:
        si.idx_keys = lambda w_, b, L=None: (lambda x: (keys_wide(x), x)[1])(orig(w_, b, L))
        w = si.uniform(121, 7, (n_q, wl.H_I), -1.5, 1.5)
        _check(wl, n_q, scale_fn=q_wide, w=w)
    finally:
        si.idx_keys = orig


@pytest.mark.slow
def test_prefill_workload_sampled():
    """The prefill workload at full size: 4096 queries at positions 258048..262143 of a
    262,144-token context, indexer 8 x 128, pool 2048 blocks, top-512.  Six queries are
    checked bit-exactly against the oracle; every query is checked for the properties
    that hold at any size (lengths, ascending order, top-k inside the pool, causality)."""
    wl = si.workload("prefill")
    n_q, L = wl.n_q, wl.ctx[0]
    q_pos0 = L - n_q
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    g = GpuState(wl, table, nblk, with_latent=False)
    qc, qs, wg = prefill_q(wl, 0, n_q)
    pg, plg, tg, tlg = index_prefill(g, qc, qs, wg, q_pos0)
    torch.cuda.synchronize()
    pg, plg, tg, tlg = _np(pg), _np(plg), _np(tg), _np(tlg)
    del g
    torch.cuda.empty_cache()
    assert np.all(plg == wl.K_blk) and np.all(tlg == wl.k)
    assert np.all(np.diff(pg, axis=1) > 0) and np.all(np.diff(tg, axis=1) > 0)
    t = q_pos0 + np.arange(n_q)
    assert np.all(tg[:, -1] <= t) and np.all(pg[:, -1] <= t // 8)
    assert all(np.isin(tg[i] // 8, pg[i]).all() for i in range(0, n_q, 97))
    o = OracleState(wl, table, nblk, with_latent=False)
    qo = _oracle_q(wl, n_q)
    for i in (0, 1, 127, 128, 2049, n_q - 1):
        ctx = np.array([q_pos0 + i + 1], np.int32)
        po, plo, to, tlo = oracle.index_full(o.cfg, qo[0][i:i + 1], qo[1][i:i + 1],
                                             qo[2][i:i + 1], o.idx, o.table, ctx)
        assert np.array_equal(pg[i], po[0]), (i, _first_diff(pg[i], po[0]))
        assert np.array_equal(tg[i], to[0]), (i, _first_diff(tg[i], to[0]))
