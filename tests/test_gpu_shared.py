"""GPU parity of the shared-key indexer variant (one d_I key per position scored by all H_I
query heads; the scan on the FP4 matrix cores) against the oracle's shared-key reading.

Bar: scores and block maxima bit-exact (including tiles whose scale spans force the
per-group exact path), pools and top-k bit-exact, attention within 2e-3, on small ragged
shapes, through the fused layer calls, and at the batch-8 64K size.
"""
import numpy as np
import pytest
import torch

import kv_cache_decode_csa2_amd as k
import oracle
import synth_inputs as si
from gpu_harness import GpuState
from harness import OracleState, make_table
from test_gpu_parity import _run_group
from test_gpu_timed_path import _timed_group

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _first_diff(a, b, n=5):
    idx = np.argwhere(a != b)[:n]
    return [(tuple(i), a[tuple(i)], b[tuple(i)]) for i in idx]


def _scores(wl, mixed=False, keys_fn=None, q_fn=None):
    table, nblk = make_table(wl.ctx, seed=wl.seed)
    orig_k, orig_q = si.idx_keys, si.layer_idx_q
    try:
        if keys_fn is not None:
            si.idx_keys = lambda w_, b, L=None: (lambda x: (keys_fn(x), x)[1])(orig_k(w_, b, L))
        if q_fn is not None:
            si.layer_idx_q = lambda w_, layer: (lambda x: (q_fn(x), x)[1])(orig_q(w_, layer))
        o = OracleState(wl, table, nblk, with_latent=False)
        g = GpuState(wl, table, nblk, with_latent=False)
        qo, qg = o.layer_q(0, mixed), g.layer_q(0, mixed)
    finally:
        si.idx_keys, si.layer_idx_q = orig_k, orig_q
    assert np.array_equal(_np(g.idx), o.idx)
    sc, bs = g.index_scores(*qg)
    sc, bs = _np(sc), _np(bs)
    for b, L in enumerate(wl.ctx):
        ref = oracle.index_scores(o.cfg, qo[0][b], qo[1][b], qo[2][b], o.idx, o.table[b], L)
        got = sc[b, :L]
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (b, _first_diff(got, ref))
        rb = oracle.block_scores(ref, L)
        assert np.array_equal(bs[b, :len(rb)].view(np.uint32), rb.view(np.uint32)), b
    return o, g


@pytest.mark.parametrize("H,d,mixed", [(8, 128, False), (4, 64, False), (1, 32, False),
                                       (2, 64, True), (8, 32, True), (4, 128, False)])
def test_shared_scores_bit_exact(H, d, mixed):
    wl = si.small("shsc", 500 + H + d, [1000, 333, 9, 4096, 1], H_I=H, d_I=d, K_blk=16, k=40,
                  shared_key=True)
    _scores(wl, mixed)


def test_shared_wide_spans_take_the_exact_path():
    """Key groups scaled by 2^12 in one block of five and query groups scaled by 2^10 for
    some heads put the scale span of those items past 9, so the matrix kernel must take one
    product per group there and add the groups in order; mixed-sign head weights."""
    wl = si.small("shspan", 510, [3000, 700], H_I=8, d_I=128, K_blk=16, k=40, shared_key=True)

    def keys_wide(x):
        blk = np.arange(x.shape[0]) // 8
        x[blk % 5 == 1, :, 0:32] *= np.float32(2.0 ** 12)
        x[blk % 7 == 3, :, 96:128] *= np.float32(2.0 ** -9)

    def q_wide(q):
        q[:, 2, 32:64] *= np.float32(2.0 ** 10)

    _scores(wl, True, keys_wide, q_wide)


@pytest.mark.parametrize("H,d", [(8, 128), (4, 64)])
def test_shared_group_small_shapes(H, d):
    """Full, Reindex and Reuse layers on the shared-key variant (ragged batch, pool and
    top-k bit-exact, attention within 2e-3)."""
    wl = si.small("shgrp", 520 + H, [0, 5, 64, 130, 1000, 2049, 9000], H_I=H, d_I=d, K_blk=16,
                  k=40, W=32, layers="FRURU", shared_key=True)
    print(_run_group(wl))


def test_shared_timed_group_small():
    """The bench's step (fused layer calls) on a shared-key workload against the oracle."""
    wl = si.small("shtg", 530, [4097, 9, 20000], H_I=8, d_I=128, K_blk=64, k=128, H_q=64,
                  layers="FRURU", shared_key=True)
    print(_timed_group(wl))


@pytest.mark.slow
def test_shared_timed_group_b8_64k():
    print(_timed_group(si.workload("b8_64k_shared")))


def test_shared_prefill_is_refused():
    wl = si.small("shpf", 540, [300], H_I=8, d_I=128, K_blk=16, k=40, shared_key=True)
    table, nblk = make_table(wl.ctx, seed=wl.seed)
    g = GpuState(wl, table, nblk, with_latent=False)
    qc, qs, w = g.layer_q(0)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    with pytest.raises(k.Csa2Error) as e:
        k.csa2_index_prefill(g.cfg, qc, qs, w, 299, g.idx, g.n_blocks, g.table[0].contiguous(),
                             torch.empty((1, 16), **i32), torch.empty(1, **i32),
                             torch.empty((1, 40), **i32), torch.empty(1, **i32), ws)
    assert e.value.status == k.CSA2_ERR_UNSUPPORTED
