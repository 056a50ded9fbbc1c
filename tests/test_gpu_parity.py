"""GPU parity: every step of the HIP path against the CPU oracle on the same seeded inputs.

Bar: packed bytes, dequantised values, scores, block scores and index sets bit-exact;
attention within 2e-3 of the fp64 oracle per (sequence, head) row (max_d |o - r| over
max_d |r|) and 2e-3 * max(1, |lse|) on the log-sum-exp.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_harness import GpuState, attn_close, dev
from harness import OracleState, make_table

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _first_diff(a, b, n=5):
    idx = np.argwhere(a != b)[:n]
    return [(tuple(i), a[tuple(i)], b[tuple(i)]) for i in idx]


# ------------------------------------------------------------------ codecs

def _special_inputs(rng, e_max=120):
    grid = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0,
                     5.5, 6.0, 7.0, 7.99], np.float32)
    rows = []
    for e in (-130, -126, -20, -2, 0, 3, 60, e_max):
        g = np.concatenate([[7.5], rng.choice(grid, 31) * rng.choice([-1.0, 1.0], 31)])
        rows.append((g * np.float64(2.0) ** e).astype(np.float32))
    rows.append(np.zeros(32, np.float32))
    z = np.zeros(32, np.float32)
    z[3] = -0.0
    z[5] = -1e-40
    rows.append(z)
    rows.append(np.full(32, 1e-42, np.float32))
    rows.append(np.array([3e38] + [-1e-3] * 31, np.float32))
    return np.stack(rows)


def test_quantize_fp4_bit_exact():
    rng = np.random.default_rng(1)
    x = np.concatenate([_special_inputs(rng).reshape(-1, 64),
                        (rng.standard_normal((300, 64)) * 2.0 ** rng.integers(-20, 20, (300, 1))).astype(np.float32)])
    oc, os_ = oracle.quantize_mxfp4(x)
    gc = torch.empty(oc.shape, dtype=torch.uint8, device="cuda")
    gs = torch.empty(os_.shape, dtype=torch.uint8, device="cuda")
    import kv_cache_decode_csa2_amd as k
    k.csa2_quantize_mxfp4(dev(x), gc, gs)
    assert np.array_equal(_np(gs), os_), _first_diff(_np(gs), os_)
    assert np.array_equal(_np(gc), oc), _first_diff(_np(gc), oc)


def test_quantize_fp8_bit_exact():
    rng = np.random.default_rng(2)
    sp8 = _special_inputs(rng, e_max=100).astype(np.float64)
    big = np.abs(sp8[:, 0]) > 1e36          # inputs must stay finite
    sp8[~big, 0] = sp8[~big, 0] / 7.5 * 500.0
    sp8 = sp8.astype(np.float32)
    x = np.concatenate([sp8.reshape(-1, 64),
                        (rng.standard_normal((300, 64)) * 2.0 ** rng.integers(-20, 20, (300, 1))).astype(np.float32)])
    oc, os_ = oracle.quantize_mxfp8(x)
    import kv_cache_decode_csa2_amd as k
    gc = torch.empty(oc.shape, dtype=torch.uint8, device="cuda")
    gs = torch.empty(os_.shape, dtype=torch.uint8, device="cuda")
    k.csa2_quantize_mxfp8(dev(x), gc, gs)
    assert np.array_equal(_np(gs), os_), _first_diff(_np(gs), os_)
    assert np.array_equal(_np(gc), oc), _first_diff(_np(gc), oc)


def test_dequant_bit_exact():
    import kv_cache_decode_csa2_amd as k
    rng = np.random.default_rng(3)
    codes4 = np.tile(np.arange(256, dtype=np.uint8), 8).reshape(16, 128)
    scales = rng.integers(60, 200, (16, 8), dtype=np.uint8)
    ref4 = oracle.dequant_mxfp4(codes4, scales)
    out = torch.empty((16, 256), dtype=torch.float32, device="cuda")
    k.csa2_dequant_mxfp4(dev(codes4), dev(scales), out)
    assert np.array_equal(_np(out).astype(np.float64), ref4), _first_diff(_np(out).astype(np.float64), ref4)
    codes8 = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(8, 128)
    codes8[(codes8 & 0x7F) == 0x7F] = 0x00  # NaN codes are never produced
    s8 = rng.integers(60, 200, (8, 4), dtype=np.uint8)
    ref8 = oracle.dequant_mxfp8(codes8, s8)
    out8 = torch.empty((8, 128), dtype=torch.float32, device="cuda")
    k.csa2_dequant_mxfp8(dev(codes8), dev(s8), out8)
    assert np.array_equal(_np(out8).astype(np.float64), ref8), _first_diff(_np(out8).astype(np.float64), ref8)


# ------------------------------------------------------------------ caches and scores

def _pair(wl, with_latent=True, permute=True):
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=permute)
    return OracleState(wl, table, nblk, with_latent), GpuState(wl, table, nblk, with_latent)


def test_append_caches_bit_exact():
    wl = si.small("app", 50, [300, 77, 1029, 0, 8], H_I=4, d_I=64, K_blk=16, k=40, W=32)
    o, g = _pair(wl)
    assert np.array_equal(_np(g.idx), o.idx), _first_diff(_np(g.idx), o.idx)
    assert np.array_equal(_np(g.kv), o.kv), _first_diff(_np(g.kv), o.kv)
    for layer in (0, 1):
        assert np.array_equal(_np(g.layer_swa(layer)), o.layer_swa(layer))
        qo = o.layer_q(layer)
        qg = g.layer_q(layer)
        assert np.array_equal(_np(qg[0]), qo[0]) and np.array_equal(_np(qg[1]), qo[1])


@pytest.mark.parametrize("H,d,mixed", [(4, 64, False), (8, 128, False), (1, 32, False),
                                       (2, 64, True), (8, 32, True), (4, 128, False)])
def test_scores_bit_exact(H, d, mixed):
    wl = si.small("sc", 60 + H + d, [1000, 333, 9, 4096], H_I=H, d_I=d, K_blk=16, k=40)
    o, g = _pair(wl, with_latent=False)
    qo, qg = o.layer_q(0, mixed), g.layer_q(0, mixed)
    sc, bs = g.index_scores(*qg)
    sc, bs = _np(sc), _np(bs)
    for b, L in enumerate(wl.ctx):
        ref = oracle.index_scores(o.cfg, qo[0][b], qo[1][b], qo[2][b], o.idx, o.table[b], L)
        got = sc[b, :L]
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (b, _first_diff(got, ref))
        rb = oracle.block_scores(ref, L)
        assert np.array_equal(bs[b, :len(rb)].view(np.uint32), rb.view(np.uint32)), b


# ------------------------------------------------------------------ index + attention groups

def _run_group(wl, permute=True, with_attn=True, mixed_layers=()):
    o, g = _pair(wl, with_latent=with_attn, permute=permute)
    pool_o = pool_g = topk_o = topk_g = None
    report = []
    for li, mode in enumerate(wl.layers):
        mixed = li in mixed_layers
        if mode == "F":
            qo, qg = o.layer_q(li, mixed), g.layer_q(li, mixed)
            po, plo, to, tlo = oracle.index_full(o.cfg, *qo, o.idx, o.table, o.ctx)
            pg, plg, tg, tlg = g.index_full(*qg)
            assert np.array_equal(_np(plg), plo), (li, "pool_len")
            assert np.array_equal(_np(pg), po), (li, "pool", _first_diff(_np(pg), po))
            pool_o, pool_g = (po, plo), (pg, plg)
            topk_o, topk_g = (to, tlo), (tg, tlg)
        elif mode == "R":
            qo, qg = o.layer_q(li, mixed), g.layer_q(li, mixed)
            to, tlo = oracle.index_reindex(o.cfg, *qo, o.idx, o.table, o.ctx, *pool_o)
            tg, tlg = g.index_reindex(*qg, *pool_g)
            topk_o, topk_g = (to, tlo), (tg, tlg)
        assert np.array_equal(_np(topk_g[1]), topk_o[1]), (li, mode, "topk_len")
        assert np.array_equal(_np(topk_g[0]), topk_o[0]), (li, mode, "topk",
                                                           _first_diff(_np(topk_g[0]), topk_o[0]))
        if with_attn:
            qa = si.layer_attn_q(wl, li)
            swo, swg = o.layer_swa(li), g.layer_swa(li)
            ro, rl = oracle.sparse_attn(o.cfg, qa, o.kv, o.table, swo, o.C, o.ctx, *topk_o)
            go, gl = g.attn(g.attn_q(li), swg, *topk_g)
            ok, rel, lerr = attn_close(_np(go), _np(gl), ro, rl)
            report.append((li, mode, rel, lerr))
            assert ok, (li, mode, rel, lerr)
    return report


def test_group_small_shapes():
    wl = si.small("grp", 70, [0, 5, 64, 130, 1000, 2049, 9000], H_I=4, d_I=64, K_blk=16, k=40, W=32)
    print(_run_group(wl))


def test_group_pool_covers_everything_and_ties():
    # nb <= K_blk for most sequences: the hierarchy reduces to a flat top-k
    wl = si.small("cov", 71, [7, 100, 512, 513], H_I=2, d_I=64, K_blk=64, k=200, W=16)
    print(_run_group(wl, mixed_layers=(1,)))


def test_group_64_heads_and_wide_indexer():
    wl = si.small("h64", 72, [4000, 3000], H_I=8, d_I=128, K_blk=32, k=96, H_q=64, W=128,
                  layers="FRURU")
    print(_run_group(wl))


def test_group_tiny_workload():
    """The tiny decode workload at its full size: batch 1, 4096 positions, 4 x 64 indexer,
    pool 64 blocks, top-128, 16 heads, window 128; layers F, R, U."""
    print(_run_group(si.workload("tiny")))


@pytest.mark.slow
def test_group_long_1m_workload():
    """Batch 1, 1,048,576 positions, pool 2048 -> top-512, 64 planted blocks."""
    wl = si.workload("long_1m")
    print(_run_group(wl, permute=False))


@pytest.mark.slow
def test_group_b8_64k_workload():
    wl = si.workload("b8_64k")
    print(_run_group(wl, permute=False))


@pytest.mark.slow
def test_group_ragged64_workload():
    wl = si.workload("ragged64")
    print(_run_group(wl, permute=False))


def test_group_all_equal_keys_long():
    """Every position holds the same indexer key, so every score, block maximum and group
    maximum ties: the pool must be blocks 0..K_blk-1 and the top-k positions 0..k-1 (lower
    index first).  With more than 2048 tied groups this takes the streaming pool path."""
    wl = si.small("tie", 81, [140000], H_I=4, d_I=64, K_blk=2048, k=512, W=16)
    row = si.normal(81, 999, (1, wl.H_I, wl.d_I))
    orig = si.idx_keys
    try:
        si.idx_keys = lambda w, b, L=None: np.repeat(row, w.ctx[b] if L is None else L, axis=0)
        o, g = _pair(wl, with_latent=False)
        qo, qg = o.layer_q(0), g.layer_q(0)
        po, plo, to, tlo = oracle.index_full(o.cfg, *qo, o.idx, o.table, o.ctx)
    finally:
        si.idx_keys = orig
    assert np.array_equal(po[0], np.arange(2048)) and np.array_equal(to[0], np.arange(512))
    pg, plg, tg, tlg = g.index_full(*qg)
    assert np.array_equal(_np(pg), po) and np.array_equal(_np(plg), plo)
    assert np.array_equal(_np(tg), to) and np.array_equal(_np(tlg), tlo)
    tg2, tlg2 = g.index_reindex(*qg, pg, plg)
    assert np.array_equal(_np(tg2), to)


@pytest.mark.parametrize("ahead,kk,W", [(0, 40, 32), (3, 40, 32), (0, 450, 100), (3, 450, 100)])
def test_fused_window_append_matches_two_calls(ahead, kk, W):
    """csa2_sparse_attn_append == csa2_append_swa followed by csa2_sparse_attn: same ring
    bytes, bit-identical outputs.  ahead = 0 appends position L-1 (attended from the fused
    registers); ahead = 3 appends a position past the window (written, not attended).
    k = 40, W = 32: one chunk pair, the appended row in either stream; k = 450, W = 100:
    nine chunks (an odd count) split over several workgroups whose partials are merged by
    the last to arrive, both calls on one workspace (its counters must come back to zero)."""
    import kv_cache_decode_csa2_amd as k
    K_blk = 16 if kk <= 128 else 64
    wl = si.small("fuse", 90 + ahead + kk, [700, 5000, 64, 1], H_I=4, d_I=64, K_blk=K_blk, k=kk, W=W)
    o, g = _pair(wl)
    qg = g.layer_q(0)
    _, _, tg, tlg = g.index_full(*qg)
    C = W + 16
    lay = k.csa2_layout(g.cfg)
    ring = torch.zeros((wl.B, C, lay.swa_row_bytes), dtype=torch.uint8, device="cuda")
    for b in range(wl.B):
        L = wl.ctx[b]
        n = min(L, wl.W)
        rows = dev(si.layer_swa_rows(wl, 0, b, n))
        k.csa2_append_swa(g.cfg, rows, dev(np.array([L - n], np.int32)), n, ring[b:b + 1], C)
    new_rows = dev(si.normal(90, 555, (wl.B, wl.D)))
    pos = dev(np.asarray(wl.ctx, np.int32) - 1 + ahead)
    qa = g.attn_q(0)
    ring_a, ring_b = ring.clone(), ring.clone()
    k.csa2_append_swa(g.cfg, new_rows, pos, 1, ring_a, C)
    out_a = torch.full((wl.B, wl.H_q, wl.D), float("nan"), device="cuda")
    lse_a = torch.full((wl.B, wl.H_q), float("nan"), device="cuda")
    k.csa2_sparse_attn(g.cfg, qa, g.kv, g.n_blocks, g.table, ring_a, C, g.ctx, tg, tlg, out_a,
                       lse_a, g.ws_attn)
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    k.csa2_sparse_attn_append(g.cfg, new_rows, pos, qa, g.kv, g.n_blocks, g.table, ring_b, C,
                              g.ctx, tg, tlg, out_b, lse_b, g.ws_attn)
    torch.cuda.synchronize()
    assert torch.equal(ring_a, ring_b)
    assert np.array_equal(_np(out_a).view(np.uint32), _np(out_b).view(np.uint32))
    assert np.array_equal(_np(lse_a).view(np.uint32), _np(lse_b).view(np.uint32))


@pytest.mark.parametrize("H,d,ctx,with_lat", [
    (4, 64, [5000], True),              # one sequence: the new block in the owner's first steps
    (4, 64, [300000], True),            # one sequence: the owner writes in its loop (3rd item)
    (8, 128, [700, 5000, 64, 1, 0, 9], True),  # ragged batch, contiguous ranges per wave
    (1, 32, [300, 17], False),          # one head, no main-KV append
])
def test_full_append_matches_two_calls(H, d, ctx, with_lat):
    """csa2_index_full_append == csa2_append_global at ctx_len - 1 followed by
    csa2_index_full: identical cache bytes (indexer keys and main KV), pools and top-k.  The
    appended token gets fresh values, unlike the slot's bytes in the cache, so a missing or
    misplaced write changes both the caches and the index sets."""
    import kv_cache_decode_csa2_amd as k
    from harness import make_table
    wl = si.small("fapp", 170 + H + d + len(ctx), ctx, H_I=H, d_I=d, K_blk=16, k=40)
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=True)
    g = GpuState(wl, table, nblk, with_latent=True)
    qc, qs, w = g.layer_q(0)
    new_key = dev(si.normal(171, 901, (wl.B, H * d)))
    new_lat = dev(si.normal(171, 902, (wl.B, wl.D))) if with_lat else None
    pos = g.ctx - 1
    res = []
    for fused in (False, True):
        kv, idx = g.kv.clone(), g.idx.clone()
        pool = torch.full((wl.B, wl.K_blk), -7, dtype=torch.int32, device="cuda")
        pl = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
        topk = torch.full((wl.B, wl.k), -7, dtype=torch.int32, device="cuda")
        tl = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
        if fused:
            k.csa2_index_full_append(g.cfg, new_lat, new_key, qc, qs, w, kv if with_lat else None,
                                     idx, g.n_blocks, g.table, g.ctx, pool, pl, topk, tl, g.ws)
        else:
            k.csa2_append_global(g.cfg, new_lat, new_key, g.table, g.n_blocks, pos, 1,
                                 kv if with_lat else None, idx)
            k.csa2_index_full(g.cfg, qc, qs, w, idx, g.n_blocks, g.table, g.ctx, pool, pl, topk,
                              tl, g.ws)
        torch.cuda.synchronize()
        res.append((_np(kv), _np(idx), _np(pool), _np(pl), _np(topk), _np(tl)))
    names = ("kv cache", "idx cache", "pool", "pool_len", "topk", "topk_len")
    for name, x, y in zip(names, res[0], res[1]):
        assert np.array_equal(x, y), (name, _first_diff(x, y))
    assert not np.array_equal(res[0][1], _np(g.idx)), "the append changed no key byte"


def test_global_tier_round_trip():
    """The persistent global-KV tier: both block caches of every sequence leave through
    csa2_blocks_gather into pinned host memory, the device caches are cleared, and the rows
    come back with csa2_blocks_scatter into a different physical placement (a new block
    table).  Every logical block's bytes are unchanged, and Full, Reindex and attention give
    bit-identical results to those before the round trip; after the restore, pool and top-k
    of both index layers equal the oracle's and attention is within 2e-3 of it."""
    import kv_cache_decode_csa2_amd as k
    wl = si.small("tier", 41, [3000, 517, 9], H_I=4, d_I=64, K_blk=32, k=64, H_q=16, W=128)
    table, nblk = make_table(wl.ctx, seed=41)
    o = OracleState(wl, table, nblk)
    g = GpuState(wl, table, nblk)
    qF, qR = g.layer_q(0), g.layer_q(1)
    swa, qa = g.layer_swa(0), g.attn_q(0)

    def run():
        pool, pl, tk, tl = g.index_full(*qF)
        tkR, tlR = g.index_reindex(*qR, pool, pl)
        out, lse = g.attn(qa, swa, tk, tl)
        torch.cuda.synchronize()
        return [_np(x) for x in (pool, pl, tk, tl, tkR, tlR, out, lse)]

    before = run()
    po, plo, to, tlo = oracle.index_full(o.cfg, *o.layer_q(0), o.idx, o.table, o.ctx)
    assert np.array_equal(before[0], po) and np.array_equal(before[2], to)

    valid = table >= 0
    src = dev(table[valid].astype(np.int32))          # (sequence, logical block) order
    new_table, _ = make_table(wl.ctx, seed=4141)       # another permutation of the blocks
    assert not np.array_equal(new_table, table)
    dst = dev(new_table[valid].astype(np.int32))
    logical_bytes = {}
    for name in ("idx", "kv"):
        cache = getattr(g, name)
        rows = torch.empty((src.numel(), cache.shape[1]), dtype=torch.uint8, device="cuda")
        k.csa2_blocks_gather(cache, src, rows)
        host = torch.empty(rows.shape, dtype=torch.uint8, pin_memory=True)
        host.copy_(rows)
        torch.cuda.synchronize()
        logical_bytes[name] = host.numpy().copy()
        cache.zero_()
        k.csa2_blocks_scatter(host.to("cuda"), dst, cache)
    g.table = dev(new_table)
    torch.cuda.synchronize()
    for name in ("idx", "kv"):
        cache = getattr(g, name)
        back = torch.empty((dst.numel(), cache.shape[1]), dtype=torch.uint8, device="cuda")
        k.csa2_blocks_gather(cache, dst, back)
        assert np.array_equal(_np(back), logical_bytes[name]), name
    after = run()
    for x, y in zip(before, after):
        assert np.array_equal(x, y)
    # and the restored caches index and attend as the oracle does on its own caches
    assert np.array_equal(after[0], po) and np.array_equal(after[1], plo)
    assert np.array_equal(after[2], to) and np.array_equal(after[3], tlo)
    tRo, tlRo = oracle.index_reindex(o.cfg, *o.layer_q(1), o.idx, o.table, o.ctx, po, plo)
    assert np.array_equal(after[4], tRo) and np.array_equal(after[5], tlRo)
    ro, rl = oracle.sparse_attn(o.cfg, si.layer_attn_q(wl, 0), o.kv, o.table, o.layer_swa(0),
                                o.C, o.ctx, to, tlo)
    ok, rel, lerr = attn_close(after[6], after[7], ro, rl)
    assert ok, (rel, lerr)

    # entries outside the cache: gather writes zero rows, scatter leaves the cache alone
    bad = dev(np.array([-1, nblk, 0], np.int32))
    rows = torch.full((3, g.idx.shape[1]), 0xAB, dtype=torch.uint8, device="cuda")
    k.csa2_blocks_gather(g.idx, bad, rows)
    r = _np(rows)
    assert not r[:2].any() and np.array_equal(r[2], _np(g.idx[0]))
    snapshot = _np(g.idx).copy()
    k.csa2_blocks_scatter(torch.full_like(rows, 0x5A), dev(np.array([-1, nblk, -5], np.int32)), g.idx)
    torch.cuda.synchronize()
    assert np.array_equal(_np(g.idx), snapshot)


# ------------------------------------------------------------------ two-phase Full selection

@pytest.mark.parametrize("ctx,K_blk,k", [
    ([150000, 3000, 100, 70000, 9000], 256, 100),   # 3 and 2 gather workgroups, a sequence
                                                     # that fits the pool, ragged tails
    ([40000, 200000], 1024, 512),                    # sequence 0 has ng <= K_blk: all of its
                                                     # groups hold candidates
    ([20000, 333], 64, 64),                          # K_blk == k
])
def test_full_two_phase_selection(ctx, K_blk, k):
    """Contexts with more blocks than the pool take the two-phase Full selection (gather
    workgroups per 1024 groups, the last one selecting pool and top-k from the compact
    candidates) once the table has at least 2 K_blk groups; pools, top-k, Reindex and
    attention equal the oracle's."""
    wl = si.small("tp", 610 + K_blk + len(ctx), ctx, H_I=4, d_I=64, K_blk=K_blk, k=k, W=32,
                  layers="FRU")
    print(_run_group(wl, permute=True))


def test_full_two_phase_ties_fall_back():
    """Every key of the first 30000 positions equal: thousands of blocks tie at the top, so
    the regions of bound-reaching blocks overflow and the last workgroup runs the
    one-workgroup selection;
    the results still equal the oracle's (lower index first among equal scores)."""
    wl = si.small("tpt", 620, [60000, 5000], H_I=4, d_I=64, K_blk=256, k=256, W=16)
    row = si.normal(620, 999, (1, wl.H_I, wl.d_I))
    orig = si.idx_keys

    def keys(w, b, L=None):
        x = orig(w, b, L)
        if b == 0:
            x[:30000] = row
        return x

    try:
        si.idx_keys = keys
        print(_run_group(wl, with_attn=False))
    finally:
        si.idx_keys = orig
