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
import kv_cache_decode_csa2_amd as k
from gpu_harness import GpuState, attn_close, dev, index_prefill, prefill_q
from harness import OracleState, make_table

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _first_diff(a, b, n=5):
    idx = np.argwhere(a != b)[:n]
    return [(tuple(i), a[tuple(i)], b[tuple(i)]) for i in idx]


def _ngmax(maxb):
    return (((maxb + 7) // 8) + 3) & ~3


def _al(x):
    return (x + 255) & ~255


def _ws_scores(ws, n_q, maxb, blk0=0, blk1=None):
    """The scoring kernel's outputs in the prefill workspace, for blocks [blk0, blk1): position
    scores [block][query][slot], block maxima [group][query][block % 8] and group maxima
    [query][group] (the layout the selection reads), as host arrays."""
    blk1 = maxb if blk1 is None else blk1
    row = n_q * 8 * 4
    ps = ws[blk0 * row:blk1 * row].view(torch.float32).reshape(blk1 - blk0, n_q, 8)
    ng = _ngmax(maxb)
    ob = _al(maxb * row)
    g0, g1 = blk0 // 8, (blk1 + 7) // 8
    bs = ws[ob + g0 * row:ob + g1 * row].view(torch.float32).reshape(g1 - g0, n_q, 8)
    og = _al(ob + ng * row)
    gm = ws[og:og + n_q * ng * 4].view(torch.float32).reshape(n_q, ng)[:, g0:g1]
    return _np(ps), _np(bs), _np(gm)


def _ws_flags(ws, n_q, maxb, K_blk):
    """More than 16 queries (two scoring passes): per query the flagged blocks (those whose
    position scores the rescoring pass wrote) from the ascending list and its count, and
    from the flag words [chunk of 256 blocks][word of 32 blocks][query]."""
    ng = _ngmax(maxb)
    row = n_q * 8 * 4
    ob = _al(maxb * row)
    og = _al(ob + ng * row)
    oks = _al(og + n_q * ng * 4)
    on = _al(oks + ng * 8)
    npc = (maxb + 255) // 256
    ol = _al(on + 8 * npc * n_q * 4)
    om = _al(ol + K_blk * n_q * 4)
    words = _np(ws[on:on + 8 * npc * n_q * 4].view(torch.int32)).view(np.uint32).reshape(npc, 8, n_q)
    lst = _np(ws[ol:ol + K_blk * n_q * 4].view(torch.int32)).reshape(n_q, K_blk)
    meta = _np(ws[om:om + 16 * n_q].view(torch.int32)).view(np.uint32).reshape(n_q, 4)
    listed = [lst[i, :meta[i, 2]].copy() for i in range(n_q)]
    bits = np.unpackbits(np.ascontiguousarray(words.transpose(2, 0, 1)).reshape(n_q, -1).view(np.uint8),
                         axis=1, bitorder="little")
    flagged = [np.flatnonzero(bits[i]).astype(np.int32) for i in range(n_q)]
    return listed, flagged


def _check_flags(o, qo, q_pos0, n_q, pool, plen, listed, flagged, k_top):
    """The flagged blocks of each query: the flag words and the list agree, ascending; they
    lie in the pool and hold every pool block whose maximum reaches the k-th largest maximum
    of the pool (all of the pool when it has fewer than k blocks or at most k positions)."""
    for i in range(n_q):
        t = q_pos0 + i
        assert np.array_equal(listed[i], flagged[i]), (i, "flag words / list")
        pl = pool[i, :plen[i]]
        assert np.isin(listed[i], pl).all(), (i, "flagged outside the pool")
        ref = oracle.index_scores(o.cfg, qo[0][i], qo[1][i], qo[2][i], o.idx, o.table[0], t + 1)
        bm = oracle.block_scores(ref, t + 1)[pl]
        nvis = sum(min(8, t + 1 - 8 * j) for j in pl)
        if len(pl) >= k_top and nvis > k_top:
            need = pl[bm >= np.sort(bm)[-k_top]]
        else:
            need = pl
        assert np.isin(need, listed[i]).all(), (i, "a block the top-k can draw from is not flagged")


def _check_scores(o, qo, q_pos0, queries, ps, bs, gm, blk0, blk1, flagged=None):
    """Scores of the listed queries at positions 8*blk0 .. 8*blk1-1 (their causal part)
    equal the oracle's bit for bit (with `flagged`, only those of each query's flagged
    blocks: the rest are never written); so do the block maxima of those blocks and the
    maxima of the groups of 8 blocks that lie wholly inside the range."""
    table_row = o.table[0]
    for i in queries:
        t = q_pos0 + i
        p0 = blk0 * 8
        n = min(blk1 * 8, t + 1) - p0
        if n <= 0:
            continue
        ref = oracle.index_scores(o.cfg, qo[0][i], qo[1][i], qo[2][i], o.idx, table_row[blk0:], n)
        got, want = ps[:, i, :].reshape(-1)[:n], ref
        if flagged is not None:
            fb = flagged[i][(flagged[i] >= blk0) & (flagged[i] < blk1)] - blk0
            sel = (fb[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
            sel = sel[sel < n]
            got, want = got[sel], ref[sel]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (i, _first_diff(got, want))
        rb = oracle.block_scores(ref, n)
        gb = bs.reshape(-1, bs.shape[1], 8)[:, i, :].reshape(-1)[blk0 % 8:][:len(rb)]
        assert np.array_equal(gb.view(np.uint32), rb.view(np.uint32)), (i, "block maxima")
        for gi in range((blk0 + 7) // 8, (blk1 + 7) // 8):
            j0 = gi * 8 - blk0
            vis = rb[j0:j0 + 8]
            whole = gi * 8 + 8 <= blk1 or blk1 * 8 > t  # every visible block of it is in range
            if len(vis) == 0 or not whole:
                continue
            assert gm[i, gi - blk0 // 8] == vis.max(), (i, gi, "group maximum")


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
    maxb = table.shape[1]
    ws = torch.empty(k.csa2_workspace_bytes(g.cfg, k.CSA2_OP_INDEX_PREFILL, n_q, maxb),
                     dtype=torch.uint8, device="cuda")
    pg, plg, tg, tlg = index_prefill(g, qc, qs, wg, q_pos0, ws=ws)
    torch.cuda.synchronize()
    # what the selection read: the block and group maxima of every query, and every causal
    # score (at most 16 queries) or those of the flagged blocks
    ps, bs, gm = _ws_scores(ws, n_q, maxb)
    flagged = None
    if n_q > 16:
        listed, flagged = _ws_flags(ws, n_q, maxb, wl.K_blk)
        _check_flags(o, qo, q_pos0, n_q, po, plo, listed, flagged, wl.k)
    _check_scores(o, qo, q_pos0, range(n_q), ps, bs, gm, 0, maxb, flagged)
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
    (2, 32, 4300, 4160),   # more queries than one listing round of the rescoring pass (4096)
    # at most 16 queries: the waves split each stage's positions
    (4, 64, 5000, 6),      # verification step: 6 queries, 3 position chunks (ragged)
    (8, 128, 2800, 16),
    (2, 32, 130, 1),       # one query, two stages
    (4, 64, 50, 2),        # one stage (the second buffer repeats it)
    (4, 64, 100, 5),       # two stages
    (1, 128, 2100, 9),
])
def test_prefill_index_bit_exact(H, d, L, n_q):
    wl = si.small("pf", 100 + H + d + L, [L], H_I=H, d_I=d, K_blk=64, k=128, W=16)
    _check(wl, n_q)


@pytest.mark.parametrize("L,n_q", [(12000, 6), (9000, 16)])
def test_prefill_few_queries_two_phase_selection(L, n_q):
    """At most 16 queries over a table of at least 2 K_blk groups with K_blk >= k: the
    selection runs in two phases (gather workgroups, the last one selecting the pool, a top-k
    workgroup per query); pools and top-k equal the oracle's per query."""
    wl = si.small("pf2p", 140 + L, [L], H_I=4, d_I=64, K_blk=64, k=48, W=16)
    _check(wl, n_q)


def test_prefill_pool_covers_everything():
    # most prefixes have at most K_blk blocks: the pool is every visible block
    wl = si.small("pfcov", 120, [900], H_I=4, d_I=128, K_blk=128, k=300, W=16)
    _check(wl, 400, permute=False)


@pytest.mark.parametrize("n_q", [10, 200])
def test_prefill_key_spans_decide_the_path(n_q):
    """Key groups scaled by 2^20 (every head's group 0, one block in seven) with plain
    queries: only the key spans (the span pass, or at most 16 queries the scoring kernel's
    own) send those tiles to the per-group path, and a single product over groups this far
    apart would lose the small groups' terms."""
    wl = si.small("pfkspan", 122, [3000], H_I=4, d_I=64, K_blk=64, k=128, W=16)

    def keys_wide(x):
        blk = np.arange(x.shape[0]) // 8
        x[blk % 7 == 2, :, 0:32] *= np.float32(2.0 ** 20)

    orig = si.idx_keys
    try:
        si.idx_keys = lambda w_, b, L=None: (lambda x: (keys_wide(x), x)[1])(orig(w_, b, L))
        _check(wl, n_q)
    finally:
        si.idx_keys = orig


@pytest.mark.parametrize("n_q", [260, 12])
def test_prefill_wide_exponent_spans_take_the_exact_path(n_q):
    """Scales that spread more than 9 binades within a head vector force the per-group
    path of the matrix kernel (at most 16 queries: spans over four groups taken from the
    staged scales); mixed-sign head weights exercise the fma chain's signs."""
    wl = si.small("pfspan", 121, [3000], H_I=8, d_I=128, K_blk=64, k=128, W=16)

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


def _rings(wl, o, g, q_pos0, n_q):
    """The sequence's window ring holding positions q_pos0-W+1 .. q_pos0+n_q-1 (oracle and
    GPU, same seeded rows), C = n_q + W slots."""
    C = n_q + wl.W
    first = max(0, q_pos0 - wl.W + 1)
    rows = si.layer_swa_rows(wl, 0, 0, q_pos0 + n_q - first)
    ro = oracle.alloc_swa(o.cfg, 1, C)
    oracle.append_swa(o.cfg, rows[None], np.array([first], np.int32), ro, C)
    rg = torch.zeros((1, C, g.lay.swa_row_bytes), dtype=torch.uint8, device="cuda")
    k.csa2_append_swa(g.cfg, dev(rows), dev(np.array([first], np.int32)), rows.shape[0], rg, C)
    return C, ro, rg


def _attn_prefill(g, q, ring, C, q_pos0, topk, tl):
    n_q = q.shape[0]
    wl = g.wl
    ws = torch.zeros(k.csa2_workspace_bytes(g.cfg, k.CSA2_OP_SPARSE_ATTN, n_q, g.table.shape[1]),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((n_q, wl.H_q, wl.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((n_q, wl.H_q), float("nan"), dtype=torch.float32, device="cuda")
    k.csa2_sparse_attn_prefill(g.cfg, q, g.kv, g.n_blocks, g.table[0].contiguous(), ring, C,
                               q_pos0, topk, tl, out, lse, ws)
    return out, lse


@pytest.mark.parametrize("L,n_q,H_q,W,k_top", [
    (3000, 200, 32, 32, 128),   # one workgroup per (query, head pair)
    (300, 300, 16, 128, 128),   # one head group: the split kernel
    (2000, 150, 64, 128, 128),  # two head pairs per query
    (300, 300, 64, 32, 96),     # a chunk holding both top-k and window rows; short prefixes
])
def test_prefill_attention_within_tolerance(L, n_q, H_q, W, k_top):
    """Per-query sparse attention of a prefill chunk: each query's own top-k (from the GPU
    prefill indexer, checked equal to the oracle's) plus its own window from the shared
    ring; within 2e-3 of the fp64 oracle."""
    wl = si.small("pfat", 130 + L, [L], H_I=8, d_I=128, K_blk=64, k=k_top, H_q=H_q, W=W)
    q_pos0 = L - n_q
    table, nblk = make_table(wl.ctx, seed=wl.seed)
    o = OracleState(wl, table, nblk)
    g = GpuState(wl, table, nblk)
    qo = _oracle_q(wl, n_q)
    _, _, to, tlo = oracle.index_prefill(o.cfg, *qo, q_pos0, o.idx, o.table[0])
    _, _, tg, tlg = index_prefill(g, *prefill_q(wl, 0, n_q), q_pos0)
    assert np.array_equal(_np(tg), to) and np.array_equal(_np(tlg), tlo)
    C, ring_o, ring_g = _rings(wl, o, g, q_pos0, n_q)
    assert np.array_equal(_np(ring_g), ring_o)
    qa = si.prefill_attn_q(wl, 0, n_q)
    ro, rl = oracle.sparse_attn_prefill(o.cfg, qa, o.kv, o.table[0], ring_o[0], C, q_pos0, to, tlo)
    go, gl = _attn_prefill(g, dev(qa.view(np.int16)), ring_g, C, q_pos0, tg, tlg)
    ok, rel, lerr = attn_close(_np(go), _np(gl), ro, rl)
    print("prefill attention rel", rel, "lse", lerr)
    assert ok, (rel, lerr)


@pytest.mark.slow
def test_prefill_workload_sampled():
    """The prefill workload at full size: 4096 queries at positions 258048..262143 of a
    262,144-token context, indexer 8 x 128, pool 2048 blocks, top-512, then attention of
    64 heads over each query's top-k and window.  Against the oracle:
    * every score, block maximum and group maximum of two whole 128-query tiles (queries
      0..127 and 2048..2175) over four 2048-position chunks each -- the first, a middle one
      and the chunks that hold the tiles' causal boundary -- bit for bit;
    * pool, top-k and attention of the queries on both sides of a query-tile boundary
      (127 | 128), of a position-chunk boundary (query 2047 at position 260095 ends chunk
      126, query 2048 opens chunk 127) and of the first and last query.
    Every query is checked for the properties that hold at any size (lengths, ascending
    order, top-k inside the pool, causality)."""
    wl = si.workload("prefill")
    n_q, L = wl.n_q, wl.ctx[0]
    q_pos0 = L - n_q
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    maxb = table.shape[1]
    g = GpuState(wl, table, nblk)
    o = OracleState(wl, table, nblk)
    qc, qs, wg = prefill_q(wl, 0, n_q)
    ws = torch.empty(k.csa2_workspace_bytes(g.cfg, k.CSA2_OP_INDEX_PREFILL, n_q, maxb),
                     dtype=torch.uint8, device="cuda")
    pgd, plgd, tgd, tlgd = index_prefill(g, qc, qs, wg, q_pos0, ws=ws)
    pg, plg, tg, tlg = [_np(x) for x in (pgd, plgd, tgd, tlgd)]
    C, ring_o, ring_g = _rings(wl, o, g, q_pos0, n_q)
    qa = si.prefill_attn_q(wl, 0, n_q)
    go, gl = _attn_prefill(g, dev(qa.view(np.int16)), ring_g, C, q_pos0, tgd, tlgd)
    go, gl = _np(go), _np(gl)
    qo = _oracle_q(wl, n_q)
    listed, flagged = _ws_flags(ws, n_q, maxb, wl.K_blk)
    for i in range(n_q):
        assert np.array_equal(listed[i], flagged[i]), (i, "flag words / list")
        assert np.isin(listed[i], pg[i]).all() and len(listed[i]) >= wl.k, (i, "flagged blocks")
    # whole tiles x chunks (chunk = 256 blocks = 2048 positions): maxima, and the scores of
    # the flagged blocks
    for tile0 in (0, 2048):
        t_first = q_pos0 + tile0
        diag = t_first // 2048
        for c in sorted({0, 63, diag, diag + 1}):
            if c * 2048 >= L:
                continue
            ps, bs, gm = _ws_scores(ws, n_q, maxb, c * 256, (c + 1) * 256)
            _check_scores(o, qo, q_pos0, range(tile0, tile0 + 128), ps, bs, gm, c * 256,
                          (c + 1) * 256, flagged)
    del ws, g
    torch.cuda.empty_cache()
    assert np.all(plg == wl.K_blk) and np.all(tlg == wl.k)
    assert np.all(np.diff(pg, axis=1) > 0) and np.all(np.diff(tg, axis=1) > 0)
    t = q_pos0 + np.arange(n_q)
    assert np.all(tg[:, -1] <= t) and np.all(pg[:, -1] <= t // 8)
    assert all(np.isin(tg[i] // 8, pg[i]).all() for i in range(0, n_q, 97))
    for i in (0, 1, 127, 128, 2047, 2048, n_q - 1):
        ctx = np.array([q_pos0 + i + 1], np.int32)
        po, plo, to, tlo = oracle.index_full(o.cfg, qo[0][i:i + 1], qo[1][i:i + 1],
                                             qo[2][i:i + 1], o.idx, o.table, ctx)
        assert np.array_equal(pg[i], po[0]), (i, _first_diff(pg[i], po[0]))
        assert np.array_equal(tg[i], to[0]), (i, _first_diff(tg[i], to[0]))
        ro, rl = oracle.sparse_attn(o.cfg, qa[i:i + 1], o.kv, o.table, ring_o, C, ctx, to, tlo)
        ok, rel, lerr = attn_close(go[i:i + 1], gl[i:i + 1], ro, rl)
        assert ok, (i, rel, lerr)


@pytest.mark.slow
def test_spec_verify_selection_by_xcd():
    """Three queries at the end of a 500,000-token context: 7,813 groups, so 8 gather
    workgroups per query and the two-phase selection's XCD layout (gather workgroup w of every
    query on XCD w % 8, idle workgroups in the padded grid).  Every query's pool and top-k
    equal the oracle's."""
    import dataclasses
    wl = dataclasses.replace(si.workload("spec_1m"), ctx=[500000], n_q=3)
    n_q, L = wl.n_q, wl.ctx[0]
    q_pos0 = L - n_q
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    g = GpuState(wl, table, nblk)
    o = OracleState(wl, table, nblk)
    qc, qs, wg = prefill_q(wl, 0, n_q)
    pgd, plgd, tgd, tlgd = index_prefill(g, qc, qs, wg, q_pos0)
    pg, plg, tg, tlg = [_np(x) for x in (pgd, plgd, tgd, tlgd)]
    del g
    torch.cuda.empty_cache()
    qo = _oracle_q(wl, n_q)
    po, plo, to, tlo = oracle.index_prefill(o.cfg, *qo, q_pos0, o.idx, o.table[0])
    assert np.all(plo == wl.K_blk) and np.all(tlo == wl.k)
    assert np.array_equal(plg, plo) and np.array_equal(tlg, tlo)
    assert np.array_equal(pg, po), _first_diff(pg, po)
    assert np.array_equal(tg, to), _first_diff(tg, to)


def test_spec_verify_1m():
    """Speculative verification at 1M context: the token and 5 draft tokens at positions
    1048570..1048575 of a 1,048,576-token context (indexer 4 x 64, pool 2048 blocks,
    top-512, 16 heads, window 128) run as one 6-query prefill chunk.  Every query's pool and
    top-k equal the oracle's (each query the Full steps at its own causal length), and its
    attention is within 2e-3 of the fp64 oracle."""
    wl = si.workload("spec_1m")
    n_q, L = wl.n_q, wl.ctx[0]
    q_pos0 = L - n_q
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    g = GpuState(wl, table, nblk)
    o = OracleState(wl, table, nblk)
    qc, qs, wg = prefill_q(wl, 0, n_q)
    pgd, plgd, tgd, tlgd = index_prefill(g, qc, qs, wg, q_pos0)
    C, ring_o, ring_g = _rings(wl, o, g, q_pos0, n_q)
    qa = si.prefill_attn_q(wl, 0, n_q)
    go, gl = _attn_prefill(g, dev(qa.view(np.int16)), ring_g, C, q_pos0, tgd, tlgd)
    pg, plg, tg, tlg, go, gl = [_np(x) for x in (pgd, plgd, tgd, tlgd, go, gl)]
    del g
    torch.cuda.empty_cache()
    qo = _oracle_q(wl, n_q)
    po, plo, to, tlo = oracle.index_prefill(o.cfg, *qo, q_pos0, o.idx, o.table[0])
    assert np.all(plo == wl.K_blk) and np.all(tlo == wl.k)
    assert np.array_equal(plg, plo) and np.array_equal(tlg, tlo)
    assert np.array_equal(pg, po), _first_diff(pg, po)
    assert np.array_equal(tg, to), _first_diff(tg, to)
    ro, rl = oracle.sparse_attn_prefill(o.cfg, qa, o.kv, o.table[0], ring_o[0], C, q_pos0, to, tlo)
    ok, rel, lerr = attn_close(go, gl, ro, rl)
    print("spec verification attention rel", rel, "lse", lerr)
    assert ok, (rel, lerr)
