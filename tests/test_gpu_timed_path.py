"""GPU parity of exactly what the bench times, and of the calls' less common code paths.

* The decode group as bench.py captures and replays it (per layer: the indexer query's
  MXFP4 quantise, the Full layer's fused global append + index, Reindex, and every layer's
  fused window append + attention) against the oracle: cache bytes, pool, every layer's
  top-k bit-exact, attention within 2e-3.  Before the replay the positions the group
  appends are overwritten with other values, so the replay must write them itself.
* One zero-once attention workspace reused by calls of different batch and query counts.
* The scan variants with 64-bit key offsets (caches larger than 4 GiB).
"""
import numpy as np
import pytest
import torch

import kv_cache_decode_csa2_amd as k
import oracle
import synth_inputs as si
from gpu_harness import GpuState, attn_close, dev, index_prefill, prefill_q
from harness import OracleState, make_table

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _first_diff(a, b, n=5):
    idx = np.argwhere(a != b)[:n]
    return [(tuple(i), a[tuple(i)], b[tuple(i)]) for i in idx]


# ------------------------------------------------------------------ the timed decode group

def _timed_group(wl):
    import bench
    b = bench.Bench(wl, replicas=1)
    b.scribble(0)
    graph = bench.capture(lambda: b.step(0))  # (runs the step once eagerly before capture)
    b.scribble(0)
    graph.replay()
    torch.cuda.synchronize()
    got = b.results()
    kv, idx = _np(b.kv[0]), _np(b.idx[0])
    rings = [_np(lay["swa"]) for lay in b.layers]
    del b, graph
    torch.cuda.empty_cache()
    o = OracleState(wl, *make_table(wl.ctx, seed=wl.seed, permute=False), with_latent=True)
    assert np.array_equal(idx, o.idx), ("indexer-key cache", _first_diff(idx, o.idx))
    assert np.array_equal(kv, o.kv), ("main-KV cache", _first_diff(kv, o.kv))
    for li, ring in enumerate(rings):
        assert np.array_equal(ring, o.layer_swa(li)), ("window ring", li)
    ref = bench.oracle_group(wl, o)
    assert np.array_equal(got["pool_len"], ref["pool_len"])
    assert np.array_equal(got["pool"], ref["pool"]), _first_diff(got["pool"], ref["pool"])
    for li, (g_, r_) in enumerate(zip(got["layers"], ref["layers"])):
        assert np.array_equal(g_["topk_len"], r_["topk_len"]), (li, "topk_len")
        assert np.array_equal(g_["topk"], r_["topk"]), (li, _first_diff(g_["topk"], r_["topk"]))
        ok, rel, lerr = attn_close(g_["out"], g_["lse"], r_["out"], r_["lse"])
        assert ok, (li, g_["mode"], rel, lerr)
    s = bench.compare_group(got, ref)
    assert s["ok"], s
    return s


def test_timed_group_tiny():
    print(_timed_group(si.workload("tiny")))


def test_timed_group_ragged_small():
    """A ragged batch through the bench's step (contiguous item ranges per wave, sequences
    of one block, a sequence whose new token opens a block)."""
    wl = si.small("tgr", 301, [4097, 9, 777, 20000, 1], H_I=4, d_I=64, K_blk=64, k=128, W=128)
    print(_timed_group(wl))


@pytest.mark.slow
def test_timed_group_long_1m():
    print(_timed_group(si.workload("long_1m")))


@pytest.mark.slow
def test_timed_group_b8_64k():
    print(_timed_group(si.workload("b8_64k")))


# ------------------------------------------------------------------ attention workspace

def test_attention_workspace_reused_across_shapes():
    """One attention workspace, zeroed once and sized for the largest call, serves a batch-8
    decode, a batch-1 decode, a 6-query prefill chunk and a batch-1 decode again: every
    call splits its rows over several workgroups whose arrival counters sit at the same
    place whatever the shape.  Each result is compared with the oracle."""
    wl = si.small("wsr", 311, [5000, 700, 3000, 4000, 64, 2500, 1000, 6000], H_I=4, d_I=64,
                  K_blk=64, k=450, H_q=32, W=100)
    table, nblk = make_table(wl.ctx, seed=wl.seed)
    o = OracleState(wl, table, nblk)
    g = GpuState(wl, table, nblk)
    qg, qo = g.layer_q(0), o.layer_q(0)
    _, _, tg, tlg = g.index_full(*qg)
    _, _, to, tlo = oracle.index_full(o.cfg, *qo, o.idx, o.table, o.ctx)
    assert np.array_equal(_np(tg), to)
    swg, swo = g.layer_swa(0), o.layer_swa(0)
    qa = si.layer_attn_q(wl, 0)
    maxb = table.shape[1]
    n_q = 6
    sizes = [k.csa2_workspace_bytes(g.cfg, k.CSA2_OP_SPARSE_ATTN, n, maxb) for n in (8, 1, n_q)]
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device="cuda")

    def decode(rows):
        B = len(rows)
        out = torch.full((B, wl.H_q, wl.D), float("nan"), device="cuda")
        lse = torch.full((B, wl.H_q), float("nan"), device="cuda")
        sel = torch.tensor(rows, device="cuda")
        k.csa2_sparse_attn(g.cfg, dev(qa[rows].view(np.int16)), g.kv, g.n_blocks,
                           g.table[sel].contiguous(), swg[sel].contiguous(), g.C,
                           g.ctx[sel].contiguous(), tg[sel].contiguous(), tlg[sel].contiguous(),
                           out, lse, ws)
        ro, rl = oracle.sparse_attn(o.cfg, qa[rows], o.kv, o.table[rows], swo[rows], o.C,
                                    o.ctx[rows], to[rows], tlo[rows])
        ok, rel, lerr = attn_close(_np(out), _np(lse), ro, rl)
        assert ok, (rows, rel, lerr)

    decode(list(range(8)))
    decode([3])
    # a 6-query prefill chunk at the end of sequence 0 (top-k from the GPU prefill indexer)
    L0 = wl.ctx[0]
    q_pos0 = L0 - n_q
    qp = si.prefill_idx_q(wl, 0, n_q)
    qpc, qps = oracle.quantize_mxfp4(qp.reshape(n_q, -1))
    _, _, tpo, tlpo = oracle.index_prefill(o.cfg, qpc, qps, si.prefill_idx_w(wl, 0, n_q), q_pos0,
                                          o.idx, o.table[0])
    _, _, tpg, tlpg = index_prefill(g, *prefill_q(wl, 0, n_q), q_pos0)
    assert np.array_equal(_np(tpg), tpo) and np.array_equal(_np(tlpg), tlpo)
    C = n_q + wl.W
    first = q_pos0 - wl.W + 1
    rows = si.layer_swa_rows(wl, 0, 0, L0 - first)
    ring_o = oracle.alloc_swa(o.cfg, 1, C)
    oracle.append_swa(o.cfg, rows[None], np.array([first], np.int32), ring_o, C)
    ring_g = torch.zeros((1, C, g.lay.swa_row_bytes), dtype=torch.uint8, device="cuda")
    k.csa2_append_swa(g.cfg, dev(rows), dev(np.array([first], np.int32)), rows.shape[0], ring_g, C)
    qpa = si.prefill_attn_q(wl, 0, n_q)
    out = torch.full((n_q, wl.H_q, wl.D), float("nan"), device="cuda")
    lse = torch.full((n_q, wl.H_q), float("nan"), device="cuda")
    k.csa2_sparse_attn_prefill(g.cfg, dev(qpa.view(np.int16)), g.kv, g.n_blocks,
                               g.table[0].contiguous(), ring_g, C, q_pos0, tpg, tlpg, out, lse, ws)
    ro, rl = oracle.sparse_attn_prefill(o.cfg, qpa, o.kv, o.table[0], ring_o[0], C, q_pos0, tpo,
                                        tlpo)
    ok, rel, lerr = attn_close(_np(out), _np(lse), ro, rl)
    assert ok, ("prefill", rel, lerr)
    decode([3])
    decode([7, 0])
    # every call leaves the counters at zero
    assert not _np(ws[:4096]).any()


# ------------------------------------------------------------------ 64-bit key offsets

@pytest.mark.parametrize("H,d", [(4, 64), (8, 128)])
def test_scan_with_64bit_offsets(H, d):
    """A cache whose declared size passes 4 GiB (n_blocks * block bytes > 2^32) takes the
    scan variants that address keys with 64-bit offsets: the plain scan, the scan carrying
    the global append (4 x 64; 8 x 128 appends in a launch of its own) and the Reindex
    rescoring.  n_blocks is only a bound, so the real cache stays small and every table
    entry lies in it; the results must equal the oracle's."""
    wl = si.small("o64", 320 + H, [3000, 517, 9, 20000], H_I=H, d_I=d, K_blk=64, k=128, W=64)
    table, nblk = make_table(wl.ctx, seed=wl.seed)
    o = OracleState(wl, table, nblk)
    g = GpuState(wl, table, nblk)
    lay = k.csa2_layout(g.cfg)
    big = (1 << 32) // lay.idx_block_bytes + 1
    assert big * lay.idx_block_bytes > (1 << 32)
    qF, qR = g.layer_q(0), g.layer_q(1)
    oF, oR = o.layer_q(0), o.layer_q(1)
    i32 = dict(dtype=torch.int32, device="cuda")

    def outs():
        return (torch.full((wl.B, wl.K_blk), -7, **i32), torch.zeros(wl.B, **i32),
                torch.full((wl.B, wl.k), -7, **i32), torch.zeros(wl.B, **i32))

    po, plo, to, tlo = oracle.index_full(o.cfg, *oF, o.idx, o.table, o.ctx)
    pool, pl, tk, tl = outs()
    k.csa2_index_full(g.cfg, *qF, g.idx, big, g.table, g.ctx, pool, pl, tk, tl, g.ws)
    assert np.array_equal(_np(pool), po) and np.array_equal(_np(pl), plo)
    assert np.array_equal(_np(tk), to) and np.array_equal(_np(tl), tlo)
    tRo, tlRo = oracle.index_reindex(o.cfg, *oR, o.idx, o.table, o.ctx, po, plo)
    tR, tlR = torch.full((wl.B, wl.k), -7, **i32), torch.zeros(wl.B, **i32)
    k.csa2_index_reindex(g.cfg, *qR, g.idx, big, g.table, g.ctx, pool, pl, tR, tlR, g.ws)
    assert np.array_equal(_np(tR), tRo) and np.array_equal(_np(tlR), tlRo)
    # attention with the same bound on the main-KV cache
    out = torch.full((wl.B, wl.H_q, wl.D), float("nan"), device="cuda")
    lse = torch.full((wl.B, wl.H_q), float("nan"), device="cuda")
    k.csa2_sparse_attn(g.cfg, g.attn_q(0), g.kv, big, g.table, g.layer_swa(0), g.C, g.ctx, tR,
                       tlR, out, lse, g.ws_attn)
    ro, rl = oracle.sparse_attn(o.cfg, si.layer_attn_q(wl, 0), o.kv, o.table, o.layer_swa(0),
                                o.C, o.ctx, tRo, tlRo)
    ok, rel, lerr = attn_close(_np(out), _np(lse), ro, rl)
    assert ok, (rel, lerr)
    # the Full layer's fused append at position L-1 with a new token
    new_key = si.normal(321, 7, (wl.B, H * d))
    new_lat = si.normal(321, 8, (wl.B, wl.D))
    pos = np.asarray(wl.ctx, np.int32) - 1
    oracle.append_global(o.cfg, new_lat[:, None], new_key[:, None], o.table, pos, o.kv, o.idx)
    po, plo, to, tlo = oracle.index_full(o.cfg, *oF, o.idx, o.table, o.ctx)
    pool, pl, tk, tl = outs()
    k.csa2_index_full_append(g.cfg, dev(new_lat), dev(new_key), *qF, g.kv, g.idx, big, g.table,
                             g.ctx, pool, pl, tk, tl, g.ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(g.idx), o.idx), _first_diff(_np(g.idx), o.idx)
    assert np.array_equal(_np(g.kv), o.kv), _first_diff(_np(g.kv), o.kv)
    assert np.array_equal(_np(pool), po) and np.array_equal(_np(tk), to)
    assert np.array_equal(_np(tl), tlo) and np.array_equal(_np(pl), plo)


# ------------------------------------------------------------------ fused layer calls

@pytest.mark.parametrize("H,d,ctx,with_lat", [
    (4, 64, [5000], True),                      # one sequence (interleaved scan items)
    (4, 64, [700, 5000, 64, 1, 9], True),       # ragged batch
    (8, 128, [3000, 517, 9], True),             # the global append runs before the scan
    (1, 32, [300, 17], False),                  # one head, no main-KV append
    (4, 64, [150000, 3000], True),              # the two-phase Full selection (3 gather WGs)
])
def test_layer_calls_equal_the_separate_calls(H, d, ctx, with_lat):
    """csa2_decode_full_layer / _reindex_layer / _reuse_layer == the separate calls they
    stand for (query quantise, fused global append + Full index or Reindex, fused window
    append + attention at ctx_len - 1), bit for bit: cache and ring bytes, pool, top-k,
    attention output and log-sum-exp.  The token's rows are fresh values, unlike the cache's."""
    wl = si.small("lay", 340 + H + d + len(ctx), ctx, H_I=H, d_I=d, K_blk=32, k=96, W=64,
                  layers="FRU")
    table, nblk = make_table(wl.ctx, seed=wl.seed)
    g = GpuState(wl, table, nblk)
    B = wl.B
    i32 = dict(dtype=torch.int32, device="cuda")
    qf = [dev(si.layer_idx_q(wl, li).reshape(B, H * d)) for li in range(2)]
    w = [dev(si.layer_idx_w(wl, li)) for li in range(2)]
    qa = [g.attn_q(li) for li in range(3)]
    swa_row = [dev(si.normal(341, 10 + li, (B, wl.D))) for li in range(3)]
    tok_key = dev(si.normal(341, 20, (B, H * d)))
    tok_lat = dev(si.normal(341, 21, (B, wl.D))) if with_lat else None
    rings0 = [g.layer_swa(li) for li in range(3)]
    res = []
    for fused in (False, True):
        kv, idx = g.kv.clone(), g.idx.clone()
        rings = [r.clone() for r in rings0]
        pool = torch.full((B, wl.K_blk), -7, **i32)
        pl = torch.zeros(B, **i32)
        tk = [torch.full((B, wl.k), -7, **i32) for _ in range(2)]
        tl = [torch.zeros(B, **i32) for _ in range(2)]
        outs = [torch.full((B, wl.H_q, wl.D), float("nan"), device="cuda") for _ in range(3)]
        lses = [torch.full((B, wl.H_q), float("nan"), device="cuda") for _ in range(3)]
        wsa = torch.zeros_like(g.ws_attn)
        if fused:
            k.csa2_decode_full_layer(g.cfg, qf[0], w[0], tok_lat, tok_key, swa_row[0], qa[0], kv,
                                     idx, g.n_blocks, g.table, rings[0], g.C, g.ctx, pool, pl,
                                     tk[0], tl[0], outs[0], lses[0], g.ws, wsa)
            k.csa2_decode_reindex_layer(g.cfg, qf[1], w[1], swa_row[1], qa[1], kv, idx,
                                        g.n_blocks, g.table, rings[1], g.C, g.ctx, pool, pl,
                                        tk[1], tl[1], outs[1], lses[1], g.ws, wsa)
            k.csa2_decode_reuse_layer(g.cfg, swa_row[2], qa[2], kv, g.n_blocks, g.table, rings[2],
                                      g.C, g.ctx, tk[1], tl[1], outs[2], lses[2], wsa)
        else:
            pos = g.ctx - 1
            for li in range(3):
                if li < 2:
                    qc = torch.empty((B, H * d // 2), dtype=torch.uint8, device="cuda")
                    qs = torch.empty((B, H * d // 32), dtype=torch.uint8, device="cuda")
                    k.csa2_quantize_mxfp4(qf[li], qc, qs)
                if li == 0:
                    k.csa2_index_full_append(g.cfg, tok_lat, tok_key, qc, qs, w[0],
                                             kv if with_lat else None, idx, g.n_blocks, g.table,
                                             g.ctx, pool, pl, tk[0], tl[0], g.ws)
                elif li == 1:
                    k.csa2_index_reindex(g.cfg, qc, qs, w[1], idx, g.n_blocks, g.table, g.ctx,
                                         pool, pl, tk[1], tl[1], g.ws)
                t = min(li, 1)
                k.csa2_sparse_attn_append(g.cfg, swa_row[li], pos, qa[li], kv, g.n_blocks,
                                          g.table, rings[li], g.C, g.ctx, tk[t], tl[t], outs[li],
                                          lses[li], wsa)
        torch.cuda.synchronize()
        res.append([_np(x) for x in [kv, idx, *rings, pool, pl, *tk, *tl, *outs, *lses]])
    for i, (x, y) in enumerate(zip(*res)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (i, _first_diff(x, y))
    assert not np.array_equal(res[1][1], _np(g.idx)), "the layer call appended no key"
