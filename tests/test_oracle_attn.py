"""Pins of the oracle's sparse attention + window merge.

Rows are dequantised independently (quantise the seeded fp32 rows, then dequantise; both
codecs are pinned in test_oracle_codecs.py), so these tests also pin the oracle's reading
of the main-KV block layout and the window ring.  References: torch's
scaled_dot_product_attention and logsumexp in float64 on the CPU, plus closed forms.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from harness import OracleState, make_table


def _rows_main(wl, b, positions):
    lat = si.latent_rows(wl, b)
    c, s = oracle.quantize_mxfp4(lat[positions])
    return oracle.dequant_mxfp4(c, s)


def _rows_win(wl, layer, b):
    L = wl.ctx[b]
    n = min(L, wl.W)
    rows = si.layer_swa_rows(wl, layer, b, n)
    c, s = oracle.quantize_mxfp8(rows)
    return oracle.dequant_mxfp8(c, s)


def _sdpa(q, rows, scale):
    """q [H, D] float64, rows [n, D] float64 -> (out [H, D], lse [H])."""
    qt = torch.from_numpy(q)[None, :, None, :]            # [1, H, 1, D]
    kt = torch.from_numpy(rows)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    lse = torch.logsumexp(scale * (torch.from_numpy(q) @ torch.from_numpy(rows).T), dim=-1)
    return out[0, :, 0].numpy(), lse.numpy()


def _qf64(qbits):
    return (qbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup(ctx, seed, k=24, W=16, H_q=4):
    wl = si.small("attn", seed, ctx, H_I=2, d_I=64, K_blk=8, k=k, H_q=H_q, W=W)
    table, nblk = make_table(ctx, seed)
    st = OracleState(wl, table, nblk, with_latent=True)
    return wl, st


@pytest.mark.parametrize("ctx,W", [([300, 40, 9], 16), ([1000], 128), ([5], 128)])
def test_attention_matches_sdpa(ctx, W):
    wl, st = _setup(ctx, 31, W=W)
    rng = np.random.default_rng(5)
    B, k = wl.B, wl.k
    topk = np.full((B, k), -1, np.int32)
    tl = np.zeros(B, np.int32)
    for b, L in enumerate(ctx):
        n = min(k, L)
        sel = np.sort(rng.choice(L, n, replace=False))
        topk[b, :n] = sel
        tl[b] = n
    q = si.layer_attn_q(wl, 0)
    swa = st.layer_swa(0)
    out, lse = oracle.sparse_attn(st.cfg, q, st.kv, st.table, swa, st.C, st.ctx, topk, tl)
    for b in range(B):
        rows = np.concatenate([_rows_main(wl, b, topk[b, :tl[b]]), _rows_win(wl, 0, b)])
        ro, rl = _sdpa(_qf64(q[b]), rows, float(np.float32(wl.sm_scale)))
        assert np.allclose(out[b], ro, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[b], rl, rtol=1e-12, atol=1e-12)


def test_window_only_is_dense_attention_over_last_rows():
    wl, st = _setup([77], 32, W=32)
    topk = np.full((1, wl.k), -1, np.int32)
    q = si.layer_attn_q(wl, 1)
    swa = st.layer_swa(1)
    out, lse = oracle.sparse_attn(st.cfg, q, st.kv, st.table, swa, st.C, st.ctx, topk,
                                  np.zeros(1, np.int32))
    ro, rl = _sdpa(_qf64(q[0]), _rows_win(wl, 1, 0), float(np.float32(wl.sm_scale)))
    assert np.allclose(out[0], ro, rtol=1e-12, atol=1e-12) and np.allclose(lse[0], rl)


def test_single_row_returns_that_row():
    wl, st = _setup([50], 33, W=0)
    topk = np.full((1, wl.k), -1, np.int32)
    topk[0, 0] = 17
    q = si.layer_attn_q(wl, 0)
    swa = oracle.alloc_swa(st.cfg, 1, 1)
    out, lse = oracle.sparse_attn(st.cfg, q, st.kv, st.table, swa, 1, st.ctx, topk,
                                  np.ones(1, np.int32))
    row = _rows_main(wl, 0, [17])[0]
    assert np.array_equal(out[0], np.broadcast_to(row, out[0].shape))
    assert np.allclose(lse[0], float(np.float32(wl.sm_scale)) * (_qf64(q[0]) @ row), rtol=1e-13)


def test_zero_query_gives_mean_of_rows_and_log_count():
    wl, st = _setup([64], 34, W=8)
    topk = np.full((1, wl.k), -1, np.int32)
    topk[0, :3] = [2, 40, 56]
    q = np.zeros((1, wl.H_q, wl.D), np.uint16)
    swa = st.layer_swa(0)
    out, lse = oracle.sparse_attn(st.cfg, q, st.kv, st.table, swa, st.C, st.ctx, topk,
                                  np.array([3], np.int32))
    rows = np.concatenate([_rows_main(wl, 0, [2, 40, 56]), _rows_win(wl, 0, 0)])
    assert np.allclose(out[0], rows.mean(0), rtol=1e-13, atol=1e-15)
    assert np.allclose(lse[0], np.log(11.0))


def test_no_dedup_padding_and_empty():
    wl, st = _setup([20, 0], 35, W=8)
    topk = np.full((2, wl.k), -1, np.int32)
    topk[0, :3] = [3, -1, 19]       # 19 is also a window position; -1 is padding
    q = si.layer_attn_q(wl, 0)
    swa = st.layer_swa(0)
    out, lse = oracle.sparse_attn(st.cfg, q, st.kv, st.table, swa, st.C, st.ctx, topk,
                                  np.array([3, 0], np.int32))
    rows = np.concatenate([_rows_main(wl, 0, [3, 19]), _rows_win(wl, 0, 0)])
    ro, rl = _sdpa(_qf64(q[0]), rows, float(np.float32(wl.sm_scale)))
    assert np.allclose(out[0], ro, rtol=1e-12, atol=1e-12) and np.allclose(lse[0], rl)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_prefill_attention_is_per_query_dense_attention():
    """Prefill query i at position t = q_pos0 + i attends to its own top-k main rows and to
    the window rows max(0, t+1-W) .. t of the shared ring: against SDPA over exactly those
    dequantised rows, per query."""
    L, n_q, W = 260, 20, 16
    wl, st = _setup([L], 37, k=12, W=W, H_q=4)
    q_pos0 = L - n_q
    C = n_q + W  # the ring keeps every window row of the chunk
    first = q_pos0 - W + 1
    rows = si.layer_swa_rows(wl, 0, 0, L - first)
    ring = oracle.alloc_swa(st.cfg, 1, C)
    oracle.append_swa(st.cfg, rows[None], np.array([first], np.int32), ring, C)
    rc, rs = oracle.quantize_mxfp8(rows)
    win = oracle.dequant_mxfp8(rc, rs)                 # row r = position first + r
    rng = np.random.default_rng(9)
    topk = np.full((n_q, wl.k), -1, np.int32)
    tl = np.zeros(n_q, np.int32)
    for i in range(n_q):
        t = q_pos0 + i
        n = int(rng.integers(0, wl.k + 1))
        sel = np.sort(rng.choice(t + 1, n, replace=False))
        topk[i, :n], tl[i] = sel, n
    qb = si.prefill_attn_q(wl, 0, n_q)
    out, lse = oracle.sparse_attn_prefill(st.cfg, qb, st.kv, st.table[0], ring[0], C, q_pos0,
                                          topk, tl)
    for i in range(n_q):
        t = q_pos0 + i
        w0 = max(0, t + 1 - W)
        main = _rows_main(wl, 0, topk[i, :tl[i]])
        rr = np.concatenate([main, win[w0 - first:t + 1 - first]])
        ro, rl = _sdpa(_qf64(qb[i]), rr, float(np.float32(wl.sm_scale)))
        np.testing.assert_allclose(out[i], ro, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[i], rl, rtol=1e-12)
