"""GPU-side state for parity tests and the bench: caches filled through the C ABI from the
same seeded fp32 rows the oracle packs."""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_decode_csa2_amd as k
import synth_inputs as si

BLK = 8
APPEND_CHUNK = 1 << 17  # positions per append call (bounds host memory)


def cfg_of(wl: si.Workload) -> k.csa2_config:
    return k.config(wl.H_I, wl.d_I, wl.D, wl.H_q, wl.W, wl.K_blk, wl.k, wl.sm_scale,
                    wl.shared_key)


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


class GpuState:
    def __init__(self, wl: si.Workload, table: np.ndarray, n_blocks: int, with_latent=True):
        self.wl = wl
        self.cfg = cfg_of(wl)
        lay = k.csa2_layout(self.cfg)
        self.lay = lay
        self.n_blocks = n_blocks
        self.table = dev(table.astype(np.int32))
        self.ctx = dev(np.asarray(wl.ctx, np.int32))
        self.kv = torch.zeros((n_blocks, lay.kv_block_bytes), dtype=torch.uint8, device="cuda")
        self.idx = torch.zeros((n_blocks, lay.idx_block_bytes), dtype=torch.uint8, device="cuda")
        for b in range(wl.B):
            L = wl.ctx[b]
            if L == 0:
                continue
            keys = si.idx_keys(wl, b)
            lat = si.latent_rows(wl, b) if with_latent else None
            for p0 in range(0, L, APPEND_CHUNK):
                n = min(APPEND_CHUNK, L - p0)
                kt = dev(keys[p0:p0 + n])
                lt = dev(lat[p0:p0 + n]) if lat is not None else None
                k.csa2_append_global(self.cfg, lt, kt, self.table[b:b + 1], n_blocks,
                                     dev(np.array([p0], np.int32)), n,
                                     self.kv if lt is not None else None, self.idx)
            del keys, lat
        self.C = wl.W if wl.W > 0 else 1
        maxb = table.shape[1]
        self.ws = torch.zeros(k.csa2_workspace_bytes(self.cfg, k.CSA2_OP_INDEX_FULL, wl.B, maxb),
                              dtype=torch.uint8, device="cuda")
        self.ws_attn = torch.zeros(
            k.csa2_workspace_bytes(self.cfg, k.CSA2_OP_SPARSE_ATTN, wl.B, maxb),
            dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    # ---- per-layer inputs
    def layer_q(self, layer: int, mixed_sign: bool = False):
        wl = self.wl
        q = dev(si.layer_idx_q(wl, layer).reshape(wl.B, wl.H_I * wl.d_I))
        qc = torch.empty((wl.B, wl.H_I * wl.d_I // 2), dtype=torch.uint8, device="cuda")
        qs = torch.empty((wl.B, wl.H_I * wl.d_I // 32), dtype=torch.uint8, device="cuda")
        k.csa2_quantize_mxfp4(q, qc, qs)
        w = dev(si.layer_idx_w(wl, layer, mixed_sign))
        return qc, qs, w

    def layer_swa(self, layer: int):
        wl = self.wl
        swa = torch.zeros((wl.B, self.C, self.lay.swa_row_bytes), dtype=torch.uint8, device="cuda")
        for b in range(wl.B):
            L = wl.ctx[b]
            n = min(L, wl.W)
            if n == 0:
                continue
            rows = dev(si.layer_swa_rows(wl, layer, b, n))
            one = swa[b:b + 1]
            k.csa2_append_swa(self.cfg, rows, dev(np.array([L - n], np.int32)), n, one, self.C)
        return swa

    def attn_q(self, layer: int):
        return dev(si.layer_attn_q(self.wl, layer).view(np.int16))

    # ---- calls
    def index_full(self, qc, qs, w):
        wl = self.wl
        pool = torch.full((wl.B, wl.K_blk), -7, dtype=torch.int32, device="cuda")
        pl = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
        topk = torch.full((wl.B, wl.k), -7, dtype=torch.int32, device="cuda")
        tl = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
        k.csa2_index_full(self.cfg, qc, qs, w, self.idx, self.n_blocks, self.table, self.ctx,
                          pool, pl, topk, tl, self.ws)
        return pool, pl, topk, tl

    def index_reindex(self, qc, qs, w, pool, pl):
        wl = self.wl
        topk = torch.full((wl.B, wl.k), -7, dtype=torch.int32, device="cuda")
        tl = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
        k.csa2_index_reindex(self.cfg, qc, qs, w, self.idx, self.n_blocks, self.table, self.ctx,
                             pool, pl, topk, tl, self.ws)
        return topk, tl

    def index_scores(self, qc, qs, w):
        wl = self.wl
        maxb = self.table.shape[1]
        sc = torch.full((wl.B, maxb * BLK), float("nan"), dtype=torch.float32, device="cuda")
        bs = torch.full((wl.B, maxb), float("nan"), dtype=torch.float32, device="cuda")
        k.csa2_index_scores(self.cfg, qc, qs, w, self.idx, self.n_blocks, self.table, self.ctx,
                            sc, bs)
        return sc, bs

    def attn(self, q, swa, topk, tl):
        wl = self.wl
        out = torch.full((wl.B, wl.H_q, wl.D), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((wl.B, wl.H_q), float("nan"), dtype=torch.float32, device="cuda")
        k.csa2_sparse_attn(self.cfg, q, self.kv, self.n_blocks, self.table, swa, self.C, self.ctx,
                           topk, tl, out, lse, self.ws_attn)
        return out, lse


def attn_close(out, lse, ref_out, ref_lse, tol=2e-3):
    """Per (sequence, head) row: max_d |o - r| <= tol * max_d |r|; |dlse| <= tol*max(1,|r|).
    Returns (ok, worst relative row error, worst lse error)."""
    out = np.asarray(out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    err = np.abs(out - ref_out).max(-1)
    scale = np.abs(ref_out).max(-1)
    empty = np.isneginf(ref_lse)
    rel = np.where(empty, err, err / np.maximum(scale, 1e-300))
    with np.errstate(invalid="ignore"):
        lerr = np.where(empty, np.where(np.isneginf(lse), 0.0, np.inf),
                        np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))
    ok = bool(np.all(rel <= tol) and np.all(lerr <= tol) and np.all(out[empty] == 0))
    return ok, float(rel.max(initial=0.0)), float(np.nanmax(lerr, initial=0.0))


def prefill_q(wl: si.Workload, layer: int, n_q: int, scale_fn=None):
    """Prefill indexer queries on the GPU: (q_codes, q_scales, w).  scale_fn, if given,
    edits the fp32 queries first (numpy, in place)."""
    q = si.prefill_idx_q(wl, layer, n_q)
    if scale_fn is not None:
        scale_fn(q)
    q = dev(q.reshape(n_q, wl.H_I * wl.d_I))
    qc = torch.empty((n_q, wl.H_I * wl.d_I // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((n_q, wl.H_I * wl.d_I // 32), dtype=torch.uint8, device="cuda")
    k.csa2_quantize_mxfp4(q, qc, qs)
    return qc, qs, dev(si.prefill_idx_w(wl, layer, n_q))


def index_prefill(g: GpuState, qc, qs, w, q_pos0: int, ws=None):
    """csa2_index_prefill over sequence 0 of g: (pool, pool_len, topk, topk_len)."""
    wl = g.wl
    n_q = qc.shape[0]
    maxb = g.table.shape[1]
    if ws is None:
        ws = torch.empty(k.csa2_workspace_bytes(g.cfg, k.CSA2_OP_INDEX_PREFILL, n_q, maxb),
                         dtype=torch.uint8, device="cuda")
    pool = torch.full((n_q, wl.K_blk), -7, dtype=torch.int32, device="cuda")
    pl = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    topk = torch.full((n_q, wl.k), -7, dtype=torch.int32, device="cuda")
    tl = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    k.csa2_index_prefill(g.cfg, qc, qs, w, q_pos0, g.idx, g.n_blocks, g.table[0].contiguous(),
                         pool, pl, topk, tl, ws)
    return pool, pl, topk, tl
