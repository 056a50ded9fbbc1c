"""Test-side helpers: block tables and oracle-side cache construction for a workload.

Nothing here computes the method: caches are filled through the oracle's own append
calls, selections and attention come from the oracle or from independent brute force
written in the individual tests.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth_inputs as si

BLK = 8


def make_table(ctx, seed: int, permute: bool = True, spare: int = 3):
    """Block table [B, maxb] (-1 beyond each sequence's blocks) and the physical block
    count.  Physical blocks are a seeded permutation, with a few spare blocks unused."""
    nbs = [(int(L) + BLK - 1) // BLK for L in ctx]
    maxb = max(1, max(nbs) if nbs else 1)
    n_blocks = sum(nbs) + spare
    order = np.arange(n_blocks, dtype=np.int32)
    if permute:
        order = np.random.default_rng(np.random.SeedSequence([seed, 77])).permutation(n_blocks).astype(np.int32)
    table = np.full((len(ctx), maxb), -1, np.int32)
    k = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = order[k:k + nb]
        k += nb
    return table, n_blocks


class OracleState:
    """The oracle's own packed caches for a workload, filled from the seeded fp32 rows."""

    def __init__(self, wl: si.Workload, table: np.ndarray, n_blocks: int,
                 with_latent: bool = True):
        self.wl = wl
        self.cfg = oracle.cfg_of(wl)
        self.table = table
        self.ctx = np.asarray(wl.ctx, np.int32)
        self.kv, self.idx = oracle.alloc_caches(self.cfg, table, n_blocks)
        for b in range(wl.B):
            L = wl.ctx[b]
            if L == 0:
                continue
            keys = si.idx_keys(wl, b)
            lat = si.latent_rows(wl, b) if with_latent else None
            oracle.append_global(self.cfg, None if lat is None else lat[None], keys[None],
                                 table[b:b + 1], np.array([0], np.int32),
                                 self.kv if with_latent else None, self.idx)
        self.C = wl.W if wl.W > 0 else 1

    def layer_q(self, layer: int, mixed_sign: bool = False):
        wl = self.wl
        q = si.layer_idx_q(wl, layer).reshape(wl.B, wl.H_I * wl.d_I)
        qc, qs = oracle.quantize_mxfp4(q)
        w = si.layer_idx_w(wl, layer, mixed_sign)
        return qc, qs, w

    def layer_swa(self, layer: int) -> np.ndarray:
        wl = self.wl
        swa = oracle.alloc_swa(self.cfg, wl.B, self.C)
        for b in range(wl.B):
            L = wl.ctx[b]
            n = min(L, wl.W)
            if n == 0:
                continue
            rows = si.layer_swa_rows(wl, layer, b, n)
            oracle.append_swa(self.cfg, rows[None], np.array([L - n], np.int32),
                              swa[b:b + 1], self.C)
        return swa


def flat_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Independent brute force: the k best positions by (score desc, index asc)."""
    order = sorted(range(len(scores)), key=lambda p: (-float(scores[p]), p))
    return np.array(sorted(order[:k]), np.int64)


def hierarchical_topk(scores: np.ndarray, K_blk: int, k: int):
    """Independent brute force of the two-stage definition: block maxima over 8
    positions, the K_blk best blocks, then the k best positions inside them."""
    L = len(scores)
    nb = (L + BLK - 1) // BLK
    bmax = [max(float(scores[p]) for p in range(j * BLK, min(L, (j + 1) * BLK))) for j in range(nb)]
    blocks = sorted(sorted(range(nb), key=lambda j: (-bmax[j], j))[:K_blk])
    cand = [p for j in blocks for p in range(j * BLK, min(L, (j + 1) * BLK))]
    best = sorted(cand, key=lambda p: (-float(scores[p]), p))[:k]
    return np.array(blocks, np.int64), np.array(sorted(best), np.int64)
