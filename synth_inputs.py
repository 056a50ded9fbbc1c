"""Seeded synthetic inputs for the CSA2 decode path (shared by tests, bench and smoke).

This module only draws random numbers and names workload shapes.  It holds none of
the method's arithmetic: no quantisation, no scoring, no selection, no attention.
Both the GPU path and the CPU oracle consume exactly the arrays produced here.

Every tensor is drawn from ``numpy.random.default_rng`` seeded with
``SeedSequence([seed, tensor_id, chunk])``, where ``chunk`` indexes fixed slices of
``CHUNK`` elements.  The result is therefore independent of how many threads fill it.

Workloads (the five decode/prefill cases the CSA2 pages motivate; the pages give no
model tensors, so every tensor is synthetic):

* tiny      : batch 1, context 4096, indexer 4 heads x 64, pool 64 blocks, top-128,
              latent 512, 16 query heads, window 128; layers F, R, U.
* b8_64k    : batch 8, context 65536 each, indexer 8 x 128, pool 2048, top-512,
              64 query heads; layers F, R, U, R, U.
* long_1m   : batch 1, context 1,048,576, indexer 4 x 64, pool 2048, top-512,
              16 query heads; layers F, R, U; 64 planted high-similarity blocks.
* ragged64  : batch 64, context lengths uniform on [4096, 131072]; dims as long_1m.
* prefill   : 4096 queries at the end of a 262,144-token causal context,
              indexer 8 x 128, pool 2048, top-512, 64 query heads.
* spec_1m   : speculative verification, 1 + 5 draft tokens at the end of a
              1,048,576-token context (6 causal queries); dims as long_1m.
* b8_64k_shared, long_1m_shared : the shared-key indexer variant (one 128-dim key per
              position scored by 8 query heads) at the batch-8 64K and one-sequence 1M
              sizes.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded slice

# tensor ids (stable; part of the recipe)
T_IDX_K = 1        # indexer keys, fp32 [B, L, H_I, d_I]
T_LATENT = 2       # main-KV latent rows, fp32 [B, L, D]
T_PLANT = 3        # planted block choice (long_1m)
T_PLANT_NOISE = 4  # noise added to planted keys
T_CTX = 5          # ragged context lengths
T_LAYER = 100      # per-layer tensors: T_LAYER + 16 * layer + k


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(seed: int, tensor_id: int, n: int, kind: str, lo=0.0, hi=1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        g = np.random.default_rng(np.random.SeedSequence([seed, tensor_id, c]))
        sl = out[c * CHUNK:min(n, (c + 1) * CHUNK)]
        if kind == "normal":
            g.standard_normal(sl.shape[0], dtype=np.float32, out=sl)
        else:
            sl[:] = g.uniform(lo, hi, sl.shape[0]).astype(np.float32)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def normal(seed: int, tensor_id: int, shape) -> np.ndarray:
    """fp32 N(0, 1) array of ``shape``."""
    n = int(np.prod(shape))
    return _fill(seed, tensor_id, n, "normal").reshape(shape)


def uniform(seed: int, tensor_id: int, shape, lo: float, hi: float) -> np.ndarray:
    """fp32 U(lo, hi) array of ``shape``."""
    n = int(np.prod(shape))
    return _fill(seed, tensor_id, n, "uniform", lo, hi).reshape(shape)


def integers(seed: int, tensor_id: int, n: int, lo: int, hi_inclusive: int) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([seed, tensor_id]))
    return g.integers(lo, hi_inclusive + 1, n, dtype=np.int64)


def choice(seed: int, tensor_id: int, population: int, k: int) -> np.ndarray:
    """k distinct integers from [0, population), sorted ascending."""
    g = np.random.default_rng(np.random.SeedSequence([seed, tensor_id]))
    return np.sort(g.choice(population, size=k, replace=False)).astype(np.int64)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 storage (uint16 bit patterns) of an fp32 array, via torch's own conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    ctx: list            # context length per sequence (positions 0 .. L-1 visible)
    H_I: int             # indexer heads
    d_I: int             # indexer head dim
    K_blk: int           # pool blocks
    k: int               # final top-k
    D: int = 512         # main-KV latent dim
    H_q: int = 16        # attention query heads
    W: int = 128         # sliding window
    layers: str = "FRU"  # layer modes of one decode group
    planted: int = 0     # planted high-similarity blocks (long_1m)
    n_q: int = 0         # prefill queries (prefill only)
    shared_key: bool = False  # one d_I indexer key per position, scored by all H_I heads
    extra: dict = field(default_factory=dict)

    @property
    def key_heads(self) -> int:
        return 1 if self.shared_key else self.H_I

    @property
    def sm_scale(self) -> float:
        return float(1.0 / np.sqrt(self.D))

    @property
    def max_ctx(self) -> int:
        return int(max(self.ctx)) if self.ctx else 0


def workload(name: str) -> Workload:
    if name == "tiny":
        return Workload("tiny", 1, 1, [4096], 4, 64, 64, 128, H_q=16)
    if name == "b8_64k":
        return Workload("b8_64k", 2, 8, [65536] * 8, 8, 128, 2048, 512, H_q=64, layers="FRURU")
    if name == "long_1m":
        return Workload("long_1m", 3, 1, [1 << 20], 4, 64, 2048, 512, H_q=16, planted=64)
    if name == "ragged64":
        lens = integers(4, T_CTX, 64, 4096, 131072)
        return Workload("ragged64", 4, 64, [int(v) for v in lens], 4, 64, 2048, 512, H_q=16)
    if name == "prefill":
        return Workload("prefill", 5, 1, [262144], 8, 128, 2048, 512, H_q=64, n_q=4096)
    if name == "spec_1m":
        return Workload("spec_1m", 6, 1, [1 << 20], 4, 64, 2048, 512, H_q=16, n_q=6)
    if name == "b8_64k_shared":  # the shared-key indexer at the batch-8 decode dims
        return Workload("b8_64k_shared", 7, 8, [65536] * 8, 8, 128, 2048, 512, H_q=64,
                        layers="FRURU", shared_key=True)
    if name == "long_1m_shared":  # the shared-key indexer, 8 heads x 128, one 1M sequence
        return Workload("long_1m_shared", 8, 1, [1 << 20], 8, 128, 2048, 512, H_q=16,
                        shared_key=True)
    raise KeyError(name)


def small(name: str, seed: int, ctx, H_I=4, d_I=64, K_blk=16, k=32, H_q=16, D=512, W=128,
          layers="FRU", planted=0, shared_key=False) -> Workload:
    """A reduced workload for tests that the oracle finishes in seconds."""
    ctx = list(ctx)
    return Workload(name, seed, len(ctx), ctx, H_I, d_I, K_blk, k, D=D, H_q=H_q, W=W,
                    layers=layers, planted=planted, shared_key=shared_key)


# ----------------------------------------------------------------------------- tensors

def idx_keys(wl: Workload, b: int, L: int | None = None) -> np.ndarray:
    """fp32 indexer keys of sequence b, shape [L, KH, d_I] (before quantisation), KH = H_I
    keys per position, or 1 with a shared key."""
    L = wl.ctx[b] if L is None else L
    x = normal(wl.seed, T_IDX_K + 1000 * b, (L, wl.key_heads, wl.d_I))
    if wl.planted:
        plant_keys(wl, b, x)
    return x


def planted_blocks(wl: Workload, b: int) -> np.ndarray:
    nb = (wl.ctx[b] + 7) // 8
    return choice(wl.seed, T_PLANT + 1000 * b, nb, wl.planted)


def plant_keys(wl: Workload, b: int, x: np.ndarray) -> None:
    """Planted blocks: every key row of the block is the Full layer's fp32 indexer query
    plus 0.5 * N(0, 1) noise."""
    blocks = planted_blocks(wl, b)
    qF = layer_idx_q(wl, 0)[b]                       # [H_I, d_I]
    noise = normal(wl.seed, T_PLANT_NOISE + 1000 * b, (len(blocks), 8, wl.H_I, wl.d_I))
    L = x.shape[0]
    for i, blk in enumerate(blocks):
        for s in range(8):
            p = int(blk) * 8 + s
            if p < L:
                x[p] = qF + np.float32(0.5) * noise[i, s]


def latent_rows(wl: Workload, b: int, L: int | None = None) -> np.ndarray:
    """fp32 main-KV latent rows of sequence b, shape [L, D]."""
    L = wl.ctx[b] if L is None else L
    return normal(wl.seed, T_LATENT + 1000 * b, (L, wl.D))


def layer_idx_q(wl: Workload, layer: int) -> np.ndarray:
    """fp32 indexer query of a layer, [B, H_I, d_I].  A Reindex layer of a planted
    workload draws q = q_Full + 0.5 * N(0, 1) so that it also prefers the plant."""
    base = T_LAYER + 16 * layer
    q = normal(wl.seed, base + 0, (wl.B, wl.H_I, wl.d_I))
    if wl.planted and layer > 0:
        q = layer_idx_q(wl, 0) + np.float32(0.5) * q
    return q


def layer_idx_w(wl: Workload, layer: int, mixed_sign: bool = False) -> np.ndarray:
    """fp32 indexer head weights of a layer, [B, H_I], U(0.5, 1.5) (or U(-1.5, 1.5))."""
    base = T_LAYER + 16 * layer
    lo = -1.5 if mixed_sign else 0.5
    return uniform(wl.seed, base + 1, (wl.B, wl.H_I), lo, 1.5)


def layer_attn_q(wl: Workload, layer: int, n_rows: int | None = None) -> np.ndarray:
    """bf16 bits of the attention query of a layer, [n_rows or B, H_q, D]."""
    base = T_LAYER + 16 * layer
    n = wl.B if n_rows is None else n_rows
    return to_bf16_bits(normal(wl.seed, base + 2, (n, wl.H_q, wl.D)))


def layer_swa_rows(wl: Workload, layer: int, b: int, n: int) -> np.ndarray:
    """fp32 sliding-window rows of a layer for the last n positions of sequence b, [n, D]."""
    base = T_LAYER + 16 * layer
    return normal(wl.seed, base + 3 + 1000 * b, (n, wl.D))


# ----------------------------------------------------------------------------- prefill

def prefill_idx_q(wl: Workload, layer: int, n_q: int) -> np.ndarray:
    """fp32 indexer queries of the n_q prefill tokens of a layer, [n_q, H_I, d_I], N(0, 1)."""
    return normal(wl.seed, T_LAYER + 16 * layer + 4, (n_q, wl.H_I, wl.d_I))


def prefill_idx_w(wl: Workload, layer: int, n_q: int) -> np.ndarray:
    """fp32 indexer head weights of the n_q prefill tokens of a layer, [n_q, H_I],
    U(0.5, 1.5)."""
    return uniform(wl.seed, T_LAYER + 16 * layer + 5, (n_q, wl.H_I), 0.5, 1.5)


def prefill_attn_q(wl: Workload, layer: int, n_q: int) -> np.ndarray:
    """bf16 bits of the attention queries of the n_q prefill tokens, [n_q, H_q, D]."""
    return to_bf16_bits(normal(wl.seed, T_LAYER + 16 * layer + 6, (n_q, wl.H_q, wl.D)))
