"""Python access to the plain CPU oracle (``csa2_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` use this module.  The product path (``kv_cache_decode_csa2_amd``) never
imports it.

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "libcsa2_oracle.so")
BLK = 8

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wno-unused-function"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over independent units)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Cfg(C.Structure):
    _fields_ = [("n_idx_heads", C.c_int32), ("idx_dim", C.c_int32), ("kv_dim", C.c_int32),
                ("n_q_heads", C.c_int32), ("swa_window", C.c_int32),
                ("pool_blocks", C.c_int32), ("topk", C.c_int32), ("sm_scale", C.c_float),
                ("shared_key", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        d = C.c_double
        _lib.csa2o_fp4_value.restype = d
        _lib.csa2o_fp8_value.restype = d
        _lib.csa2o_e8m0_value.restype = d
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _check(rc, what):
    if rc == -5:
        raise ArithmeticError(f"oracle {what}: group exponent outside the exact fp32 range")
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {rc})")


def cfg(H_I, d_I, D, H_q, W, K_blk, k, sm_scale, shared_key=False) -> Cfg:
    return Cfg(H_I, d_I, D, H_q, W, K_blk, k, sm_scale, int(shared_key))


def cfg_of(wl) -> Cfg:
    return Cfg(wl.H_I, wl.d_I, wl.D, wl.H_q, wl.W, wl.K_blk, wl.k, wl.sm_scale,
               int(getattr(wl, "shared_key", False)))


# ------------------------------------------------------------------------- layout sizes

def key_heads(c: Cfg) -> int:
    """Indexer keys stored per position: one per head, or one shared by all heads."""
    return 1 if c.shared_key else c.n_idx_heads


def idx_block_bytes(c: Cfg) -> int:
    return BLK * key_heads(c) * (c.idx_dim // 2 + c.idx_dim // 32)


def kv_row_bytes(c: Cfg) -> int:
    return c.kv_dim // 2 + c.kv_dim // 32


def swa_row_bytes(c: Cfg) -> int:
    return c.kv_dim + c.kv_dim // 32


# ------------------------------------------------------------------------- codecs

def fp4_value(code: int) -> float:
    return lib().csa2o_fp4_value(int(code))


def fp8_value(code: int) -> float:
    return lib().csa2o_fp8_value(int(code))


def e8m0_value(code: int) -> float:
    return lib().csa2o_e8m0_value(int(code))


def quantize_mxfp4(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, dim = x.reshape(-1, x.shape[-1]).shape
    codes = np.zeros((rows, dim // 2), np.uint8)
    scales = np.zeros((rows, dim // 32), np.uint8)
    _check(lib().csa2o_quantize_mxfp4(_p(x), C.c_int64(rows), C.c_int32(dim), _p(codes),
                                       _p(scales)), "quantize_mxfp4")
    return codes, scales


def quantize_mxfp8(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, dim = x.reshape(-1, x.shape[-1]).shape
    codes = np.zeros((rows, dim), np.uint8)
    scales = np.zeros((rows, dim // 32), np.uint8)
    _check(lib().csa2o_quantize_mxfp8(_p(x), C.c_int64(rows), C.c_int32(dim), _p(codes),
                                       _p(scales)), "quantize_mxfp8")
    return codes, scales


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, dim = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((rows, dim), np.float64)
    _check(lib().csa2o_dequant_mxfp4(_p(codes), _p(scales), C.c_int64(rows), C.c_int32(dim),
                                      _p(out)), "dequant_mxfp4")
    return out


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, dim = codes.shape
    out = np.zeros((rows, dim), np.float64)
    _check(lib().csa2o_dequant_mxfp8(_p(codes), _p(scales), C.c_int64(rows), C.c_int32(dim),
                                      _p(out)), "dequant_mxfp8")
    return out


# ------------------------------------------------------------------------- caches

def append_global(c: Cfg, latent, idx_k, table, pos0, kv_cache, idx_cache):
    """latent [B, n, D] fp32 (or None), idx_k [B, n, KH, d_I] fp32 (or None), KH = key_heads(c)."""
    table = np.ascontiguousarray(table, np.int32)
    pos0 = np.ascontiguousarray(pos0, np.int32)
    B, maxb = table.shape
    src = latent if latent is not None else idx_k
    n = src.shape[1]
    lat = None if latent is None else np.ascontiguousarray(latent, np.float32)
    ik = None if idx_k is None else np.ascontiguousarray(idx_k, np.float32)
    nblk = (kv_cache.shape[0] if kv_cache is not None else idx_cache.shape[0])
    _check(lib().csa2o_append_global(C.byref(c), _p(lat), _p(ik), _p(table), C.c_int32(maxb),
                                      _p(pos0), C.c_int32(B), C.c_int32(n), _p(kv_cache),
                                      _p(idx_cache), C.c_int64(nblk)), "append_global")


def append_swa(c: Cfg, rows, pos0, swa_cache, C_slots):
    rows = np.ascontiguousarray(rows, np.float32)
    pos0 = np.ascontiguousarray(pos0, np.int32)
    B, n = rows.shape[0], rows.shape[1]
    _check(lib().csa2o_append_swa(C.byref(c), _p(rows), _p(pos0), C.c_int32(B), C.c_int32(n),
                                   _p(swa_cache), C.c_int32(C_slots)), "append_swa")


# ------------------------------------------------------------------------- indexer

def index_scores(c: Cfg, q_codes, q_scales, w, idx_cache, table_row, L) -> np.ndarray:
    out = np.zeros(max(L, 1), np.float32)
    table_row = np.ascontiguousarray(table_row, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    _check(lib().csa2o_index_scores(C.byref(c), _p(np.ascontiguousarray(q_codes)),
                                     _p(np.ascontiguousarray(q_scales)), _p(w), _p(idx_cache),
                                     _p(table_row), C.c_int32(L), _p(out)), "index_scores")
    return out[:L]


def block_scores(scores: np.ndarray, L: int) -> np.ndarray:
    nb = (L + BLK - 1) // BLK
    out = np.zeros(max(nb, 1), np.float32)
    s = np.ascontiguousarray(scores, np.float32)
    _check(lib().csa2o_block_scores(_p(s), C.c_int32(L), _p(out)), "block_scores")
    return out[:nb]


def index_full(c: Cfg, q_codes, q_scales, w, idx_cache, table, ctx_len, want_block_scores=False):
    table = np.ascontiguousarray(table, np.int32)
    ctx = np.ascontiguousarray(ctx_len, np.int32)
    B, maxb = table.shape
    pool = np.full((B, c.pool_blocks), -7, np.int32)
    pool_len = np.zeros(B, np.int32)
    topk = np.full((B, c.topk), -7, np.int32)
    topk_len = np.zeros(B, np.int32)
    bs = np.full((B, maxb), -np.inf, np.float32) if want_block_scores else None
    _check(lib().csa2o_index_full(
        C.byref(c), _p(np.ascontiguousarray(q_codes, np.uint8)),
        _p(np.ascontiguousarray(q_scales, np.uint8)), _p(np.ascontiguousarray(w, np.float32)),
        _p(idx_cache), C.c_int64(idx_cache.shape[0]), _p(table), C.c_int32(maxb), _p(ctx),
        C.c_int32(B), _p(pool), _p(pool_len), _p(topk), _p(topk_len), _p(bs)), "index_full")
    if want_block_scores:
        return pool, pool_len, topk, topk_len, bs
    return pool, pool_len, topk, topk_len


def index_reindex(c: Cfg, q_codes, q_scales, w, idx_cache, table, ctx_len, pool, pool_len):
    table = np.ascontiguousarray(table, np.int32)
    B, maxb = table.shape
    topk = np.full((B, c.topk), -7, np.int32)
    topk_len = np.zeros(B, np.int32)
    _check(lib().csa2o_index_reindex(
        C.byref(c), _p(np.ascontiguousarray(q_codes, np.uint8)),
        _p(np.ascontiguousarray(q_scales, np.uint8)), _p(np.ascontiguousarray(w, np.float32)),
        _p(idx_cache), C.c_int64(idx_cache.shape[0]), _p(table), C.c_int32(maxb),
        _p(np.ascontiguousarray(ctx_len, np.int32)), C.c_int32(B),
        _p(np.ascontiguousarray(pool, np.int32)), _p(np.ascontiguousarray(pool_len, np.int32)),
        _p(topk), _p(topk_len)), "index_reindex")
    return topk, topk_len


def index_prefill(c: Cfg, q_codes, q_scales, w, q_pos0, idx_cache, table_row):
    n_q = q_codes.shape[0]
    table = np.ascontiguousarray(np.asarray(table_row, np.int32).reshape(1, -1))
    maxb = table.shape[1]
    pool = np.full((n_q, c.pool_blocks), -7, np.int32)
    pool_len = np.zeros(n_q, np.int32)
    topk = np.full((n_q, c.topk), -7, np.int32)
    topk_len = np.zeros(n_q, np.int32)
    _check(lib().csa2o_index_prefill(
        C.byref(c), _p(np.ascontiguousarray(q_codes, np.uint8)),
        _p(np.ascontiguousarray(q_scales, np.uint8)), _p(np.ascontiguousarray(w, np.float32)),
        C.c_int32(q_pos0), C.c_int32(n_q), _p(idx_cache), C.c_int64(idx_cache.shape[0]),
        _p(table), C.c_int32(maxb), _p(pool), _p(pool_len), _p(topk), _p(topk_len)),
        "index_prefill")
    return pool, pool_len, topk, topk_len


# ------------------------------------------------------------------------- attention

def sparse_attn(c: Cfg, q_bf16, kv_cache, table, swa_cache, C_slots, ctx_len, topk, topk_len):
    """q_bf16 [B, H_q, D] uint16 bf16 bits -> (out [B, H_q, D] f64, lse [B, H_q] f64)."""
    table = np.ascontiguousarray(table, np.int32)
    B, maxb = table.shape
    q = np.ascontiguousarray(q_bf16, np.uint16)
    out = np.zeros((B, c.n_q_heads, c.kv_dim), np.float64)
    lse = np.zeros((B, c.n_q_heads), np.float64)
    _check(lib().csa2o_sparse_attn(
        C.byref(c), _p(q), _p(kv_cache), C.c_int64(kv_cache.shape[0]), _p(table),
        C.c_int32(maxb), _p(swa_cache), C.c_int32(C_slots),
        _p(np.ascontiguousarray(ctx_len, np.int32)), C.c_int32(B),
        _p(np.ascontiguousarray(topk, np.int32)), _p(np.ascontiguousarray(topk_len, np.int32)),
        _p(out), _p(lse)), "sparse_attn")
    return out, lse


def sparse_attn_prefill(c: Cfg, q_bf16, kv_cache, table_row, swa_ring, C_slots, q_pos0, topk,
                        topk_len):
    """Prefill attention: q_bf16 [n_q, H_q, D]; query i attends as a decode step at context
    length q_pos0 + i + 1 of the one sequence (its top-k rows + its window from the ring
    [C_slots, row]).  Returns (out [n_q, H_q, D] f64, lse [n_q, H_q] f64)."""
    q = np.ascontiguousarray(q_bf16, np.uint16)
    n_q = q.shape[0]
    table = np.ascontiguousarray(np.asarray(table_row, np.int32).reshape(-1))
    out = np.zeros((n_q, c.n_q_heads, c.kv_dim), np.float64)
    lse = np.zeros((n_q, c.n_q_heads), np.float64)
    _check(lib().csa2o_sparse_attn_prefill(
        C.byref(c), _p(q), _p(kv_cache), C.c_int64(kv_cache.shape[0]), _p(table),
        C.c_int32(table.shape[0]), _p(np.ascontiguousarray(swa_ring, np.uint8)),
        C.c_int32(C_slots), C.c_int32(q_pos0), C.c_int32(n_q),
        _p(np.ascontiguousarray(topk, np.int32)), _p(np.ascontiguousarray(topk_len, np.int32)),
        _p(out), _p(lse)), "sparse_attn_prefill")
    return out, lse


# ------------------------------------------------------------------------- workload driver

@dataclass
class OracleCaches:
    cfg: Cfg
    table: np.ndarray      # [B, maxb] int32
    ctx: np.ndarray        # [B] int32
    kv: np.ndarray         # [n_blocks, 8 * kv_row_bytes] uint8
    idx: np.ndarray        # [n_blocks, idx_block_bytes] uint8


def alloc_caches(c: Cfg, table: np.ndarray, n_blocks: int) -> tuple:
    kv = np.zeros((n_blocks, BLK * kv_row_bytes(c)), np.uint8)
    idx = np.zeros((n_blocks, idx_block_bytes(c)), np.uint8)
    return kv, idx


def alloc_swa(c: Cfg, B: int, C_slots: int) -> np.ndarray:
    return np.zeros((B, C_slots, swa_row_bytes(c)), np.uint8)
