"""ctypes binding of libcsa2.so: the C entry points under the same names, taking torch
device tensors.  Argument marshalling only -- every step of the path runs in the HIP
kernels of the library.  torch supplies device memory and the current stream.

If the library is not built, importing works but every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

CSA2_OK, CSA2_ERR_INVALID, CSA2_ERR_UNSUPPORTED, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP = 0, -1, -2, -3, -4
CSA2_ERR_SCRATCH = -5
CSA2_OP_INDEX_FULL, CSA2_OP_INDEX_REINDEX, CSA2_OP_SPARSE_ATTN, CSA2_OP_INDEX_PREFILL = 1, 2, 3, 4
CSA2_BLOCK = 8

EXPORTS = [
    "csa2_layout", "csa2_workspace_bytes", "csa2_quantize_mxfp4", "csa2_quantize_mxfp8",
    "csa2_dequant_mxfp4", "csa2_dequant_mxfp8", "csa2_append_global", "csa2_append_swa",
    "csa2_index_scores", "csa2_index_full", "csa2_index_full_scan", "csa2_index_full_finish",
    "csa2_index_reindex", "csa2_index_prefill", "csa2_index_prefill_scan",
    "csa2_index_prefill_finish", "csa2_sparse_attn", "csa2_sparse_attn_append",
    "csa2_sparse_attn_prefill", "csa2_index_full_append", "csa2_blocks_gather",
    "csa2_blocks_scatter", "csa2_sparse_attn_noalloc", "csa2_decode_full_layer",
    "csa2_decode_reindex_layer", "csa2_decode_reuse_layer", "csa2_status_str",
]


class csa2_config(C.Structure):
    _fields_ = [("n_idx_heads", C.c_int32), ("idx_dim", C.c_int32), ("kv_dim", C.c_int32),
                ("n_q_heads", C.c_int32), ("swa_window", C.c_int32),
                ("pool_blocks", C.c_int32), ("topk", C.c_int32), ("sm_scale", C.c_float),
                ("shared_key", C.c_int32)]


class csa2_layout_info(C.Structure):
    _fields_ = [("idx_block_bytes", C.c_size_t), ("kv_row_bytes", C.c_size_t),
                ("kv_block_bytes", C.c_size_t), ("swa_row_bytes", C.c_size_t)]


class Csa2Error(RuntimeError):
    def __init__(self, name, status):
        super().__init__(f"{name}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def load() -> C.CDLL:
    """Load libcsa2.so; raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                              "the CSA2 path has no CPU fallback")
        lib = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        cfgp = C.POINTER(csa2_config)
        sig = {
            "csa2_layout": [cfgp, C.POINTER(csa2_layout_info)],
            "csa2_workspace_bytes": [cfgp, C.c_int, i32, i32, C.POINTER(C.c_size_t)],
            "csa2_quantize_mxfp4": [vp, i64, i32, vp, vp, vp],
            "csa2_quantize_mxfp8": [vp, i64, i32, vp, vp, vp],
            "csa2_dequant_mxfp4": [vp, vp, i64, i32, vp, vp],
            "csa2_dequant_mxfp8": [vp, vp, i64, i32, vp, vp],
            "csa2_append_global": [cfgp, vp, vp, vp, i32, i64, vp, i32, i32, vp, vp, vp],
            "csa2_append_swa": [cfgp, vp, vp, i32, i32, vp, i32, vp],
            "csa2_blocks_gather": [vp, i64, i64, vp, i32, vp, vp],
            "csa2_blocks_scatter": [vp, vp, i32, vp, i64, i64, vp],
            "csa2_index_scores": [cfgp, vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, vp],
            "csa2_index_full": [cfgp, vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp, vp,
                                sz, vp],
            "csa2_index_full_scan": [cfgp, vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, sz, vp],
            "csa2_index_full_finish": [cfgp, vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, vp,
                                       vp, vp, sz, vp],
            "csa2_index_full_append": [cfgp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, i32,
                                       vp, vp, vp, vp, vp, sz, vp],
            "csa2_index_reindex": [cfgp, vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp,
                                   vp, sz, vp],
            "csa2_index_prefill": [cfgp, vp, vp, vp, i32, i32, vp, i64, vp, i32, vp, vp, vp, vp,
                                   vp, sz, vp],
            "csa2_index_prefill_scan": [cfgp, vp, vp, vp, i32, i32, vp, i64, vp, i32, vp, sz, vp],
            "csa2_index_prefill_finish": [cfgp, vp, vp, vp, i32, i32, vp, i64, vp, i32, vp, vp, vp,
                                          vp, vp, sz, vp],
            "csa2_sparse_attn": [cfgp, vp, vp, i64, vp, i32, vp, i32, vp, i32, vp, vp, vp, vp, vp,
                                 sz, vp],
            "csa2_decode_full_layer": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, i32,
                                       vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp],
            "csa2_decode_reindex_layer": [cfgp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, i32, vp,
                                          i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp],
            "csa2_decode_reuse_layer": [cfgp, vp, vp, vp, i64, vp, i32, vp, i32, vp, i32, vp, vp,
                                        vp, vp, vp, sz, vp],
            "csa2_sparse_attn_noalloc": [cfgp, vp, vp, i64, vp, i32, vp, i32, vp, i32, vp, vp, vp,
                                         vp, vp],
            "csa2_sparse_attn_prefill": [cfgp, vp, vp, i64, vp, i32, vp, i32, i32, i32, vp, vp,
                                         vp, vp, vp, sz, vp],
            "csa2_sparse_attn_append": [cfgp, vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, i32, vp, vp,
                                        vp, vp, vp, sz, vp],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = C.c_int
        lib.csa2_status_str.argtypes = [C.c_int]
        lib.csa2_status_str.restype = C.c_char_p
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().csa2_status_str(int(status)).decode()


def _p(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if not t.is_cuda:
            raise ValueError("csa2: tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("csa2: tensors must be contiguous")
        return C.c_void_p(t.data_ptr())
    return C.c_void_p(int(t))


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _call(name, *args):
    st = getattr(load(), name)(*args)
    if st != CSA2_OK:
        raise Csa2Error(name, st)


def config(H_I, d_I, D, H_q, W, K_blk, k, sm_scale, shared_key=False) -> csa2_config:
    return csa2_config(H_I, d_I, D, H_q, W, K_blk, k, sm_scale, int(shared_key))


def csa2_layout(cfg: csa2_config) -> csa2_layout_info:
    out = csa2_layout_info()
    _call("csa2_layout", C.byref(cfg), C.byref(out))
    return out


def csa2_workspace_bytes(cfg: csa2_config, op: int, batch: int, maxb: int) -> int:
    out = C.c_size_t(0)
    _call("csa2_workspace_bytes", C.byref(cfg), int(op), int(batch), int(maxb), C.byref(out))
    return out.value


def csa2_quantize_mxfp4(x, codes, scales, stream=None):
    rows, dim = x.numel() // x.shape[-1], x.shape[-1]
    _call("csa2_quantize_mxfp4", _p(x), rows, dim, _p(codes), _p(scales), _stream(stream))


def csa2_quantize_mxfp8(x, codes, scales, stream=None):
    rows, dim = x.numel() // x.shape[-1], x.shape[-1]
    _call("csa2_quantize_mxfp8", _p(x), rows, dim, _p(codes), _p(scales), _stream(stream))


def csa2_dequant_mxfp4(codes, scales, out, stream=None):
    rows, dim = out.numel() // out.shape[-1], out.shape[-1]
    _call("csa2_dequant_mxfp4", _p(codes), _p(scales), rows, dim, _p(out), _stream(stream))


def csa2_dequant_mxfp8(codes, scales, out, stream=None):
    rows, dim = out.numel() // out.shape[-1], out.shape[-1]
    _call("csa2_dequant_mxfp8", _p(codes), _p(scales), rows, dim, _p(out), _stream(stream))


def csa2_append_global(cfg, latent, idx_k, block_table, n_blocks, pos0, n_new, kv_cache,
                       idx_cache, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_append_global", C.byref(cfg), _p(latent), _p(idx_k), _p(block_table), maxb,
          int(n_blocks), _p(pos0), batch, int(n_new), _p(kv_cache), _p(idx_cache),
          _stream(stream))


def csa2_append_swa(cfg, rows, pos0, n_new, swa_cache, C_slots, stream=None):
    batch = pos0.shape[0]
    _call("csa2_append_swa", C.byref(cfg), _p(rows), _p(pos0), batch, int(n_new),
          _p(swa_cache), int(C_slots), _stream(stream))


def csa2_blocks_gather(cache, blocks, rows, stream=None):
    """rows[r] = cache[blocks[r]] for the n listed physical blocks (cache [n_blocks, bytes])."""
    n_blocks, block_bytes = cache.shape
    _call("csa2_blocks_gather", _p(cache), int(n_blocks), int(block_bytes), _p(blocks),
          int(blocks.numel()), _p(rows), _stream(stream))


def csa2_blocks_scatter(rows, blocks, cache, stream=None):
    """cache[blocks[r]] = rows[r] for the n listed physical blocks."""
    n_blocks, block_bytes = cache.shape
    _call("csa2_blocks_scatter", _p(rows), _p(blocks), int(blocks.numel()), _p(cache),
          int(n_blocks), int(block_bytes), _stream(stream))


def csa2_index_scores(cfg, q_codes, q_scales, w, idx_cache, n_blocks, block_table, ctx_len,
                      scores, block_scores, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_index_scores", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w), _p(idx_cache),
          int(n_blocks), _p(block_table), maxb, _p(ctx_len), batch, _p(scores),
          _p(block_scores), _stream(stream))


def csa2_index_full_scan(cfg, q_codes, q_scales, w, idx_cache, n_blocks, block_table, ctx_len,
                         ws, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_index_full_scan", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w),
          _p(idx_cache), int(n_blocks), _p(block_table), maxb, _p(ctx_len), batch, _p(ws),
          ws.numel(), _stream(stream))


def csa2_index_full_finish(cfg, q_codes, q_scales, w, idx_cache, n_blocks, block_table,
                           ctx_len, pool_blocks, pool_len, topk, topk_len, ws, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_index_full_finish", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w),
          _p(idx_cache), int(n_blocks), _p(block_table), maxb, _p(ctx_len), batch,
          _p(pool_blocks), _p(pool_len), _p(topk), _p(topk_len), _p(ws), ws.numel(),
          _stream(stream))


def csa2_index_full(cfg, q_codes, q_scales, w, idx_cache, n_blocks, block_table, ctx_len,
                    pool_blocks, pool_len, topk, topk_len, ws, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_index_full", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w), _p(idx_cache),
          int(n_blocks), _p(block_table), maxb, _p(ctx_len), batch, _p(pool_blocks),
          _p(pool_len), _p(topk), _p(topk_len), _p(ws), ws.numel(), _stream(stream))


def csa2_index_full_append(cfg, latent, idx_k, q_codes, q_scales, w, kv_cache, idx_cache,
                           n_blocks, block_table, ctx_len, pool_blocks, pool_len, topk, topk_len,
                           ws, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_index_full_append", C.byref(cfg), _p(latent), _p(idx_k), _p(q_codes),
          _p(q_scales), _p(w), _p(kv_cache), _p(idx_cache), int(n_blocks), _p(block_table), maxb,
          _p(ctx_len), batch, _p(pool_blocks), _p(pool_len), _p(topk), _p(topk_len), _p(ws),
          ws.numel(), _stream(stream))


def csa2_index_reindex(cfg, q_codes, q_scales, w, idx_cache, n_blocks, block_table, ctx_len,
                       pool_blocks, pool_len, topk, topk_len, ws, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_index_reindex", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w), _p(idx_cache),
          int(n_blocks), _p(block_table), maxb, _p(ctx_len), batch, _p(pool_blocks),
          _p(pool_len), _p(topk), _p(topk_len), _p(ws), ws.numel(), _stream(stream))


def csa2_index_prefill(cfg, q_codes, q_scales, w, q_pos0, idx_cache, n_blocks, table_row,
                       pool_blocks, pool_len, topk, topk_len, ws, stream=None):
    n_q = q_codes.shape[0]
    maxb = table_row.numel()
    _call("csa2_index_prefill", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w), int(q_pos0),
          int(n_q), _p(idx_cache), int(n_blocks), _p(table_row), maxb, _p(pool_blocks),
          _p(pool_len), _p(topk), _p(topk_len), _p(ws), ws.numel(), _stream(stream))


def csa2_index_prefill_scan(cfg, q_codes, q_scales, w, q_pos0, idx_cache, n_blocks, table_row,
                            ws, stream=None):
    _call("csa2_index_prefill_scan", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w),
          int(q_pos0), int(q_codes.shape[0]), _p(idx_cache), int(n_blocks), _p(table_row),
          table_row.numel(), _p(ws), ws.numel(), _stream(stream))


def csa2_index_prefill_finish(cfg, q_codes, q_scales, w, q_pos0, idx_cache, n_blocks, table_row,
                              pool_blocks, pool_len, topk, topk_len, ws, stream=None):
    _call("csa2_index_prefill_finish", C.byref(cfg), _p(q_codes), _p(q_scales), _p(w),
          int(q_pos0), int(q_codes.shape[0]), _p(idx_cache), int(n_blocks), _p(table_row),
          table_row.numel(), _p(pool_blocks), _p(pool_len), _p(topk), _p(topk_len), _p(ws),
          ws.numel(), _stream(stream))


def csa2_sparse_attn(cfg, q, kv_cache, n_blocks, block_table, swa_cache, C_slots, ctx_len,
                     topk, topk_len, out, lse, ws, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_sparse_attn", C.byref(cfg), _p(q), _p(kv_cache), int(n_blocks), _p(block_table),
          maxb, _p(swa_cache), int(C_slots), _p(ctx_len), batch, _p(topk), _p(topk_len),
          _p(out), _p(lse), _p(ws), ws.numel(), _stream(stream))


def csa2_sparse_attn_append(cfg, swa_rows, pos, q, kv_cache, n_blocks, block_table, swa_cache,
                            C_slots, ctx_len, topk, topk_len, out, lse, ws, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_sparse_attn_append", C.byref(cfg), _p(swa_rows), _p(pos), _p(q), _p(kv_cache),
          int(n_blocks), _p(block_table), maxb, _p(swa_cache), int(C_slots), _p(ctx_len), batch,
          _p(topk), _p(topk_len), _p(out), _p(lse), _p(ws), ws.numel(), _stream(stream))


def csa2_sparse_attn_prefill(cfg, q, kv_cache, n_blocks, table_row, swa_ring, C_slots, q_pos0,
                             topk, topk_len, out, lse, ws, stream=None):
    n_q = q.shape[0]
    _call("csa2_sparse_attn_prefill", C.byref(cfg), _p(q), _p(kv_cache), int(n_blocks),
          _p(table_row), table_row.numel(), _p(swa_ring), int(C_slots), int(q_pos0), int(n_q),
          _p(topk), _p(topk_len), _p(out), _p(lse), _p(ws), ws.numel(), _stream(stream))


def csa2_sparse_attn_noalloc(cfg, q, kv_cache, n_blocks, block_table, swa_cache, C_slots, ctx_len,
                             topk, topk_len, out, lse, stream=None):
    """csa2_sparse_attn with the library's static per-device scratch instead of a workspace."""
    batch, maxb = block_table.shape
    _call("csa2_sparse_attn_noalloc", C.byref(cfg), _p(q), _p(kv_cache), int(n_blocks),
          _p(block_table), maxb, _p(swa_cache), int(C_slots), _p(ctx_len), batch, _p(topk),
          _p(topk_len), _p(out), _p(lse), _stream(stream))


def csa2_decode_full_layer(cfg, q_idx, w_idx, tok_latent, tok_key, swa_row, q_attn, kv_cache,
                           idx_cache, n_blocks, block_table, swa_cache, C_slots, ctx_len,
                           pool_blocks, pool_len, topk, topk_len, out, lse, ws_index, ws_attn,
                           stream=None):
    batch, maxb = block_table.shape
    _call("csa2_decode_full_layer", C.byref(cfg), _p(q_idx), _p(w_idx), _p(tok_latent),
          _p(tok_key), _p(swa_row), _p(q_attn), _p(kv_cache), _p(idx_cache), int(n_blocks),
          _p(block_table), maxb, _p(swa_cache), int(C_slots), _p(ctx_len), batch,
          _p(pool_blocks), _p(pool_len), _p(topk), _p(topk_len), _p(out), _p(lse), _p(ws_index),
          ws_index.numel(), _p(ws_attn), ws_attn.numel(), _stream(stream))


def csa2_decode_reindex_layer(cfg, q_idx, w_idx, swa_row, q_attn, kv_cache, idx_cache, n_blocks,
                              block_table, swa_cache, C_slots, ctx_len, pool_blocks, pool_len,
                              topk, topk_len, out, lse, ws_index, ws_attn, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_decode_reindex_layer", C.byref(cfg), _p(q_idx), _p(w_idx), _p(swa_row),
          _p(q_attn), _p(kv_cache), _p(idx_cache), int(n_blocks), _p(block_table), maxb,
          _p(swa_cache), int(C_slots), _p(ctx_len), batch, _p(pool_blocks), _p(pool_len),
          _p(topk), _p(topk_len), _p(out), _p(lse), _p(ws_index), ws_index.numel(), _p(ws_attn),
          ws_attn.numel(), _stream(stream))


def csa2_decode_reuse_layer(cfg, swa_row, q_attn, kv_cache, n_blocks, block_table, swa_cache,
                            C_slots, ctx_len, topk, topk_len, out, lse, ws_attn, stream=None):
    batch, maxb = block_table.shape
    _call("csa2_decode_reuse_layer", C.byref(cfg), _p(swa_row), _p(q_attn), _p(kv_cache),
          int(n_blocks), _p(block_table), maxb, _p(swa_cache), int(C_slots), _p(ctx_len), batch,
          _p(topk), _p(topk_len), _p(out), _p(lse), _p(ws_attn), ws_attn.numel(), _stream(stream))
