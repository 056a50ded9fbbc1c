"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/csa2.h declares, and rejects bad arguments on the host (no kernel is launched)."""
import ctypes as C
import os
import re

import pytest

import kv_cache_decode_csa2_amd as k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(k.LIB_PATH),
                                reason="libcsa2.so not built (run __graft_entry__.build())")


def _declared():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_entry_point_is_exported():
    names = _declared()
    assert len(names) >= 14
    lib = k.load()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing
    assert sorted(k.EXPORTS) == names


def test_layout_sizes():
    c = k.config(4, 64, 512, 16, 128, 2048, 512, 0.044)
    lay = k.csa2_layout(c)
    assert (lay.idx_block_bytes, lay.kv_row_bytes, lay.kv_block_bytes, lay.swa_row_bytes) == \
        (1088, 272, 2176, 528)
    c2 = k.config(8, 128, 512, 64, 128, 2048, 512, 0.044)
    assert k.csa2_layout(c2).idx_block_bytes == 4352


def test_workspace_sizes_grow_with_batch_and_context():
    c = k.config(4, 64, 512, 16, 128, 2048, 512, 0.044)
    a = k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 1, 1024)
    b = k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 1, 131072)
    d = k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 8, 131072)
    assert 0 < a < b < d and all(x % 256 == 0 for x in (a, b, d))
    # 640 rows = 10 chunks of 64 in 5 pairs: at 8 sequences every pair is a split, whose
    # partial numerators (16 heads x 512 fp32) sit in the workspace
    assert k.csa2_workspace_bytes(c, k.CSA2_OP_SPARSE_ATTN, 8, 1) >= 8 * 5 * 16 * 512 * 4
    # a batch that fills the chip alone takes one split: no partials, only the fixed
    # 1024-counter region every attention workspace starts with
    assert k.csa2_workspace_bytes(c, k.CSA2_OP_SPARSE_ATTN, 4096, 1) == 4096


@pytest.mark.parametrize("bad", [
    dict(idx_dim=48), dict(kv_dim=500), dict(pool_blocks=0), dict(topk=0),
    dict(topk=8 * 64 + 1), dict(n_idx_heads=0), dict(swa_window=-1),
])
def test_invalid_configs_rejected(bad):
    args = dict(n_idx_heads=4, idx_dim=64, kv_dim=512, n_q_heads=16, swa_window=128,
                pool_blocks=64, topk=128, sm_scale=0.044)
    args.update(bad)
    c = k.csa2_config(**args)
    with pytest.raises(k.Csa2Error) as e:
        k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 1, 512)
    assert e.value.status == k.CSA2_ERR_INVALID


def test_unsupported_shapes_reported():
    c = k.config(16, 64, 512, 16, 128, 64, 128, 0.044)   # 16 indexer heads: no kernel
    with pytest.raises(k.Csa2Error) as e:
        k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 1, 512)
    assert e.value.status == k.CSA2_ERR_UNSUPPORTED
    c = k.config(4, 64, 512, 16, 128, 4096, 128, 0.044)  # pool beyond 2048 blocks
    with pytest.raises(k.Csa2Error) as e:
        k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 1, 512)
    assert e.value.status == k.CSA2_ERR_UNSUPPORTED


def test_host_side_argument_errors_launch_nothing():
    lib = k.load()
    c = k.config(4, 64, 512, 16, 128, 64, 128, 0.044)
    nul = None
    # null pointers -> INVALID before any HIP call
    st = lib.csa2_index_full(C.byref(c), nul, nul, nul, nul, 1, nul, 8, nul, 1, nul, nul, nul,
                             nul, nul, 0, nul)
    assert st == k.CSA2_ERR_INVALID
    st = lib.csa2_sparse_attn(C.byref(c), nul, nul, 1, nul, 8, nul, 128, nul, 1, nul, nul, nul,
                              nul, nul, 0, nul)
    assert st == k.CSA2_ERR_INVALID
    st = lib.csa2_quantize_mxfp4(C.c_void_p(16), 4, 48, C.c_void_p(16), C.c_void_p(16), nul)
    assert st == k.CSA2_ERR_INVALID
    # a workspace that is too small is reported, not used
    fake = C.c_void_p(256)
    st = lib.csa2_index_full(C.byref(c), fake, fake, fake, fake, 1, fake, 8, fake, 1, fake, fake,
                             fake, fake, fake, 16, nul)
    assert st == k.CSA2_ERR_WORKSPACE
    # batch 0 is a no-op
    ws = k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 0, 8)
    st = lib.csa2_index_full(C.byref(c), fake, fake, fake, fake, 1, fake, 8, fake, 0, fake, fake,
                             fake, fake, fake, ws, nul)
    assert st == k.CSA2_OK
    assert k.status_str(k.CSA2_ERR_WORKSPACE) == "workspace too small"


def test_attention_shape_limits():
    lib = k.load()
    fake = C.c_void_p(256)
    c = k.config(4, 64, 256, 16, 128, 64, 128, 0.044)   # latent 256: no kernel
    st = lib.csa2_sparse_attn(C.byref(c), fake, fake, 1, fake, 8, fake, 128, fake, 1, fake, fake,
                              fake, fake, fake, 1 << 30, None)
    assert st == k.CSA2_ERR_UNSUPPORTED
    c = k.config(4, 64, 512, 16, 128, 64, 128, 0.044)
    st = lib.csa2_sparse_attn(C.byref(c), fake, fake, 1, fake, 8, fake, 64, fake, 1, fake, fake,
                              fake, fake, fake, 1 << 30, None)   # ring smaller than window
    assert st == k.CSA2_ERR_INVALID

    def prefill(C_slots, n_q):
        return lib.csa2_sparse_attn_prefill(C.byref(c), fake, fake, 1, fake, 64, fake, C_slots,
                                            100, n_q, fake, fake, fake, fake, fake, 1 << 30, None)
    # a prefill chunk of 10 queries with a 128-row window needs a ring of 10 + 127 slots
    assert prefill(136, 10) == k.CSA2_ERR_INVALID
    assert prefill(128, 2) == k.CSA2_ERR_INVALID
    assert prefill(137, 0) == k.CSA2_OK                                   # no query: no-op


def test_block_transfer_and_fused_append_host_errors():
    """Argument errors of the block-transfer calls and of the fused Full-layer append are
    found on the host (nothing is launched); empty calls are no-ops."""
    lib = k.load()
    nul, f = None, C.c_void_p(256)
    INV = k.CSA2_ERR_INVALID
    assert lib.csa2_blocks_gather(f, 10, 24, f, 3, f, nul) == INV       # not a multiple of 16
    assert lib.csa2_blocks_gather(f, 10, 32, f, -1, f, nul) == INV      # n < 0
    assert lib.csa2_blocks_gather(nul, 10, 32, f, 3, f, nul) == INV     # NULL cache
    assert lib.csa2_blocks_scatter(f, f, 3, f, 0, 32, nul) == INV       # no blocks
    assert lib.csa2_blocks_gather(nul, 10, 32, nul, 0, nul, nul) == k.CSA2_OK
    assert lib.csa2_blocks_scatter(nul, nul, 0, nul, 10, 32, nul) == k.CSA2_OK
    c = k.config(4, 64, 512, 16, 128, 64, 128, 0.044)
    ws = k.csa2_workspace_bytes(c, k.CSA2_OP_INDEX_FULL, 1, 8)

    def fused(cfg, idx_k, batch, ws_bytes):
        return lib.csa2_index_full_append(C.byref(cfg), f, idx_k, f, f, f, f, f, 1, f, 8, f,
                                          batch, f, f, f, f, f, ws_bytes, nul)
    assert fused(c, nul, 1, ws) == INV                                   # no indexer key
    assert fused(c, f, 1, 16) == k.CSA2_ERR_WORKSPACE
    assert fused(c, f, 0, ws) == k.CSA2_OK                               # empty batch
    c256 = k.config(4, 64, 256, 16, 128, 64, 128, 0.044)
    assert fused(c256, f, 1, ws) == k.CSA2_ERR_UNSUPPORTED               # latent of 256


def test_noalloc_attention_rejects_shapes_beyond_its_scratch():
    """csa2_sparse_attn_noalloc checks the shape against its 16 MiB static scratch on the host
    before any HIP call: 16 heads at batch 600 (two splits of 16 x 512 fp32 partials per
    sequence, about 39 MB) is refused; argument errors come first."""
    lib = k.load()
    f = C.c_void_p(256)
    c = k.config(4, 64, 512, 16, 128, 2048, 512, 0.044)
    st = lib.csa2_sparse_attn_noalloc(C.byref(c), f, f, 1, f, 8, f, 128, f, 600, f, f, f, f, None)
    assert st == k.CSA2_ERR_SCRATCH
    assert "static scratch" in k.status_str(st)
    st = lib.csa2_sparse_attn_noalloc(C.byref(c), f, f, 1, f, 8, f, 64, f, 200, f, f, f, f, None)
    assert st == k.CSA2_ERR_INVALID  # ring smaller than the window
    st = lib.csa2_sparse_attn_noalloc(C.byref(c), f, f, 1, f, 8, f, 128, None, 1, f, f, f, f, None)
    assert st == k.CSA2_ERR_INVALID  # no lengths
