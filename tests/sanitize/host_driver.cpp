// Exercises the host side of libcsa2 (argument checks, layouts, workspace and split sizes)
// without a GPU: every call below is rejected, or sized, before any kernel is launched.
// Built host-only with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitize.py (hipcc --cuda-host-only, each -fsanitize= after -Xarch_host).
// Device pointers are small host arrays that the library must never dereference; a read
// of one would show up as an overflow.  Exit status 0 when every status is as expected.
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "csa2.h"

static int failures = 0;
static void expect(int got, std::initializer_list<int> ok, const char *what) {
    for (int v : ok)
        if (got == v) return;
    std::fprintf(stderr, "FAIL %s: status %d\n", what, got);
    failures++;
}

static csa2_config cfg(int H, int d, int Hq, int W, int Kb, int k, int shared = 0) {
    csa2_config c;
    std::memset(&c, 0, sizeof c);
    c.n_idx_heads = H; c.idx_dim = d; c.kv_dim = 512; c.n_q_heads = Hq; c.swa_window = W;
    c.pool_blocks = Kb; c.topk = k; c.sm_scale = 0.0441941738f; c.shared_key = shared;
    return c;
}

int main() {
    static unsigned char buf[64];
    void *p = buf;
    auto u8 = (uint8_t *)p;
    auto i32 = (int32_t *)p;
    auto f32 = (float *)p;
    auto u16 = (uint16_t *)p;
    const hipStream_t s = nullptr;
    const int INV = CSA2_ERR_INVALID, UNS = CSA2_ERR_UNSUPPORTED, WSE = CSA2_ERR_WORKSPACE;

    const csa2_config good[] = {cfg(4, 64, 16, 128, 2048, 512), cfg(8, 128, 64, 128, 2048, 512),
                                cfg(8, 128, 16, 128, 2048, 512, 1), cfg(1, 32, 16, 0, 1, 8),
                                cfg(2, 64, 128, 32, 64, 64)};
    // configs each kind of call must reject: bad dims (every call), a bad index shape
    // (index calls), a bad attention shape (attention calls)
    csa2_config bad_dims[] = {cfg(4, 48, 16, 128, 2048, 512), cfg(0, 64, 16, 128, 2048, 512),
                              cfg(4, 64, 16, 128, 2048, 512), cfg(4, 64, 16, 128, 2048, 512, 2)};
    bad_dims[2].kv_dim = 500;
    const csa2_config bad_index[] = {cfg(4, 64, 16, 128, 0, 512), cfg(4, 64, 16, 128, 64, 513),
                                     cfg(4, 64, 16, 128, 4096, 512)};
    csa2_config bad_attn[] = {cfg(4, 64, 24, 128, 64, 64), cfg(4, 64, 16, -1, 64, 64),
                              cfg(4, 64, 16, 128, 64, 0), cfg(4, 64, 16, 128, 64, 64)};
    bad_attn[3].kv_dim = 500;
    for (const auto &c : good) {
        csa2_layout_info li;
        expect(csa2_layout(&c, &li), {CSA2_OK}, "layout");
        const size_t kh = c.shared_key ? 1 : c.n_idx_heads;
        if (li.kv_row_bytes != 272 || li.kv_block_bytes != 2176 || li.swa_row_bytes != 528 ||
            li.idx_block_bytes != 8 * kh * (c.idx_dim / 2 + c.idx_dim / 32) || li.idx_block_bytes % 8) {
            std::fprintf(stderr, "FAIL layout sizes\n");
            failures++;
        }
        const int32_t batches[] = {0, 1, 3, 64, 1000, 4096};
        const int32_t widths[] = {0, 1, 17, 1024, 131072, 524288};
        for (int op = 1; op <= 4; op++)
            for (int32_t b : batches)
                for (int32_t m : widths) {
                    size_t bytes = 0;
                    const int st = csa2_workspace_bytes(&c, op, b, m, &bytes);
                    expect(st, {CSA2_OK, INV, UNS}, "workspace_bytes");
                    if (st == CSA2_OK && bytes % 256) {
                        std::fprintf(stderr, "FAIL workspace alignment op %d\n", op);
                        failures++;
                    }
                }
        size_t bytes;
        expect(csa2_workspace_bytes(&c, 9, 1, 1, &bytes), {INV}, "workspace op");
        expect(csa2_workspace_bytes(&c, 1, -1, 1, &bytes), {INV}, "workspace batch");
        expect(csa2_workspace_bytes(&c, 1, 1, 1, nullptr), {INV}, "workspace out");
    }
    for (const auto &c : bad_dims) {
        csa2_layout_info li;
        expect(csa2_layout(&c, &li), {INV}, "bad dims layout");
        size_t bytes;
        expect(csa2_workspace_bytes(&c, CSA2_OP_INDEX_FULL, 1, 1, &bytes), {INV, UNS}, "bad dims workspace");
        expect(csa2_index_full(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, i32, i32, i32, i32, p, 1 << 20, s),
               {INV, UNS}, "bad dims index_full");
        expect(csa2_append_swa(&c, f32, i32, 1, 1, u8, 256, s), {INV}, "bad dims append_swa");
    }
    for (const auto &c : bad_index) {
        size_t bytes;
        expect(csa2_workspace_bytes(&c, CSA2_OP_INDEX_FULL, 1, 1, &bytes), {INV, UNS}, "bad index workspace");
        expect(csa2_index_full(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, i32, i32, i32, i32, p, 1 << 20, s),
               {INV, UNS}, "bad index_full");
        expect(csa2_index_reindex(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, i32, i32, i32, i32, p, 1 << 20, s),
               {INV, UNS}, "bad index reindex");
    }
    for (const auto &c : bad_attn) {
        size_t bytes;
        expect(csa2_workspace_bytes(&c, CSA2_OP_SPARSE_ATTN, 1, 1, &bytes), {INV, UNS}, "bad attn workspace");
        expect(csa2_sparse_attn(&c, u16, u8, 8, i32, 1, u8, 256, i32, 1, i32, i32, f32, f32, p, 1 << 20, s),
               {INV, UNS}, "bad sparse_attn");
        expect(csa2_decode_reuse_layer(&c, f32, u16, u8, 8, i32, 1, u8, 256, i32, 1, i32, i32, f32, f32,
                                       p, 1 << 20, s), {INV, UNS}, "bad reuse_layer");
    }
    expect(csa2_layout(nullptr, nullptr), {INV}, "null layout");

    const csa2_config c = good[0];
    // codecs and transfers
    expect(csa2_quantize_mxfp4(nullptr, 1, 64, u8, u8, s), {INV}, "quant4 null");
    expect(csa2_quantize_mxfp4(f32, 1, 48, u8, u8, s), {INV}, "quant4 dim");
    expect(csa2_quantize_mxfp8(f32, -1, 64, u8, u8, s), {INV}, "quant8 rows");
    expect(csa2_dequant_mxfp4(u8, nullptr, 1, 64, f32, s), {INV}, "deq4 null");
    expect(csa2_dequant_mxfp8(u8, u8, 1, 40, f32, s), {INV}, "deq8 dim");
    expect(csa2_blocks_gather(nullptr, 8, 1088, i32, 1, u8, s), {INV}, "gather null");
    expect(csa2_blocks_gather(u8, 8, 1000, i32, 1, u8, s), {INV}, "gather block bytes");
    expect(csa2_blocks_scatter(u8, i32, -1, u8, 8, 1088, s), {INV}, "scatter n");
    // appends
    expect(csa2_append_global(&c, nullptr, nullptr, i32, 1, 8, i32, 1, 1, u8, u8, s), {INV}, "append_global null");
    expect(csa2_append_global(&c, f32, f32, i32, 1, 8, i32, 1, 1, u8, nullptr, s), {INV}, "append_global no cache");
    expect(csa2_append_global(&c, f32, f32, i32, 1, 8, i32, -1, 1, u8, u8, s), {INV}, "append_global batch");
    expect(csa2_append_swa(&c, f32, i32, 1, 1, u8, 0, s), {INV}, "append_swa no ring");
    expect(csa2_append_swa(&c, nullptr, i32, 1, 1, u8, 256, s), {INV}, "append_swa null");
    // index calls
    expect(csa2_index_scores(&c, nullptr, u8, f32, u8, 8, i32, 1, i32, 1, f32, f32, s), {INV}, "scores null");
    expect(csa2_index_full(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, i32, i32, i32, i32, p, 0, s), {WSE, INV}, "full ws");
    expect(csa2_index_full(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, nullptr, i32, i32, i32, p, 1 << 20, s), {INV}, "full null");
    expect(csa2_index_full_scan(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, p, 16, s), {WSE, INV}, "full_scan ws");
    expect(csa2_index_full_finish(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, i32, i32, nullptr, i32, p, 1 << 20, s), {INV}, "finish null");
    expect(csa2_index_full_append(&c, f32, f32, u8, u8, f32, u8, nullptr, 8, i32, 1, i32, 1, i32, i32, i32, i32, p, 1 << 20, s), {INV}, "full_append null");
    expect(csa2_index_reindex(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, nullptr, i32, i32, i32, p, 1 << 20, s), {INV}, "reindex null");
    expect(csa2_index_reindex(&c, u8, u8, f32, u8, 8, i32, 1, i32, 1, i32, i32, i32, i32, p, 0, s), {WSE, INV}, "reindex ws");
    expect(csa2_index_prefill(&c, u8, u8, f32, 0, 4, u8, 8, i32, 1, i32, i32, i32, i32, p, 0, s), {WSE, INV}, "prefill ws");
    expect(csa2_index_prefill(&c, u8, u8, f32, 6, 4, u8, 8, i32, 1, i32, i32, i32, i32, p, 1 << 20, s), {INV}, "prefill past table");
    expect(csa2_index_prefill_scan(&c, u8, u8, f32, -1, 4, u8, 8, i32, 4, p, 1 << 20, s), {INV}, "prefill_scan pos");
    expect(csa2_index_prefill_finish(&c, u8, u8, f32, 0, 4, u8, 8, i32, 4, nullptr, i32, i32, i32, p, 1 << 20, s), {INV}, "prefill_finish null");
    const csa2_config sk = good[2];
    expect(csa2_index_prefill(&sk, u8, u8, f32, 0, 4, u8, 8, i32, 4, i32, i32, i32, i32, p, 1 << 20, s), {UNS, INV}, "prefill shared key");
    // attention
    expect(csa2_sparse_attn(&c, nullptr, u8, 8, i32, 1, u8, 256, i32, 1, i32, i32, f32, f32, p, 1 << 20, s), {INV}, "attn null");
    expect(csa2_sparse_attn(&c, u16, u8, 8, i32, 1, u8, 64, i32, 1, i32, i32, f32, f32, p, 1 << 20, s), {INV}, "attn ring < W");
    expect(csa2_sparse_attn(&c, u16, u8, 8, i32, 1, u8, 256, i32, 8, i32, i32, f32, f32, p, 64, s), {WSE, INV}, "attn ws");
    expect(csa2_sparse_attn_append(&c, f32, nullptr, u16, u8, 8, i32, 1, u8, 256, i32, 1, i32, i32, f32, f32, p, 1 << 20, s), {INV}, "attn_append null");
    expect(csa2_sparse_attn_prefill(&c, u16, u8, 8, i32, 16, u8, 128, 0, 8, i32, i32, f32, f32, p, 1 << 20, s), {INV}, "attn_prefill ring");
    expect(csa2_sparse_attn_noalloc(&c, u16, u8, 8, i32, 1, u8, 256, i32, 600, i32, i32, f32, f32, s), {CSA2_ERR_SCRATCH}, "noalloc scratch");
    // fused layer calls
    expect(csa2_decode_full_layer(&c, f32, f32, f32, f32, f32, u16, u8, u8, 8, i32, 1, u8, 256, i32, 1,
                                  i32, i32, i32, i32, f32, f32, p, 0, p, 1 << 20, s), {WSE, INV}, "full_layer ws");
    expect(csa2_decode_reindex_layer(&c, f32, f32, f32, u16, u8, u8, 8, i32, 1, u8, 256, i32, 1,
                                     nullptr, i32, i32, i32, f32, f32, p, 1 << 20, p, 1 << 20, s), {INV}, "reindex_layer null");
    expect(csa2_decode_reuse_layer(&c, f32, u16, u8, 8, i32, 1, u8, 256, i32, 1, i32, i32, f32, f32,
                                   p, 0, s), {WSE, INV}, "reuse_layer ws");
    for (int st = -6; st <= 1; st++)
        if (!csa2_status_str(st)) {
            std::fprintf(stderr, "FAIL status_str %d\n", st);
            failures++;
        }
    if (failures) {
        std::fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    std::puts("host driver: ok");
    return 0;
}
