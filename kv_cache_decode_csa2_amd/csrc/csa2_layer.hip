// csa2_layer.hip -- one decode layer per call, in each of the three modes of CSA2
// (dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心": a Full layer scans the whole
// visible context into a pool and a top-k, a Reindex layer rescores only the pool, a Reuse
// layer keeps the previous top-k; every layer attends its top-k rows plus its own sliding
// window, 10100.com/article/150771503, "三招压缩，各有分工").
//
// Each call runs the layer's steps in as few launches as the steps' data dependences allow,
// and equals the sequence of the separate calls bit for bit:
//   Full     scan (indexer-query quantise + the token's global append + scores, block and
//            group maxima) -> selection (pool, top-k) -> attention (+ the token's window row)
//   Reindex  rescoring scan (query quantise + pool scores) -> selection -> attention
//   Reuse    attention (+ window row)
// Host-side argument errors of any step are found before anything is launched.
#include "csa2_layer.h"

using namespace csa2;

extern "C" int csa2_decode_full_layer(const csa2_config *c, const float *q_idx, const float *w_idx,
                                      const float *tok_latent, const float *tok_key,
                                      const float *swa_row, const uint16_t *q_attn,
                                      uint8_t *kv_cache, uint8_t *idx_cache, int64_t n_blocks,
                                      const int32_t *block_table, int32_t maxb, uint8_t *swa_cache,
                                      int32_t C, const int32_t *ctx_len, int32_t batch,
                                      int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                                      int32_t *topk_len, float *out, float *lse, void *ws_index,
                                      size_t ws_index_bytes, void *ws_attn, size_t ws_attn_bytes,
                                      hipStream_t stream) {
    if (!q_idx || !kv_cache) return CSA2_ERR_INVALID;
    int st = sparse_attn_layer(c, swa_row, q_attn, kv_cache, n_blocks, block_table, maxb,
                               swa_cache, C, ctx_len, batch, topk, topk_len, out, lse, ws_attn,
                               ws_attn_bytes, stream, true);
    if (st) return st;
    st = index_full_append(c, tok_latent, tok_key, nullptr, nullptr, q_idx, w_idx, kv_cache,
                           idx_cache, n_blocks, block_table, maxb, ctx_len, batch, pool_blocks,
                           pool_len, topk, topk_len, ws_index, ws_index_bytes, stream);
    if (st) return st;
    return sparse_attn_layer(c, swa_row, q_attn, kv_cache, n_blocks, block_table, maxb, swa_cache,
                             C, ctx_len, batch, topk, topk_len, out, lse, ws_attn, ws_attn_bytes,
                             stream, false);
}

extern "C" int csa2_decode_reindex_layer(const csa2_config *c, const float *q_idx,
                                         const float *w_idx, const float *swa_row,
                                         const uint16_t *q_attn, const uint8_t *kv_cache,
                                         const uint8_t *idx_cache, int64_t n_blocks,
                                         const int32_t *block_table, int32_t maxb,
                                         uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                                         int32_t batch, const int32_t *pool_blocks,
                                         const int32_t *pool_len, int32_t *topk, int32_t *topk_len,
                                         float *out, float *lse, void *ws_index,
                                         size_t ws_index_bytes, void *ws_attn, size_t ws_attn_bytes,
                                         hipStream_t stream) {
    if (!q_idx) return CSA2_ERR_INVALID;
    int st = sparse_attn_layer(c, swa_row, q_attn, kv_cache, n_blocks, block_table, maxb,
                               swa_cache, C, ctx_len, batch, topk, topk_len, out, lse, ws_attn,
                               ws_attn_bytes, stream, true);
    if (st) return st;
    st = index_reindex(c, nullptr, nullptr, q_idx, w_idx, idx_cache, n_blocks, block_table, maxb,
                       ctx_len, batch, pool_blocks, pool_len, topk, topk_len, ws_index,
                       ws_index_bytes, stream);
    if (st) return st;
    return sparse_attn_layer(c, swa_row, q_attn, kv_cache, n_blocks, block_table, maxb, swa_cache,
                             C, ctx_len, batch, topk, topk_len, out, lse, ws_attn, ws_attn_bytes,
                             stream, false);
}

extern "C" int csa2_decode_reuse_layer(const csa2_config *c, const float *swa_row,
                                       const uint16_t *q_attn, const uint8_t *kv_cache,
                                       int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                                       uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                                       int32_t batch, const int32_t *topk, const int32_t *topk_len,
                                       float *out, float *lse, void *ws_attn, size_t ws_attn_bytes,
                                       hipStream_t stream) {
    return sparse_attn_layer(c, swa_row, q_attn, kv_cache, n_blocks, block_table, maxb, swa_cache,
                             C, ctx_len, batch, topk, topk_len, out, lse, ws_attn, ws_attn_bytes,
                             stream, false);
}
