// csa2_layer.h -- the steps of one decode layer as the fused layer calls launch them.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

// csa2_index_full_append, with the indexer query given either as MXFP4 codes and scales or
// unquantised (q_f32 non-null: quantised inside the scan).  Returns a csa2 status.
int index_full_append(const csa2_config *c, const float *latent, const float *idx_k,
                      const uint8_t *q_codes, const uint8_t *q_scales, const float *q_f32,
                      const float *w, uint8_t *kv_cache, uint8_t *idx_cache, int64_t n_blocks,
                      const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                      int32_t batch, int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                      int32_t *topk_len, void *ws, size_t ws_bytes, hipStream_t stream);

// csa2_index_reindex, with the query as above.
int index_reindex(const csa2_config *c, const uint8_t *q_codes, const uint8_t *q_scales,
                  const float *q_f32, const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                  const int32_t *block_table, int32_t maxb, const int32_t *ctx_len, int32_t batch,
                  const int32_t *pool_blocks, const int32_t *pool_len, int32_t *topk,
                  int32_t *topk_len, void *ws, size_t ws_bytes, hipStream_t stream);

// csa2_sparse_attn_append with pos = ctx_len - 1.  dry: only the host-side checks (topk,
// topk_len may then be null), nothing is launched.
int sparse_attn_layer(const csa2_config *c, const float *swa_rows, const uint16_t *q,
                      const uint8_t *kv_cache, int64_t n_blocks, const int32_t *block_table,
                      int32_t maxb, uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                      int32_t batch, const int32_t *topk, const int32_t *topk_len, float *out,
                      float *lse, void *ws, size_t ws_bytes, hipStream_t stream, bool dry);

}  // namespace csa2
