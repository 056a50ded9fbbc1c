// csa2_select.h -- the per-sequence selection kernel of the indexer, as other translation
// units launch it (the prefill indexer reuses the Full-mode selection per query).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

struct SelectArgs {
    const int32_t *ctx_len;  // [B] device lengths; NULL: L_b = q_pos0 + b + 1 (prefill)
    int32_t q_pos0;
    int32_t maxb;
    int32_t B;
    int32_t K_blk;
    int32_t k;
    // Full: position score of (b, p) at pscore[b*ps_b + (p/8)*ps_j + p%8] and block maximum
    // of (b, j) at bscore[b*bs_b + (j/8)*bs_g + j%8]: row-major per sequence for decode,
    // block-major for the prefill queries
    const float *pscore;
    int64_t ps_b, ps_j;
    const float *bscore;
    int64_t bs_b, bs_g;
    const float *gmax;    // Full: group maxima (8 blocks) [B][ngmax]
    int32_t ngmax;
    const float *poolsc;    // Reindex: pool scores [B][K_blk*8]
    const float *poolbmax;  // Reindex: pool block maxima [B][K_blk]
    int32_t *pool_blocks;  // Full: out; Reindex: in
    int32_t *pool_len;     // Full: out; Reindex: in
    int32_t *topk;
    int32_t *topk_len;
};

// Enqueues the selection: one workgroup per sequence b < a.B.  Full: pool from the block
// and group maxima, then top-k from the position scores.  Reindex: top-k from the rescored
// pool.  Returns a csa2 status.
int launch_select(const SelectArgs &a, bool reindex, hipStream_t stream);

// Row stride of the group maxima of a table of width maxb (multiple of 4 floats).
int ngmax_of(int maxb);

// Validates the index-call shape of cfg (dims, pool and top-k limits, compiled kernels).
int check_index_cfg(const csa2_config *cfg);

// Workspace bytes of csa2_index_prefill for n_q queries and table width maxb.
size_t prefill_ws_bytes(const csa2_config *cfg, int32_t n_q, int32_t maxb);

}  // namespace csa2
