// csa2_select.h -- the per-sequence selection kernel of the indexer, as other translation
// units launch it (the prefill indexer reuses the Full-mode selection per query).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

// Regions of the two-phase Full selection (decode contexts with more blocks than the pool):
// per sequence b and gather workgroup w (groups [w*1024, (w+1)*1024)), the candidate blocks
// as (order key, block) pairs, the blocks that reach the top-k bound with their 8 position
// scores, and the two counts (-1: more bound-reaching blocks than the region holds).
constexpr int kSel2GroupsPerW = 1024;
constexpr int kSel2MuCap = 256;   // bound-reaching blocks per region
constexpr int kSel2MaxW = 64;     // gather workgroups per sequence (contexts up to 4M)
constexpr int kSel2LdsCap = 8192; // candidates the last workgroup selects from (in LDS)
struct Sel2Ws {
    int32_t nw;        // gather workgroups per sequence (0: the one-workgroup selection)
    uint2 *cand;       // [B][nw][kSel2GroupsPerW * 8]
    float *mu_sc;      // [B][nw][kSel2MuCap][8]
    int32_t *mu_blk;   // [B][nw][kSel2MuCap]
    int32_t *cnt;      // [B][nw][2]
    int32_t *arrive;   // [B] arrivals: zeroed by the scan, reset by the last workgroup
};

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
    Sel2Ws sel2;  // two-phase Full selection (sel2.nw > 0)
    // Prefill in two passes (csa2_index_prefill with more than 16 queries): flags of the
    // blocks whose position scores the top-k reads, word w (blocks 32w .. 32w + 31) of chunk
    // c (256 blocks) of query b at pf_need[(c*8 + w)*B + b]; those blocks of each query,
    // ascending, at pf_list[b*K_blk];
    // per query (lower bound key of its k-th best score, upper bound key, count) in pf_meta.
    uint32_t *pf_need;
    int32_t *pf_list;
    uint4 *pf_meta;
};

// Gather workgroups per sequence of the two-phase Full selection for a table of width maxb
// (0 when the one-workgroup selection serves: every sequence fits the pool, K_blk < k, or the
// context is beyond kSel2MaxW workgroups).
int sel2_workgroups(const csa2_config *cfg, int32_t maxb);

// Enqueues the selection: one workgroup per sequence b < a.B.  Full: pool from the block
// and group maxima, then top-k from the position scores.  Reindex: top-k from the rescored
// pool.  Returns a csa2 status.
int launch_select(const SelectArgs &a, bool reindex, hipStream_t stream);

// The two-phase Full selection (sel2.nw + 1 workgroups per sequence; with several sequences
// and sel2.nw a multiple of 8, laid out by XCD); a.sel2 filled.
int launch_select_full2(const SelectArgs &a, hipStream_t stream);

// Prefill selection in two phases around the rescoring pass.  Phase 0: the pool of every
// query (written out) and its flagged blocks (pf_need, pf_list, pf_meta; pf_need zeroed
// beforehand).  Phase 1: the top-k of every query from the position scores of its flagged
// blocks.
int launch_select_prefill(const SelectArgs &a, int phase, hipStream_t stream);

// Row stride of the group maxima of a table of width maxb (multiple of 4 floats).
int ngmax_of(int maxb);

// Validates the index-call shape of cfg (dims, pool and top-k limits, compiled kernels).
int check_index_cfg(const csa2_config *cfg);

// Workspace bytes of csa2_index_prefill for n_q queries and table width maxb.
size_t prefill_ws_bytes(const csa2_config *cfg, int32_t n_q, int32_t maxb);

}  // namespace csa2
