/*
 * csa2.h -- C ABI of the CSA2 decode hot path on MI355X (gfx950).
 *
 * The operations follow the description of DeepSeek-V4.1-Flash's CSA2 attention on these
 * web pages (cited by address and section heading):
 *   [KV]  dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心": layers run in Full,
 *         Reindex or Reuse mode; the first Full layer scans the whole visible context and
 *         keeps a candidate pool of at most 2048 blocks of 8 positions; later layers pick
 *         the final top-512 inside the pool; indexer Q/K and main KV are FP4, the
 *         sliding-window KV is FP8; the global KV is kept in a persistent cache (host
 *         memory or SSD) for later prefix hits, the window KV only briefly.
 *   [3]   10100.com/article/150771503, "三招压缩，各有分工": the decoder keeps layer-local
 *         sliding-window attention; later indexers search only the pool.
 *   [HSI] prism.simon-ai.net/article/7901, "层级稀疏索引器：精准筛选关键信息".
 *   [W]   prism.simon-ai.net/article/7901, "短期记忆的去留：从SSD存储到GPU重算": the local
 *         window is the last 128 tokens.
 * The pages fix no formula, layout or rounding; where a call below states one, it is this
 * library's definition (formats: OCP MX E2M1 / E4M3FN with per-32 E8M0 scales).
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers unless stated otherwise, owned by the caller,
 *     16-byte aligned.  The library allocates nothing and keeps no state between calls.
 *   - Calls enqueue work on `stream` and return without synchronising.  A non-zero status
 *     means nothing was enqueued (argument errors are found on the host), except
 *     CSA2_ERR_HIP, which reports a failed launch.
 *   - Values that live in device memory (context lengths, positions, block-table entries,
 *     index lists) cannot be checked on the host.  Kernels bounds-check them and skip
 *     entries that are out of range, so a bad value never reads or writes outside the
 *     buffers described here; the results for such entries are unspecified.
 *   - A workspace `ws` of at least csa2_workspace_bytes() bytes is needed by the index
 *     and attention calls (one per kind of call).  An index workspace needs no
 *     initialisation.  An attention workspace starts with a fixed region of 1024 arrival
 *     counters (4 KB, the same bytes for every shape): zero it once after allocating it
 *     (hipMemset); every attention call leaves the counters at zero again, so one
 *     attention workspace of the largest size needed serves decode, append and prefill
 *     attention calls of any batch or query count.  It must not be shared with index
 *     calls.  Calls that share a workspace must not run concurrently.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_BLOCK 8                /* positions per cache block [KV] */
#define CSA2_MAX_POOL_BLOCKS 2048   /* pool capacity named in [KV] */

enum {
    CSA2_OK = 0,
    CSA2_ERR_INVALID = -1,     /* null pointer, bad size, dims % 32 != 0, k > 8*K_blk, ... */
    CSA2_ERR_UNSUPPORTED = -2, /* a shape this build has no kernel for */
    CSA2_ERR_WORKSPACE = -3,   /* ws_bytes < csa2_workspace_bytes() */
    CSA2_ERR_HIP = -4,         /* a kernel launch failed */
    CSA2_ERR_SCRATCH = -5      /* csa2_sparse_attn_noalloc: the shape needs more than its
                                  static scratch (16 MiB) */
};

enum {
    CSA2_OP_INDEX_FULL = 1,
    CSA2_OP_INDEX_REINDEX = 2,
    CSA2_OP_SPARSE_ATTN = 3,
    CSA2_OP_INDEX_PREFILL = 4 /* batch = number of prefill queries */
};

/* Shapes of one CSA2 layer. */
typedef struct csa2_config {
    int32_t n_idx_heads; /* H_I: indexer heads (1, 2, 4 or 8)                      */
    int32_t idx_dim;     /* d_I: indexer head dim (32, 64 or 128)                    */
    int32_t kv_dim;      /* D: main latent dim (512)                                 */
    int32_t n_q_heads;   /* H_q: attention query heads (multiple of 16, <= 128)      */
    int32_t swa_window;  /* W: sliding window (>= 0) [W]                             */
    int32_t pool_blocks; /* K_blk: pool capacity in blocks (1 .. 2048) [KV]          */
    int32_t topk;        /* k: final selection (1 .. 8*K_blk) [KV]                   */
    float sm_scale;      /* softmax scale applied to q.k                             */
    int32_t shared_key;  /* 0: one indexer key per head per position (H_I keys);
                            1: one d_I key per position, scored by all H_I query heads
                            (the shared-key indexer variant; the index calls take the
                            same query, the caches hold KH = 1 key per position)     */
} csa2_config;

/* Byte sizes of the cache layouts (multiples of 16, except idx_block_bytes = 136 KH with
 * d_I = 32: a multiple of 8 when KH is odd).
 *
 * Global caches are paged: physical block `phys` of 8 positions holds
 *   idx_cache + phys*idx_block_bytes : indexer keys of the 8 positions.  With H the key heads
 *       (H_I, or 1 with shared_key) and G = d_I/32, the 16 bytes of FP4 codes of group g of
 *       head h of the position in slot s sit at 16*((g*8 + s)*H + h); the E8M0 scale of that
 *       group sits at 8*H*d_I/2 + (s*H + h)*G + g.
 *   kv_cache + phys*kv_block_bytes : main latent rows, slot s at s*kv_row_bytes:
 *       D/2 bytes of FP4 codes (element 2i in the low nibble) then D/32 E8M0 scales.
 * block_table[b*maxb + j] is the physical block of positions 8j..8j+7 of sequence b.
 * Window ring (one per layer): sequence b, slot t at (b*C + t)*swa_row_bytes: D E4M3FN
 *   codes then D/32 E8M0 scales; position p lives in slot p % C, C >= W.                */
typedef struct csa2_layout_info {
    size_t idx_block_bytes; /* 8*KH*(d_I/2 + d_I/32), KH = 1 with shared_key else H_I */
    size_t kv_row_bytes;    /* D/2 + D/32             */
    size_t kv_block_bytes;  /* 8*kv_row_bytes         */
    size_t swa_row_bytes;   /* D + D/32               */
} csa2_layout_info;

/* Fills *out for cfg.  Host only. */
int csa2_layout(const csa2_config *cfg, csa2_layout_info *out);

/* Workspace bytes for op (CSA2_OP_*) at `batch` sequences and block-table width `maxb`.
 * Host only; *bytes is written. */
int csa2_workspace_bytes(const csa2_config *cfg, int op, int32_t batch, int32_t maxb,
                         size_t *bytes);

/* MXFP4 quantisation of n_rows rows of `dim` fp32 values (dim % 32 == 0) [KV]:
 * per 32-group e = floor(log2(amax)) - 2 (>= -127; amax = 0 gives -127), scale code e+127;
 * element code = E2M1 value nearest to x*2^-e, ties to the even code, saturating at 6,
 * sign bit = sign bit of x.  codes [n_rows][dim/2], scales [n_rows][dim/32]. */
int csa2_quantize_mxfp4(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                        uint8_t *scales, hipStream_t stream);

/* MXFP8 (E4M3FN) quantisation, same rules with e = floor(log2(amax)) - 8 and saturation at
 * 448 [KV].  codes [n_rows][dim], scales [n_rows][dim/32]. */
int csa2_quantize_mxfp8(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                        uint8_t *scales, hipStream_t stream);

/* Exact dequantisation to fp32 (code value * 2^(scale-127)); for tests and inspection. */
int csa2_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                       int32_t dim, float *out, hipStream_t stream);
int csa2_dequant_mxfp8(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                       int32_t dim, float *out, hipStream_t stream);

/* Full-layer append [KV]: for each sequence b and t < n_new, quantise position
 * p = pos0[b] + t -- main latent row latent[(b*n_new + t)*D ..] (MXFP4) and indexer key
 * idx_k[(b*n_new + t)*KH*d_I ..] (head-major, MXFP4 per head group; KH = 1 with shared_key,
 * else H_I) -- into the block
 * table's block p/8, slot p%8.  Either latent or idx_k may be NULL to skip that cache.
 * pos0 [batch] is a device array; positions whose block is outside the table or whose
 * physical block is outside [0, n_blocks) are skipped. */
int csa2_append_global(const csa2_config *cfg, const float *latent, const float *idx_k,
                       const int32_t *block_table, int32_t maxb, int64_t n_blocks,
                       const int32_t *pos0, int32_t batch, int32_t n_new, uint8_t *kv_cache,
                       uint8_t *idx_cache, hipStream_t stream);

/* Block transfer for the persistent global-KV tier [KV] (the global caches are kept in host
 * memory or on SSD for later prefix hits; the window cache is not): csa2_blocks_gather
 * copies the n physical blocks blocks[0..n) (device int32) of a block cache (n_blocks blocks
 * of block_bytes each -- csa2_layout's kv_block_bytes or idx_block_bytes) into n
 * consecutive rows of `rows` (device, n * block_bytes bytes); csa2_blocks_scatter copies the
 * rows back into the listed blocks, which may differ from the ones they came from (a
 * restored sequence gets a new block table).  The caller moves `rows` between device and
 * host memory (hipMemcpyAsync with pinned host memory).  The bytes are copied unchanged, so
 * a restored cache indexes and attends exactly as the saved one.  Entries outside
 * [0, n_blocks): gather writes a zero row, scatter skips the row.  INVALID if block_bytes
 * is not a positive multiple of 16, n < 0, n_blocks <= 0 or a pointer is NULL with n > 0.
 * Rows and cache must not overlap. */
int csa2_blocks_gather(const uint8_t *cache, int64_t n_blocks, int64_t block_bytes,
                       const int32_t *blocks, int32_t n, uint8_t *rows, hipStream_t stream);
int csa2_blocks_scatter(const uint8_t *rows, const int32_t *blocks, int32_t n, uint8_t *cache,
                        int64_t n_blocks, int64_t block_bytes, hipStream_t stream);

/* Window append (every layer) [KV][W]: quantise rows[(b*n_new + t)*D ..] to MXFP8 into the
 * ring slot (pos0[b] + t) % C of sequence b.  Negative positions are skipped. */
int csa2_append_swa(const csa2_config *cfg, const float *rows, const int32_t *pos0,
                    int32_t batch, int32_t n_new, uint8_t *swa_cache, int32_t C,
                    hipStream_t stream);

/* Indexer scores of every visible position, for tests and inspection [KV]:
 *   s(p) = sum_h w_h * ReLU(q_h . k_{p,h}), in this fixed fp32 order: per 32-group the
 *   exact dot N_j of doubled E2M1 values, t_j = N_j * 2^(E_j - 2) with E_j the sum of the
 *   two unbiased scale exponents, D_h = ((t_0 + t_1) + t_2) + ..., r_h = max(D_h, +0),
 *   s = fma(w_{H-1}, r_{H-1}, ... fma(w_0, r_0, +0)).
 *   Precondition: |E_j - 2| <= 100 for every group whose N_j != 0 (so each t_j is exact).
 * q_codes [batch][H_I*d_I/2], q_scales [batch][H_I*d_I/32] (an MXFP4 row per sequence,
 * head-major), w [batch][H_I] fp32, ctx_len [batch] (device).  Writes scores
 * [batch][maxb*8] for p < L_b and block maxima block_scores [batch][maxb] for blocks
 * j < ceil(L_b/8) (either may be NULL); other entries are not written.  batch <= 4096. */
int csa2_index_scores(const csa2_config *cfg, const uint8_t *q_codes, const uint8_t *q_scales,
                      const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                      const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                      int32_t batch, float *scores, float *block_scores, hipStream_t stream);

/* Full mode [KV][HSI]: score every visible position (as csa2_index_scores), reduce each
 * 8-position block to the max over its visible positions, keep the pool of the K_blk best
 * blocks, then the k best positions inside the pool (same scores).  Order: score
 * descending, lower index first on ties.  Outputs ascending, padded with -1:
 * pool_blocks [batch][K_blk] (logical block ids), pool_len [batch], topk [batch][k]
 * (positions), topk_len [batch].  A sequence with L_b <= 0 gets empty outputs.
 * Workspace: CSA2_OP_INDEX_FULL bytes (do not share it with csa2_sparse_attn).
 * batch <= 4096. */
int csa2_index_full(const csa2_config *cfg, const uint8_t *q_codes, const uint8_t *q_scales,
                    const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                    const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                    int32_t batch, int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                    int32_t *topk_len, void *ws, size_t ws_bytes, hipStream_t stream);

/* csa2_index_full in two phases on the same workspace and arguments: the scan (one
 * kernel: scores, block maxima, pool threshold) and the rest (pool selection, in-pool
 * rescoring and top-k).  Full == full_scan followed by full_finish. */
int csa2_index_full_scan(const csa2_config *cfg, const uint8_t *q_codes,
                         const uint8_t *q_scales, const float *w, const uint8_t *idx_cache,
                         int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                         const int32_t *ctx_len, int32_t batch, void *ws, size_t ws_bytes,
                         hipStream_t stream);
int csa2_index_full_finish(const csa2_config *cfg, const uint8_t *q_codes,
                           const uint8_t *q_scales, const float *w, const uint8_t *idx_cache,
                           int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                           const int32_t *ctx_len, int32_t batch, int32_t *pool_blocks,
                           int32_t *pool_len, int32_t *topk, int32_t *topk_len, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* Global append fused with the Full index step (a Full layer appends its token to the
 * global caches [KV], then indexes the context that includes it): exactly
 * csa2_append_global(cfg, latent, idx_k, block_table, maxb, n_blocks, pos0 = ctx_len - 1,
 * batch, 1, kv_cache, idx_cache) followed by csa2_index_full(cfg, q_codes, ...), bit for bit
 * (cache bytes, pool and top-k), in one scan launch and one selection launch: the wave that
 * scores the block of position ctx_len[b] - 1 quantises that token's key and writes it (and
 * the latent row) before it reads the block.  With d_I = 128 and H_I >= 2 the append runs as
 * a launch of its own before the scan (same results).  latent [batch][512] fp32 (may be NULL: no
 * main-KV append; kv_cache may then be NULL), idx_k [batch][H_I*d_I] fp32, on the device.
 * A sequence with ctx_len <= 0 or ctx_len > 8*maxb appends nothing (as the two calls).
 * Workspace: CSA2_OP_INDEX_FULL bytes.  UNSUPPORTED if latent is given and kv_dim != 512. */
int csa2_index_full_append(const csa2_config *cfg, const float *latent, const float *idx_k,
                           const uint8_t *q_codes, const uint8_t *q_scales, const float *w,
                           uint8_t *kv_cache, uint8_t *idx_cache, int64_t n_blocks,
                           const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                           int32_t batch, int32_t *pool_blocks, int32_t *pool_len,
                           int32_t *topk, int32_t *topk_len, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* Reindex mode [KV][RR]: rescore only the positions of the stored pool (pool_blocks /
 * pool_len of the latest Full layer) with this layer's q/w and keep the k best, as in
 * csa2_index_full (same workspace rules).  Reuse mode has no index call: pass the previous
 * topk on. */
int csa2_index_reindex(const csa2_config *cfg, const uint8_t *q_codes,
                       const uint8_t *q_scales, const float *w, const uint8_t *idx_cache,
                       int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                       const int32_t *ctx_len, int32_t batch, const int32_t *pool_blocks,
                       const int32_t *pool_len, int32_t *topk, int32_t *topk_len, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* Prefill indexer [KV]: n_q consecutive query tokens of ONE sequence, query i at position
 * t_i = q_pos0 + i, each run the Full-mode steps of csa2_index_full on their own causal
 * prefix (context length L_i = t_i + 1): score every position p <= t_i, block maxima, pool
 * of the K_blk best blocks, top-k inside the pool.  Same score definition, order and
 * output conventions as csa2_index_full, per query: pool_blocks [n_q][K_blk], pool_len
 * [n_q], topk [n_q][k], topk_len [n_q].  q_codes [n_q][H_I*d_I/2], q_scales
 * [n_q][H_I*d_I/32], w [n_q][H_I]; block_table is the sequence's row of maxb entries
 * (device), q_pos0 and n_q are host values with q_pos0 + n_q <= 8*maxb.  The products run
 * on the FP4 matrix cores; results are bit-identical to the per-query Full mode.
 * Workspace: CSA2_OP_INDEX_PREFILL bytes for batch = n_q (about 32*maxb bytes per query). */
int csa2_index_prefill(const csa2_config *cfg, const uint8_t *q_codes, const uint8_t *q_scales,
                       const float *w, int32_t q_pos0, int32_t n_q, const uint8_t *idx_cache,
                       int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                       int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                       int32_t *topk_len, void *ws, size_t ws_bytes, hipStream_t stream);

/* Sparse attention [KV][3][W]: for each sequence b and head h, one softmax over
 *   the main-KV rows of positions topk[b][0 .. topk_len[b]) (entries -1 are padding), and
 *   the window rows of positions max(0, L_b - W) .. L_b - 1 from the ring,
 * with K = V = the dequantised 512-d latent / window row and logits sm_scale * q.k (no
 * de-duplication between the two sets).  q [batch][H_q][D] bf16 bits; out [batch][H_q][D]
 * fp32; lse [batch][H_q] fp32 (natural log).  An empty set gives out = 0, lse = -inf. */
int csa2_sparse_attn(const csa2_config *cfg, const uint16_t *q, const uint8_t *kv_cache,
                     int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                     const uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                     int32_t batch, const int32_t *topk, const int32_t *topk_len, float *out,
                     float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/* Window append fused with sparse attention (every layer appends its own window row [W]
 * and then attends [KV][3]): exactly csa2_append_swa(cfg, swa_rows, pos, batch, 1,
 * swa_cache, C) followed by csa2_sparse_attn(cfg, q, ...), in one launch pair.  swa_rows
 * [batch][D] fp32 on the device; pos [batch] device positions (negative: no append).  The
 * appended row is quantised once and attended from registers, so it is bit-identical to
 * the two-call sequence.  Precondition (as for the two calls): slot pos[b] % C holds no row
 * of the attended window other than position pos[b] itself (C > W, or pos[b] = L_b - 1). */
int csa2_sparse_attn_append(const csa2_config *cfg, const float *swa_rows, const int32_t *pos,
                            const uint16_t *q, const uint8_t *kv_cache, int64_t n_blocks,
                            const int32_t *block_table, int32_t maxb, uint8_t *swa_cache,
                            int32_t C, const int32_t *ctx_len, int32_t batch,
                            const int32_t *topk, const int32_t *topk_len, float *out,
                            float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/* csa2_index_prefill in two phases on the same workspace and arguments: the scoring (key
 * spans + the matrix-core kernel: block and group maxima of every query, and with at most
 * 16 queries every causal position score) and the per-query selection (with more than 16
 * queries: the pools, then a second matrix-core pass that recomputes the position scores of
 * the pool blocks whose maximum reaches the k-th largest maximum of the pool -- the only
 * blocks the top-k can draw from -- then the top-k).  prefill == prefill_scan followed by
 * prefill_finish. */
int csa2_index_prefill_scan(const csa2_config *cfg, const uint8_t *q_codes,
                            const uint8_t *q_scales, const float *w, int32_t q_pos0,
                            int32_t n_q, const uint8_t *idx_cache, int64_t n_blocks,
                            const int32_t *block_table, int32_t maxb, void *ws, size_t ws_bytes,
                            hipStream_t stream);
int csa2_index_prefill_finish(const csa2_config *cfg, const uint8_t *q_codes,
                              const uint8_t *q_scales, const float *w, int32_t q_pos0,
                              int32_t n_q, const uint8_t *idx_cache, int64_t n_blocks,
                              const int32_t *block_table, int32_t maxb, int32_t *pool_blocks,
                              int32_t *pool_len, int32_t *topk, int32_t *topk_len, void *ws,
                              size_t ws_bytes, hipStream_t stream);

/* Prefill attention [KV][3][W]: n_q consecutive query tokens of ONE sequence, query i at
 * position t_i = q_pos0 + i, each attend as csa2_sparse_attn does for a sequence of length
 * t_i + 1: the main-KV rows of topk[i][0 .. topk_len[i]) and the window rows
 * max(0, t_i + 1 - W) .. t_i.  block_table is the sequence's row of maxb entries;
 * swa_ring is the sequence's ring of C slots (position p in slot p % C), which must still
 * hold every attended window row, i.e. C >= n_q + W - 1 once the chunk's rows are in it
 * (INVALID otherwise, with W > 0 and n_q > 0).
 * q [n_q][H_q][D] bf16 bits; out [n_q][H_q][D], lse [n_q][H_q].  q_pos0, n_q are host values
 * with q_pos0 + n_q <= 8*maxb.  Workspace: CSA2_OP_SPARSE_ATTN bytes for batch = n_q. */
int csa2_sparse_attn_prefill(const csa2_config *cfg, const uint16_t *q,
                             const uint8_t *kv_cache, int64_t n_blocks,
                             const int32_t *block_table, int32_t maxb, const uint8_t *swa_ring,
                             int32_t C, int32_t q_pos0, int32_t n_q, const int32_t *topk,
                             const int32_t *topk_len, float *out, float *lse, void *ws,
                             size_t ws_bytes, hipStream_t stream);

/* One decode layer per call (N4 of the design: the steps of a layer fused into as few
 * launches as their data dependences allow).  Modes as [KV] defines them: a Full layer
 * appends its token and scans the whole visible context into a pool and a top-k, a Reindex
 * layer rescores the latest pool, a Reuse layer keeps the latest top-k; every layer appends
 * its token's window row and attends its top-k rows plus its window [3][W].  The token is
 * the one at position ctx_len[b] - 1 of each sequence.  Each call equals, bit for bit, the
 * separate calls it stands for (outputs, cache and ring bytes):
 *   full:    csa2_quantize_mxfp4(q_idx); csa2_index_full_append(tok_latent, tok_key, ...);
 *            csa2_sparse_attn_append(swa_row, pos = ctx_len - 1, ...)
 *   reindex: csa2_quantize_mxfp4(q_idx); csa2_index_reindex(...); csa2_sparse_attn_append
 *   reuse:   csa2_sparse_attn_append(swa_row, pos = ctx_len - 1, ...) with the given topk
 * The indexer query is quantised inside the scan, so the kernels per layer are: Full 3
 * (scan with the query quantise and the global append, selection, attention with the window
 * append; 4 when d_I = 128 and H_I >= 2, whose global append runs first), Reindex 3
 * (rescoring scan, selection, attention), Reuse 1.  q_idx [batch][H_I*d_I] fp32 (head-major),
 * w_idx [batch][H_I] fp32, tok_latent [batch][D] fp32 (may be NULL: no main-KV append),
 * tok_key [batch][H_I*d_I] fp32, swa_row [batch][D] fp32, q_attn [batch][H_q][D] bf16 bits.
 * ws_index: CSA2_OP_INDEX_FULL bytes; ws_attn: CSA2_OP_SPARSE_ATTN bytes (zeroed once, as
 * for csa2_sparse_attn).  Host-side argument errors of any step return before anything is
 * launched. */
int csa2_decode_full_layer(const csa2_config *cfg, const float *q_idx, const float *w_idx,
                           const float *tok_latent, const float *tok_key, const float *swa_row,
                           const uint16_t *q_attn, uint8_t *kv_cache, uint8_t *idx_cache,
                           int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                           uint8_t *swa_cache, int32_t C, const int32_t *ctx_len, int32_t batch,
                           int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                           int32_t *topk_len, float *out, float *lse, void *ws_index,
                           size_t ws_index_bytes, void *ws_attn, size_t ws_attn_bytes,
                           hipStream_t stream);
int csa2_decode_reindex_layer(const csa2_config *cfg, const float *q_idx, const float *w_idx,
                              const float *swa_row, const uint16_t *q_attn,
                              const uint8_t *kv_cache, const uint8_t *idx_cache,
                              int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                              uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                              int32_t batch, const int32_t *pool_blocks, const int32_t *pool_len,
                              int32_t *topk, int32_t *topk_len, float *out, float *lse,
                              void *ws_index, size_t ws_index_bytes, void *ws_attn,
                              size_t ws_attn_bytes, hipStream_t stream);
int csa2_decode_reuse_layer(const csa2_config *cfg, const float *swa_row, const uint16_t *q_attn,
                            const uint8_t *kv_cache, int64_t n_blocks, const int32_t *block_table,
                            int32_t maxb, uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                            int32_t batch, const int32_t *topk, const int32_t *topk_len,
                            float *out, float *lse, void *ws_attn, size_t ws_attn_bytes,
                            hipStream_t stream);

/* csa2_sparse_attn without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results as csa2_sparse_attn, bit for bit, with the split
 * partials and arrival counters in a 16 MiB device array the library holds on each GPU it
 * runs on (for the life of the process).  It allocates nothing, and calls no allocating
 * routine.  The first call on a device looks the array's address up (hipGetSymbolAddress,
 * the device current) and clears its counters with a fill kernel on `stream`; every call
 * leaves them at zero again.  All calls on one GPU share the array, so calls that overlap
 * on one GPU (other streams, other threads) race: serialise them.  A shape whose partials
 * exceed the array (csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN) > 16 MiB; with k = 512 and
 * W = 128: 16 heads at batch 512..1023, 64 heads at 128..255, 128 heads at 64..127) returns
 * CSA2_ERR_SCRATCH and launches nothing. */
int csa2_sparse_attn_noalloc(const csa2_config *cfg, const uint16_t *q, const uint8_t *kv_cache,
                             int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                             const uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                             int32_t batch, const int32_t *topk, const int32_t *topk_len,
                             float *out, float *lse, hipStream_t stream);

/* Human-readable status. */
const char *csa2_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
