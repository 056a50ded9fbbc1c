/* Runs every oracle entry point once on small seeded inputs (ragged batch, a prefill chunk,
 * edge values for the quantisers) so that AddressSanitizer and UndefinedBehaviorSanitizer
 * see each code path of oracle/csa2_oracle.c.  Built and run by tests/test_sanitize.py:
 *   gcc -std=c11 -g -O1 -fsanitize=address,undefined -fno-sanitize-recover=all
 *       -fno-omit-frame-pointer oracle/csa2_oracle.c tests/sanitize/oracle_driver.c -lm
 * Exit status 0 when every call returns the expected status and the outputs are in range. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_idx_heads, idx_dim, kv_dim, n_q_heads, swa_window, pool_blocks, topk;
    float sm_scale;
    int32_t shared_key;
} o_cfg;

int csa2o_quantize_mxfp4(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                         uint8_t *scales);
int csa2o_quantize_mxfp8(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                         uint8_t *scales);
int csa2o_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                        int32_t dim, double *out);
int csa2o_dequant_mxfp8(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                        int32_t dim, double *out);
int csa2o_append_global(const o_cfg *c, const float *latent, const float *idx_k,
                        const int32_t *block_table, int32_t maxb, const int32_t *pos0,
                        int32_t B, int32_t n_new, uint8_t *kv_cache, uint8_t *idx_cache,
                        int64_t n_blocks);
int csa2o_append_swa(const o_cfg *c, const float *rows, const int32_t *pos0, int32_t B,
                     int32_t n_new, uint8_t *swa_cache, int32_t C);
int csa2o_index_scores(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                       const float *w, const uint8_t *idx_cache, const int32_t *table_row,
                       int32_t L, float *scores);
int csa2o_block_scores(const float *scores, int32_t L, float *bscore);
int csa2o_index_full(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                     const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                     const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                     int32_t B, int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                     int32_t *topk_len, float *block_scores_out);
int csa2o_index_reindex(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                        const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                        const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                        int32_t B, const int32_t *pool_blocks, const int32_t *pool_len,
                        int32_t *topk, int32_t *topk_len);
int csa2o_index_prefill(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                        const float *w, int32_t q_pos0, int32_t n_q, const uint8_t *idx_cache,
                        int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                        int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                        int32_t *topk_len);
int csa2o_sparse_attn(const o_cfg *c, const uint16_t *q, const uint8_t *kv_cache,
                      int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                      const uint8_t *swa_cache, int32_t C, const int32_t *ctx_len, int32_t B,
                      const int32_t *topk, const int32_t *topk_len, double *out, double *lse);
int csa2o_sparse_attn_prefill(const o_cfg *c, const uint16_t *q, const uint8_t *kv_cache,
                              int64_t n_blocks, const int32_t *table_row, int32_t maxb,
                              const uint8_t *swa_ring, int32_t C, int32_t q_pos0, int32_t n_q,
                              const int32_t *topk, const int32_t *topk_len, double *out,
                              double *lse);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni(void) { /* xorshift64*, [0, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
static float gauss(void) {
    double u = uni() + 1e-12, v = uni();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static void fill(float *x, size_t n) { for (size_t i = 0; i < n; i++) x[i] = gauss(); }
static void *xcalloc(size_t n, size_t sz) {
    void *p = calloc(n ? n : 1, sz);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static int failures = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #cond); failures++; } } while (0)

static void codecs(void) {
    enum { R = 5, D = 64 };
    float x[R * D];
    double y[R * D];
    uint8_t c4[R * D / 2], c8[R * D], s[R * D / 32];
    fill(x, R * D);
    x[0] = 0.0f; x[1] = -0.0f; x[2] = 1e-40f; x[3] = -6.0f; x[4] = 7.5f; x[5] = 448.0f;
    for (int i = 64; i < 96; i++) x[i] = 0.0f;              /* an all-zero group */
    for (int i = 96; i < 128; i++) x[i] = 1e30f * (i & 1 ? 1 : -1);
    EXPECT(csa2o_quantize_mxfp4(x, R, D, c4, s) == 0);
    EXPECT(csa2o_dequant_mxfp4(c4, s, R, D, y) == 0);
    for (int i = 0; i < R * D; i++) EXPECT(isfinite(y[i]));
    EXPECT(csa2o_quantize_mxfp8(x, R, D, c8, s) == 0);
    EXPECT(csa2o_dequant_mxfp8(c8, s, R, D, y) == 0);
    for (int i = 0; i < R * D; i++) EXPECT(isfinite(y[i]));
    EXPECT(csa2o_quantize_mxfp4(x, R, 48, c4, s) != 0);     /* dim not a multiple of 32 */
}

static void decode_group(int shared) {
    o_cfg c = {4, 64, 512, 16, 16, 8, 20, 0.0441941738f, shared};
    const int B = 3, ctx[3] = {0, 37, 300}, maxb = 40, C = 24;
    const int KH = shared ? 1 : c.n_idx_heads;
    const int64_t nblk = (int64_t)B * maxb + 5;
    const size_t ib = 8 * (size_t)KH * (c.idx_dim / 2 + c.idx_dim / 32), kb = 8 * 272;
    uint8_t *idx = xcalloc(nblk, ib), *kv = xcalloc(nblk, kb), *swa = xcalloc((size_t)B * C, 528);
    int32_t *table = xcalloc((size_t)B * maxb, 4);
    for (int i = 0; i < B * maxb; i++) table[i] = (int32_t)((i * 7 + 3) % nblk);
    /* append every position of every sequence, one token at a time */
    float *lat = xcalloc(512, 4), *key = xcalloc((size_t)KH * c.idx_dim, 4), *row = xcalloc(512, 4);
    for (int b = 0; b < B; b++)
        for (int p = 0; p < ctx[b]; p++) {
            const int32_t pos = p;
            fill(lat, 512); fill(key, (size_t)KH * c.idx_dim); fill(row, 512);
            EXPECT(csa2o_append_global(&c, lat, key, table + (size_t)b * maxb, maxb, &pos, 1, 1,
                                       kv, idx, nblk) == 0);
            EXPECT(csa2o_append_swa(&c, row, &pos, 1, 1, swa + (size_t)b * C * 528, C) == 0);
        }
    float qf[4 * 64], w[4];
    uint8_t qc[4 * 32], qs[4 * 2];
    fill(qf, 4 * 64);
    for (int h = 0; h < 4; h++) w[h] = (float)(0.5 + uni());
    w[2] = -w[2];
    EXPECT(csa2o_quantize_mxfp4(qf, 4, 64, qc, qs) == 0);
    uint8_t *qcb = xcalloc((size_t)B * 128, 1), *qsb = xcalloc((size_t)B * 8, 1);
    float *wb = xcalloc((size_t)B * 4, 4);
    for (int b = 0; b < B; b++) {
        memcpy(qcb + b * 128, qc, 128); memcpy(qsb + b * 8, qs, 8); memcpy(wb + b * 4, w, 16);
    }
    float *sc = xcalloc(300, 4), *bs = xcalloc(40, 4);
    EXPECT(csa2o_index_scores(&c, qc, qs, w, idx, table + 2 * maxb, 300, sc) == 0);
    EXPECT(csa2o_block_scores(sc, 300, bs) == 0);
    int32_t pool[3 * 8], pl[3], topk[3 * 20], tl[3];
    float *bso = xcalloc((size_t)B * maxb, 4);
    EXPECT(csa2o_index_full(&c, qcb, qsb, wb, idx, nblk, table, maxb, ctx, B, pool, pl, topk, tl,
                            bso) == 0);
    for (int b = 0; b < B; b++) {
        EXPECT(pl[b] >= 0 && pl[b] <= 8 && tl[b] >= 0 && tl[b] <= 20);
        for (int i = 1; i < tl[b]; i++) EXPECT(topk[b * 20 + i - 1] < topk[b * 20 + i]);
    }
    EXPECT(csa2o_index_reindex(&c, qcb, qsb, wb, idx, nblk, table, maxb, ctx, B, pool, pl, topk,
                               tl) == 0);
    uint16_t *qa = xcalloc((size_t)B * 16 * 512, 2);
    for (size_t i = 0; i < (size_t)B * 16 * 512; i++) {
        float f = gauss(); uint32_t u; memcpy(&u, &f, 4); qa[i] = (uint16_t)(u >> 16);
    }
    double *out = xcalloc((size_t)B * 16 * 512, 8), *lse = xcalloc((size_t)B * 16, 8);
    EXPECT(csa2o_sparse_attn(&c, qa, kv, nblk, table, maxb, swa, C, ctx, B, topk, tl, out, lse) == 0);
    EXPECT(isinf(lse[0]) && lse[0] < 0);                    /* empty sequence */
    for (int i = 16; i < B * 16; i++) EXPECT(isfinite(lse[i]));
    /* prefill: 9 queries at 291..299 of sequence 2 (the ring holds their window) */
    if (!shared) {
        const int nq = 9, q0 = 291;
        uint8_t *pqc = xcalloc((size_t)nq * 128, 1), *pqs = xcalloc((size_t)nq * 8, 1);
        float *pw = xcalloc((size_t)nq * 4, 4);
        for (int q = 0; q < nq; q++) {
            memcpy(pqc + q * 128, qc, 128); memcpy(pqs + q * 8, qs, 8); memcpy(pw + q * 4, w, 16);
        }
        int32_t *ppool = xcalloc((size_t)nq * 8, 4), *ppl = xcalloc(nq, 4);
        int32_t *ptk = xcalloc((size_t)nq * 20, 4), *ptl = xcalloc(nq, 4);
        EXPECT(csa2o_index_prefill(&c, pqc, pqs, pw, q0, nq, idx, nblk, table + 2 * maxb, maxb,
                                   ppool, ppl, ptk, ptl) == 0);
        double *po = xcalloc((size_t)nq * 16 * 512, 8), *pl2 = xcalloc((size_t)nq * 16, 8);
        uint16_t *pqa = xcalloc((size_t)nq * 16 * 512, 2);
        for (size_t i = 0; i < (size_t)nq * 16 * 512; i++) pqa[i] = qa[i % ((size_t)B * 16 * 512)];
        EXPECT(csa2o_sparse_attn_prefill(&c, pqa, kv, nblk, table + 2 * maxb, maxb,
                                         swa + 2 * C * 528, C, q0, nq, ptk, ptl, po, pl2) == 0);
        for (int i = 0; i < nq * 16; i++) EXPECT(isfinite(pl2[i]));
        free(pqc); free(pqs); free(pw); free(ppool); free(ppl); free(ptk); free(ptl);
        free(po); free(pl2); free(pqa);
    }
    /* rejected shapes */
    o_cfg bad = c;
    bad.idx_dim = 48;
    EXPECT(csa2o_index_full(&bad, qcb, qsb, wb, idx, nblk, table, maxb, ctx, B, pool, pl, topk,
                            tl, bso) != 0);
    free(idx); free(kv); free(swa); free(table); free(lat); free(key); free(row); free(qcb);
    free(qsb); free(wb); free(sc); free(bs); free(bso); free(qa); free(out); free(lse);
}

int main(void) {
    codecs();
    decode_group(0);
    decode_group(1);
    if (failures) { fprintf(stderr, "%d failed checks\n", failures); return 1; }
    puts("oracle driver: ok");
    return 0;
}
