/*
 * csa2_oracle.c -- plain, slow CPU oracle for the CSA2 decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
 * baseline leg may load this library.  The GPU product path never calls it and shares
 * no code, header, table or constant with it.
 *
 * What it computes (sources are web pages on DeepSeek-V4.1-Flash, cited by address and
 * section heading):
 *   [KV]  dbyun.net/article/10794, section "KV Cache 成为这一代架构改造的核心":
 *         Full / Reindex / Reuse layer modes; the first Full layer of the decoder scans
 *         the whole visible context into a pool of at most 2048 blocks of 8 positions,
 *         later layers pick the final top-512 inside that pool; indexer Q/K and main KV
 *         are FP4, sliding-window KV stays FP8.
 *   [3]   10100.com/article/150771503, section "三招压缩，各有分工": decoder layers keep
 *         a layer-local sliding window; later indexers only search the candidate pool.
 *   [HSI] prism.simon-ai.net/article/7901, section "层级稀疏索引器：精准筛选关键信息".
 *   [RR]  prism.simon-ai.net/article/7901, section "重索引与复用的具体运作逻辑".
 *   [W]   prism.simon-ai.net/article/7901, section "短期记忆的去留：从SSD存储到GPU重算":
 *         the local window is 128 tokens.
 *
 * The pages fix none of the following; each is a stated reading (R-numbers are the
 * readings listed in the design notes of this repository):
 *   R1  FP4 = OCP MX E2M1, two codes per byte (even element in the low nibble), one
 *       E8M0 scale per 32 elements.  FP8 = OCP E4M3FN with the same E8M0 scaling.
 *   R2  shared exponent e = floor(log2(amax)) - emax_elem (2 for E2M1, 8 for E4M3FN),
 *       clamped to >= -127; amax == 0 gives e = -127.
 *   R3  element = nearest representable value of x * 2^-e, ties to the even code,
 *       magnitudes beyond the largest finite value saturate; the code's sign bit is the
 *       sign bit of x.
 *   R5  indexer score s(p) = sum_h w_h * ReLU(q_h . k_{p,h}), evaluated in fp32 in a
 *       fixed order: per 32-group an exact integer dot of doubled codes N_j, then
 *       t_j = N_j * 2^(E_j - 2), D_h = ((t_0 + t_1) + t_2) + ..., r_h = max(D_h, +0),
 *       s = fma(w_{H-1}, r_{H-1}, ... fma(w_0, r_0, +0)).
 *       Shared-key reading (a "next" variant, config field shared_key = 1): each position
 *       stores ONE d_I key, and s(p) = sum_h w_h * ReLU(q_h . k_p) with the same fixed
 *       order (query head h's group j meets the key's group j).
 *   R6  block score = max of s over the visible positions of an 8-position block.
 *   R7  selection order (score desc, index asc); outputs ascending, -1 padded.
 *   R9  attention: K = V = dequantised latent (512), joint softmax over the selected
 *       rows plus the window rows, no de-duplication, computed here in fp64.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * OpenMP only splits independent units (positions, sequences, heads); no arithmetic is
 * reordered by it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BLK 8 /* positions per block [KV] */

typedef struct {
    int32_t n_idx_heads; /* H_I */
    int32_t idx_dim;     /* d_I, multiple of 32 */
    int32_t kv_dim;      /* D, multiple of 32 */
    int32_t n_q_heads;   /* H_q */
    int32_t swa_window;  /* W */
    int32_t pool_blocks; /* K_blk */
    int32_t topk;        /* k */
    float sm_scale;
    int32_t shared_key;  /* 0: one key per head per position; 1: one key per position, scored
                            by all H_I query heads (the shared-key indexer reading) */
} o_cfg;

enum { O_OK = 0, O_BAD = -1, O_PRECOND = -5 };

/* ------------------------------------------------------------------ format values */

/* E2M1 (R1): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0. */
double csa2o_fp4_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? ldexp((double)m, -1)                 /* subnormal: m/2 * 2^0 */
                          : ldexp(1.0 + (double)m / 2.0, e - 1); /* normal */
    return s ? -mag : mag;
}

/* E4M3FN (R1): sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0; S.1111.111
 * is NaN, there is no infinity. */
double csa2o_fp8_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0: 2^(code - 127); 0xFF is NaN. */
double csa2o_e8m0_value(int code) {
    if (code == 255) return NAN;
    return ldexp(1.0, code - 127);
}

/* ------------------------------------------------------------------ quantisers */

static int floor_log2(double a) { /* a finite, > 0; exact */
    int e;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    return e - 1;
}

/* Shared exponent of one 32-group (R2). */
static int group_exponent(const float *x, int emax_elem) {
    double amax = 0.0;
    for (int i = 0; i < 32; i++) {
        double a = fabs((double)x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0) return -127;
    int e = floor_log2(amax) - emax_elem;
    return e < -127 ? -127 : e;
}

/* Nearest non-negative code to magnitude a among codes 0..n-1 (values increasing),
 * ties to the even code (R3).  A tie can only be between neighbours, one even, one odd. */
static int nearest_code(double a, double (*value)(int), int n) {
    int best = 0;
    double bestd = fabs(a - value(0));
    for (int c = 1; c < n; c++) {
        double d = fabs(a - value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

static int sign_bit(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return (int)(u >> 31);
}

/* One MXFP4 row of dim elements -> dim/2 code bytes + dim/32 scale bytes. */
static void quant_row_fp4(const float *x, int dim, uint8_t *codes, uint8_t *scales) {
    memset(codes, 0, (size_t)dim / 2);
    for (int g = 0; g < dim / 32; g++) {
        const float *xg = x + 32 * g;
        int e = group_exponent(xg, 2);
        scales[g] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; i++) {
            double a = ldexp(fabs((double)xg[i]), -e); /* exact */
            int c = nearest_code(a, csa2o_fp4_value, 8) | (sign_bit(xg[i]) << 3);
            int el = 32 * g + i;
            codes[el / 2] |= (uint8_t)(c << ((el & 1) * 4));
        }
    }
}

static void quant_row_fp8(const float *x, int dim, uint8_t *codes, uint8_t *scales) {
    for (int g = 0; g < dim / 32; g++) {
        const float *xg = x + 32 * g;
        int e = group_exponent(xg, 8);
        scales[g] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; i++) {
            double a = ldexp(fabs((double)xg[i]), -e);
            int c = nearest_code(a, csa2o_fp8_value, 127) | (sign_bit(xg[i]) << 7);
            codes[32 * g + i] = (uint8_t)c;
        }
    }
}

int csa2o_quantize_mxfp4(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                         uint8_t *scales) {
    if (dim <= 0 || dim % 32) return O_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; r++)
        quant_row_fp4(x + r * dim, dim, codes + r * (dim / 2), scales + r * (dim / 32));
    return O_OK;
}

int csa2o_quantize_mxfp8(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                         uint8_t *scales) {
    if (dim <= 0 || dim % 32) return O_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; r++)
        quant_row_fp8(x + r * dim, dim, codes + r * dim, scales + r * (dim / 32));
    return O_OK;
}

int csa2o_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                        int32_t dim, double *out) {
    if (dim <= 0 || dim % 32) return O_BAD;
    for (int64_t r = 0; r < n_rows; r++)
        for (int i = 0; i < dim; i++) {
            int c = (codes[r * (dim / 2) + i / 2] >> ((i & 1) * 4)) & 15;
            out[r * dim + i] =
                csa2o_fp4_value(c) * csa2o_e8m0_value(scales[r * (dim / 32) + i / 32]);
        }
    return O_OK;
}

int csa2o_dequant_mxfp8(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                        int32_t dim, double *out) {
    if (dim <= 0 || dim % 32) return O_BAD;
    for (int64_t r = 0; r < n_rows; r++)
        for (int i = 0; i < dim; i++)
            out[r * dim + i] = csa2o_fp8_value(codes[r * dim + i]) *
                               csa2o_e8m0_value(scales[r * (dim / 32) + i / 32]);
    return O_OK;
}

/* ------------------------------------------------------------------ cache layout
 * Global caches are paged in blocks of 8 positions; block_table[b*maxb + j] is the
 * physical block holding positions 8j .. 8j+7 of sequence b.
 *
 * Indexer-key block (H = H_I, G = d_I/32 groups per head):
 *   codes : 16 bytes (one 32-group) at offset ((g*8 + s)*H + h)*16 for group g of head h
 *           of the position in slot s;  8*H*d_I/2 bytes in all
 *   scales: one byte at 8*H*d_I/2 + (s*H + h)*G + g
 * Main-KV block: slot s at s*(D/2 + D/32): D/2 code bytes, then D/32 scale bytes.
 * Window ring: sequence b, slot t at (b*C + t)*(D + D/32): D FP8 codes, D/32 scales;
 *   position p lives in slot p % C.                                                 */

/* Key heads stored per position: H_I, or 1 when every query head scores the same key. */
static int key_heads(const o_cfg *c) { return c->shared_key ? 1 : c->n_idx_heads; }

static size_t idx_block_bytes(const o_cfg *c) {
    return (size_t)BLK * key_heads(c) * (c->idx_dim / 2 + c->idx_dim / 32);
}
static size_t kv_row_bytes(const o_cfg *c) { return (size_t)c->kv_dim / 2 + c->kv_dim / 32; }
static size_t swa_row_bytes(const o_cfg *c) { return (size_t)c->kv_dim + c->kv_dim / 32; }

static int cfg_ok(const o_cfg *c) {
    return c && c->n_idx_heads > 0 && c->idx_dim > 0 && c->idx_dim % 32 == 0 &&
           c->kv_dim > 0 && c->kv_dim % 32 == 0 && c->n_q_heads > 0 && c->swa_window >= 0 &&
           c->pool_blocks > 0 && c->topk > 0 && (c->shared_key == 0 || c->shared_key == 1);
}

/* Write position p's indexer key (one MXFP4 row of KH*d_I, head-major, KH = key heads)
 * into its block. */
static void put_idx_key(const o_cfg *c, uint8_t *blk, int s, const uint8_t *codes,
                        const uint8_t *scales) {
    int H = key_heads(c), G = c->idx_dim / 32;
    size_t codes_bytes = (size_t)BLK * H * c->idx_dim / 2;
    for (int h = 0; h < H; h++)
        for (int g = 0; g < G; g++) {
            memcpy(blk + ((size_t)(g * BLK + s) * H + h) * 16, codes + (h * G + g) * 16, 16);
            blk[codes_bytes + (size_t)(s * H + h) * G + g] = scales[h * G + g];
        }
}

/* Read position p's key back as a head-major MXFP4 row. */
static void get_idx_key(const o_cfg *c, const uint8_t *blk, int s, uint8_t *codes,
                        uint8_t *scales) {
    int H = key_heads(c), G = c->idx_dim / 32;
    size_t codes_bytes = (size_t)BLK * H * c->idx_dim / 2;
    for (int h = 0; h < H; h++)
        for (int g = 0; g < G; g++) {
            memcpy(codes + (h * G + g) * 16, blk + ((size_t)(g * BLK + s) * H + h) * 16, 16);
            scales[h * G + g] = blk[codes_bytes + (size_t)(s * H + h) * G + g];
        }
}

/* Append n_new positions per sequence, starting at pos0[b], to the global caches. */
int csa2o_append_global(const o_cfg *c, const float *latent, const float *idx_k,
                        const int32_t *block_table, int32_t maxb, const int32_t *pos0,
                        int32_t B, int32_t n_new, uint8_t *kv_cache, uint8_t *idx_cache,
                        int64_t n_blocks) {
    if (!cfg_ok(c) || B < 0 || n_new < 0) return O_BAD;
    int D = c->kv_dim, HI = key_heads(c) * c->idx_dim;
    for (int b = 0; b < B; b++)
        for (int t = 0; t < n_new; t++) {
            int64_t p = (int64_t)pos0[b] + t;
            if (p < 0 || p / BLK >= maxb) return O_BAD;
            int64_t phys = block_table[(int64_t)b * maxb + p / BLK];
            if (phys < 0 || phys >= n_blocks) return O_BAD;
        }
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int t = 0; t < n_new; t++) {
            int64_t p = (int64_t)pos0[b] + t;
            int64_t phys = block_table[(int64_t)b * maxb + p / BLK];
            int s = (int)(p % BLK);
            size_t row = (size_t)b * n_new + t;
            if (kv_cache) {
                uint8_t *dst = kv_cache + phys * BLK * kv_row_bytes(c) + s * kv_row_bytes(c);
                quant_row_fp4(latent + row * D, D, dst, dst + D / 2);
            }
            if (idx_cache) {
                uint8_t codes[4096], scales[256];
                if (HI > 8192) continue; /* not reached: checked by callers' configs */
                quant_row_fp4(idx_k + row * HI, HI, codes, scales);
                put_idx_key(c, idx_cache + phys * idx_block_bytes(c), s, codes, scales);
            }
        }
    return O_OK;
}

int csa2o_append_swa(const o_cfg *c, const float *rows, const int32_t *pos0, int32_t B,
                     int32_t n_new, uint8_t *swa_cache, int32_t C) {
    if (!cfg_ok(c) || C <= 0 || B < 0 || n_new < 0) return O_BAD;
    int D = c->kv_dim;
    for (int b = 0; b < B; b++)
        for (int t = 0; t < n_new; t++) {
            int64_t p = (int64_t)pos0[b] + t;
            if (p < 0) return O_BAD;
            uint8_t *dst = swa_cache + ((size_t)b * C + (size_t)(p % C)) * swa_row_bytes(c);
            quant_row_fp8(rows + ((size_t)b * n_new + t) * D, D, dst, dst + D);
        }
    return O_OK;
}

/* ------------------------------------------------------------------ indexer score (R5) */

/* Doubled E2M1 value: an integer in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}. */
static int doubled(int code) { return (int)(2.0 * csa2o_fp4_value(code)); }

static int nib(const uint8_t *codes, int i) { return (codes[i / 2] >> ((i & 1) * 4)) & 15; }

/* Score of one key against the query (head-major MXFP4 row of H*d_I); the key is a
 * head-major row of H*d_I, or of d_I when the key is shared by the heads (query head h then
 * meets the same key groups g = 0..G-1).  Returns O_PRECOND through *bad when a group
 * exponent leaves the range where t_j is an exact fp32. */
static float score_key(const o_cfg *c, const uint8_t *qc, const uint8_t *qs, const float *w,
                       const uint8_t *kc, const uint8_t *ks, int *bad) {
    int H = c->n_idx_heads, G = c->idx_dim / 32;
    float s = 0.0f;
    for (int h = 0; h < H; h++) {
        float Dh = 0.0f;
        for (int g = 0; g < G; g++) {
            int base = (h * G + g) * 32;                      /* query group */
            int kg = c->shared_key ? g : h * G + g;           /* key group */
            long N = 0;
            for (int i = 0; i < 32; i++)
                N += (long)doubled(nib(qc, base + i)) * doubled(nib(kc, kg * 32 + i));
            int E = ((int)qs[h * G + g] - 127) + ((int)ks[kg] - 127);
            if (N != 0 && (E - 2 > 100 || E - 2 < -100)) *bad = 1; /* t_j exact */
            float t = ldexpf((float)N, E - 2);
            Dh = Dh + t;
        }
        float r = Dh > 0.0f ? Dh : 0.0f;
        s = fmaf(w[h], r, s);
    }
    return s;
}

/* Per-position scores s(p) for p < L of one sequence (all positions scanned, [KV]). */
int csa2o_index_scores(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                       const float *w, const uint8_t *idx_cache, const int32_t *table_row,
                       int32_t L, float *scores) {
    if (!cfg_ok(c)) return O_BAD;
    int HI = c->n_idx_heads * c->idx_dim;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int32_t p = 0; p < L; p++) {
        uint8_t kc[4096], ks[256];
        const uint8_t *blk = idx_cache + (size_t)table_row[p / BLK] * idx_block_bytes(c);
        get_idx_key(c, blk, p % BLK, kc, ks);
        int b1 = 0;
        scores[p] = score_key(c, q_codes, q_scales, w, kc, ks, &b1);
        bad |= b1;
    }
    (void)HI;
    return bad ? O_PRECOND : O_OK;
}

/* ------------------------------------------------------------------ selection (R7) */

typedef struct {
    float score;
    int32_t index;
} o_item;

static int by_score_desc_index_asc(const void *a, const void *b) {
    const o_item *x = a, *y = b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->index > y->index) - (x->index < y->index);
}

static int int_asc(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Top-K of n items by (score desc, index asc) -> indices ascending, -1 padded. */
static int32_t select_top(o_item *items, int32_t n, int32_t K, int32_t *out) {
    qsort(items, (size_t)n, sizeof(o_item), by_score_desc_index_asc);
    int32_t m = n < K ? n : K;
    for (int32_t i = 0; i < m; i++) out[i] = items[i].index;
    qsort(out, (size_t)m, sizeof(int32_t), int_asc);
    for (int32_t i = m; i < K; i++) out[i] = -1;
    return m;
}

/* Block scores (R6): max of s(p) over visible positions of each block. */
int csa2o_block_scores(const float *scores, int32_t L, float *bscore) {
    int32_t nb = (L + BLK - 1) / BLK;
    for (int32_t j = 0; j < nb; j++) {
        float m = -INFINITY;
        for (int s = 0; s < BLK; s++) {
            int32_t p = j * BLK + s;
            if (p < L && scores[p] > m) m = scores[p];
        }
        bscore[j] = m;
    }
    return O_OK;
}

/* Final top-k among the visible positions of the pool blocks, scored with (q, w). */
static int32_t final_in_pool(const o_cfg *c, const uint8_t *qc, const uint8_t *qs,
                             const float *w, const uint8_t *idx_cache, const int32_t *table_row,
                             int32_t L, const int32_t *pool, int32_t pool_len, int32_t *topk,
                             const float *known_scores, int *bad) {
    o_item *items = malloc(sizeof(o_item) * (size_t)(pool_len > 0 ? pool_len : 1) * BLK);
    int32_t n = 0;
    for (int32_t i = 0; i < pool_len; i++) {
        int32_t j = pool[i];
        for (int s = 0; s < BLK; s++) {
            int32_t p = j * BLK + s;
            if (p >= L) continue;
            float sc;
            if (known_scores) {
                sc = known_scores[p];
            } else {
                uint8_t kc[4096], ks[256];
                get_idx_key(c, idx_cache + (size_t)table_row[j] * idx_block_bytes(c), s, kc, ks);
                sc = score_key(c, qc, qs, w, kc, ks, bad);
            }
            items[n].score = sc;
            items[n].index = p;
            n++;
        }
    }
    int32_t m = select_top(items, n, c->topk, topk);
    free(items);
    return m;
}

static int check_table(const o_cfg *c, const int32_t *table, int32_t maxb, int32_t B,
                       const int32_t *ctx_len, int64_t n_blocks) {
    for (int b = 0; b < B; b++) {
        int32_t L = ctx_len[b];
        if (L < 0 || (int64_t)L > (int64_t)maxb * BLK) return O_BAD;
        for (int32_t j = 0; j < (L + BLK - 1) / BLK; j++) {
            int32_t ph = table[(int64_t)b * maxb + j];
            if (ph < 0 || ph >= n_blocks) return O_BAD;
        }
    }
    (void)c;
    return O_OK;
}

/* Full mode: score everything, block-max, pool of top-K_blk blocks, final top-k inside
 * the pool with the same scores ([KV], [HSI]).  Optional block_scores_out [B, maxb]. */
int csa2o_index_full(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                     const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                     const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                     int32_t B, int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                     int32_t *topk_len, float *block_scores_out) {
    if (!cfg_ok(c) || B < 0) return O_BAD;
    if (check_table(c, block_table, maxb, B, ctx_len, n_blocks)) return O_BAD;
    int HI = c->n_idx_heads * c->idx_dim;
    int status = O_OK;
    for (int b = 0; b < B; b++) {
        int32_t L = ctx_len[b], nb = (L + BLK - 1) / BLK;
        const int32_t *row = block_table + (int64_t)b * maxb;
        const uint8_t *qc = q_codes + (size_t)b * HI / 2, *qs = q_scales + (size_t)b * HI / 32;
        float *scores = malloc(sizeof(float) * (size_t)(L > 0 ? L : 1));
        float *bs = malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
        if (csa2o_index_scores(c, qc, qs, w + (size_t)b * c->n_idx_heads, idx_cache, row, L,
                               scores) == O_PRECOND)
            status = O_PRECOND;
        csa2o_block_scores(scores, L, bs);
        if (block_scores_out)
            for (int32_t j = 0; j < nb; j++) block_scores_out[(int64_t)b * maxb + j] = bs[j];
        o_item *items = malloc(sizeof(o_item) * (size_t)(nb > 0 ? nb : 1));
        for (int32_t j = 0; j < nb; j++) {
            items[j].score = bs[j];
            items[j].index = j;
        }
        int32_t *pool = pool_blocks + (int64_t)b * c->pool_blocks;
        pool_len[b] = select_top(items, nb, c->pool_blocks, pool);
        int bad = 0;
        topk_len[b] = final_in_pool(c, qc, qs, NULL, idx_cache, row, L, pool, pool_len[b],
                                    topk + (int64_t)b * c->topk, scores, &bad);
        free(items);
        free(bs);
        free(scores);
    }
    return status;
}

/* Reindex mode: rescore the stored pool with this layer's own (q, w) ([KV], [RR]). */
int csa2o_index_reindex(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                        const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                        const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                        int32_t B, const int32_t *pool_blocks, const int32_t *pool_len,
                        int32_t *topk, int32_t *topk_len) {
    if (!cfg_ok(c) || B < 0) return O_BAD;
    if (check_table(c, block_table, maxb, B, ctx_len, n_blocks)) return O_BAD;
    int HI = c->n_idx_heads * c->idx_dim;
    int bad = 0;
    for (int b = 0; b < B; b++) {
        int32_t L = ctx_len[b], nb = (L + BLK - 1) / BLK;
        int32_t n = pool_len[b];
        const int32_t *pool = pool_blocks + (int64_t)b * c->pool_blocks;
        if (n < 0 || n > c->pool_blocks) return O_BAD;
        for (int32_t i = 0; i < n; i++)
            if (pool[i] < 0 || pool[i] >= nb) return O_BAD;
        topk_len[b] = final_in_pool(c, q_codes + (size_t)b * HI / 2,
                                    q_scales + (size_t)b * HI / 32,
                                    w + (size_t)b * c->n_idx_heads, idx_cache,
                                    block_table + (int64_t)b * maxb, L, pool, n,
                                    topk + (int64_t)b * c->topk, NULL, &bad);
    }
    return bad ? O_PRECOND : O_OK;
}

/* Prefill: query i sits at position t = q_pos0 + i and sees positions p <= t of the one
 * sequence; each query runs the Full-mode steps on its own visible prefix. */
int csa2o_index_prefill(const o_cfg *c, const uint8_t *q_codes, const uint8_t *q_scales,
                        const float *w, int32_t q_pos0, int32_t n_q, const uint8_t *idx_cache,
                        int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                        int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                        int32_t *topk_len) {
    if (!cfg_ok(c) || n_q < 0 || q_pos0 < 0) return O_BAD;
    int HI = c->n_idx_heads * c->idx_dim;
    int status = O_OK;
    for (int32_t i = 0; i < n_q; i++) {
        int32_t L = q_pos0 + i + 1;
        int st = csa2o_index_full(c, q_codes + (size_t)i * HI / 2, q_scales + (size_t)i * HI / 32,
                                  w + (size_t)i * c->n_idx_heads, idx_cache, n_blocks,
                                  block_table, maxb, &L, 1,
                                  pool_blocks + (int64_t)i * c->pool_blocks, pool_len + i,
                                  topk + (int64_t)i * c->topk, topk_len + i, NULL);
        if (st == O_BAD) return st;
        if (st == O_PRECOND) status = O_PRECOND;
    }
    return status;
}

/* ------------------------------------------------------------------ attention (R9) */

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Sparse attention over the selected main-KV rows plus the window rows (positions
 * max(0, L-W) .. L-1 of the layer's own ring), one joint softmax per (sequence, head).
 * out [B, H_q, D] and lse [B, H_q] in fp64; empty sets give out = 0, lse = -inf.
 * Entries of topk equal to -1 are padding; other entries must lie in [0, L). */
int csa2o_sparse_attn(const o_cfg *c, const uint16_t *q, const uint8_t *kv_cache,
                      int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                      const uint8_t *swa_cache, int32_t C, const int32_t *ctx_len, int32_t B,
                      const int32_t *topk, const int32_t *topk_len, double *out, double *lse) {
    if (!cfg_ok(c) || B < 0 || (c->swa_window > 0 && C < c->swa_window)) return O_BAD;
    int D = c->kv_dim, Hq = c->n_q_heads, k = c->topk, W = c->swa_window;
    for (int b = 0; b < B; b++) {
        int32_t L = ctx_len[b];
        if (L < 0 || (int64_t)L > (int64_t)maxb * BLK) return O_BAD;
        if (topk_len[b] < 0 || topk_len[b] > k) return O_BAD;
        for (int32_t i = 0; i < topk_len[b]; i++) {
            int32_t p = topk[(int64_t)b * k + i];
            if (p < -1 || p >= L) return O_BAD;
            if (p >= 0) {
                int32_t ph = block_table[(int64_t)b * maxb + p / BLK];
                if (ph < 0 || ph >= n_blocks) return O_BAD;
            }
        }
    }
    int status = O_OK;
    for (int b = 0; b < B; b++) {
        int32_t L = ctx_len[b];
        int32_t w0 = L - W > 0 ? L - W : 0;
        int32_t nsel = topk_len[b], nwin = L - w0;
        int32_t nrows = nsel + nwin;
        double *rows = malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1) * D);
        int32_t r = 0;
        for (int32_t i = 0; i < nsel; i++) {
            int32_t p = topk[(int64_t)b * k + i];
            if (p < 0) continue;
            const uint8_t *src = kv_cache +
                                 (size_t)block_table[(int64_t)b * maxb + p / BLK] * BLK * kv_row_bytes(c) +
                                 (size_t)(p % BLK) * kv_row_bytes(c);
            csa2o_dequant_mxfp4(src, src + D / 2, 1, D, rows + (size_t)r * D);
            r++;
        }
        for (int32_t p = w0; p < L; p++) {
            const uint8_t *src = swa_cache + ((size_t)b * C + (size_t)(p % C)) * swa_row_bytes(c);
            csa2o_dequant_mxfp8(src, src + D, 1, D, rows + (size_t)r * D);
            r++;
        }
        nrows = r;
#pragma omp parallel for schedule(static)
        for (int h = 0; h < Hq; h++) {
            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;
            double *o = out + ((size_t)b * Hq + h) * D;
            for (int d = 0; d < D; d++) o[d] = 0.0;
            if (nrows == 0) {
                lse[(size_t)b * Hq + h] = -INFINITY;
                continue;
            }
            double *z = malloc(sizeof(double) * (size_t)nrows);
            double m = -INFINITY;
            for (int32_t i = 0; i < nrows; i++) {
                double acc = 0.0;
                for (int d = 0; d < D; d++) acc += bf16_value(qh[d]) * rows[(size_t)i * D + d];
                z[i] = (double)c->sm_scale * acc;
                if (z[i] > m) m = z[i];
            }
            double l = 0.0;
            for (int32_t i = 0; i < nrows; i++) {
                double e = exp(z[i] - m);
                l += e;
                for (int d = 0; d < D; d++) o[d] += e * rows[(size_t)i * D + d];
            }
            for (int d = 0; d < D; d++) o[d] /= l;
            lse[(size_t)b * Hq + h] = m + log(l);
            free(z);
        }
        free(rows);
    }
    return status;
}

/* Prefill attention: query i sits at position t = q_pos0 + i of the one sequence and
 * attends, as a decode step with context length t + 1 would, to its own top-k rows and to
 * the window rows max(0, t+1-W) .. t of the sequence's ring (the ring must still hold
 * them).  q [n_q, H_q, D]; out [n_q, H_q, D], lse [n_q, H_q]. */
int csa2o_sparse_attn_prefill(const o_cfg *c, const uint16_t *q, const uint8_t *kv_cache,
                              int64_t n_blocks, const int32_t *table_row, int32_t maxb,
                              const uint8_t *swa_ring, int32_t C, int32_t q_pos0, int32_t n_q,
                              const int32_t *topk, const int32_t *topk_len, double *out,
                              double *lse) {
    if (!cfg_ok(c) || n_q < 0 || q_pos0 < 0) return O_BAD;
    size_t qrow = (size_t)c->n_q_heads * c->kv_dim;
    for (int32_t i = 0; i < n_q; i++) {
        int32_t L = q_pos0 + i + 1;
        int st = csa2o_sparse_attn(c, q + i * qrow, kv_cache, n_blocks, table_row, maxb,
                                   swa_ring, C, &L, 1, topk + (int64_t)i * c->topk,
                                   topk_len + i, out + i * qrow,
                                   lse + (size_t)i * c->n_q_heads);
        if (st != O_OK) return st;
    }
    return O_OK;
}
