// csa2_attn.hip -- sparse attention over the selected FP4 main-KV rows plus the FP8
// sliding window, one softmax per (sequence, head).
//
// The pages: Reuse layers only run attention over reused indices, every decoder layer
// keeps a local window (dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心";
// 10100.com/article/150771503, "三招压缩，各有分工"); the window is 128 tokens
// (prism.simon-ai.net/article/7901, "短期记忆的去留：从SSD存储到GPU重算").  The attention
// form itself is this library's reading: K = V = the dequantised 512-d latent (or window
// row), shared by all H_q query heads; logits sm_scale * q.k; selected and window rows are
// not de-duplicated.
//
// Work split: the row list of a sequence is [0, k) = top-k entries (padding masked),
// then [k, k+W) = window positions; workgroup (split, sequence, head group of 16) owns 64
// consecutive rows.
//   1. Each lane loads its slice of the 16 query rows while the row addresses resolve
//      (top-k entry, then block table), so those loads overlap that chain.
//   2. Each lane gathers one row's 128-dim quarter and converts it to bf16 with the
//      gfx950 scaled converters (exact: E2M1 / E4M3 values times a power of two fit
//      bf16).  Those registers are the B operand of S = Q K^T on MFMA 16x16x32 bf16 (fp32
//      accumulation); the same values go to LDS transposed (V^T).
//   3. Softmax statistics per head over the 64 rows (wave shuffles + LDS).
//   4. O = P V on MFMA with P split into bf16 hi + lo parts (error ~2^-17 relative).
//   5. One split per sequence writes the outputs; with several, each writes its partial
//      (O, max, sum) to the workspace and the last split of (sequence, head group) to
//      arrive (an atomic counter) combines them.
#include "csa2_quant.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kD = 512;            // latent dim handled by these kernels
constexpr int kPStride = 64 + 4;   // padded row of the P tile (floats)
constexpr int kMaxSplits = 512;    // splits a merge handles (k + W <= 32768)

struct AttnArgs {
    const uint16_t *q;
    const uint8_t *kv;
    int64_t n_blocks;
    const int32_t *table;
    int32_t maxb;
    int32_t tstride;   // block-table row stride (maxb; 0 when every row is one sequence's)
    const uint8_t *swa;
    int32_t C;
    int32_t rstride;   // ring stride in slots (C; 0 when the rows share one ring)
    const int32_t *ctx_len;  // [B]; NULL: row b is the prefill query at q_pos0 + b
    int32_t q_pos0;
    int32_t B;
    const int32_t *topk;
    const int32_t *topk_len;
    int32_t k;
    int32_t W;
    int32_t Hq;
    int32_t HG;        // head groups of 16
    float scale_log2;  // sm_scale * log2(e)
    float sm_scale;
    int32_t nsplit;
    int32_t cps;       // 64-row chunks per split
    float *part_o;
    float *part_ml;
    int32_t *count;   // [B][HG] arrivals of splits; zero between calls
    float *out;
    float *lse;
    // fused window append (null: none): row swa_new[b] (fp32, D) is quantised into ring
    // slot new_pos[b] % C before it is attended
    const float *swa_new;
    const int32_t *new_pos;
    uint8_t *swa_out;
};

__device__ __forceinline__ int clamp_ctx(int32_t L, int maxb) {
    const int64_t cap = (int64_t)maxb * kBlk;
    return L < 0 ? 0 : (int)(L > cap ? cap : L);
}

// Reductions over the 16 lanes of a DPP row (quad swaps, half-row and row mirrors); every
// lane of the row receives the result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));   // quad [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));   // quad [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
    return fmaxf(x, dpp_f<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    return x + dpp_f<0x140>(x);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &u, int i) {
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

__device__ __forceinline__ bf16x8_t join4(bf16x2_t a, bf16x2_t b, bf16x2_t c, bf16x2_t d) {
    bf16x8_t v;
    v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
    v[4] = c[0]; v[5] = c[1]; v[6] = d[0]; v[7] = d[1];
    return v;
}

// Position in the swizzled V^T tile [512][64] of element (dim d, row r): 8-row chunks are
// XOR-permuted by (d >> 1) & 7 so that 16 lanes reading 16 consecutive d hit all banks.
__device__ __forceinline__ int vt_index(int d, int r) {
    return d * 64 + ((((r >> 3) ^ (d >> 1)) & 7) << 3) + (r & 7);
}

struct AttnShared {
    __bf16 vt[kD * 64];                    // V^T tile (64 KB)
    float ptile[16 * kPStride];
    float red_m[4][16], red_l[4][16];
    __align__(16) uint8_t fresh_row[kD + kD / 32];  // the appended window row (MXFP8)
    int any_valid, has_fresh, last;
};

// Combine the splits of (b, head group hg), run by the last split to finish:
// out = sum_s 2^((m_s - M) c) O_s / sum_s 2^((m_s - M) c) l_s per head, accumulated with a
// running maximum over batches of kMergeBatch splits.  Thread (head h = tid / 16,
// q = tid % 16) owns dims 4q + 64i (i = 0..7) of head h, so 16 threads read one partial row
// in 256-byte runs; a batch's rows and (max, sum) pairs are all loaded before any is used.
// An empty split's row was never written: its values are discarded by a select, which
// keeps the loads unconditional.
constexpr int kMergeBatch = 4;

__device__ __forceinline__ void merge_splits(const AttnArgs &a, int b, int hg) {
    const int tid = threadIdx.x, h = tid >> 4, q = tid & 15;
    const int64_t row0 = (int64_t)b * a.nsplit * a.Hq + hg * 16 + h;  // split 0, head h
    const float4 *src = reinterpret_cast<const float4 *>(a.part_o + row0 * kD) + q;
    const float2 *mlp = reinterpret_cast<const float2 *>(a.part_ml) + row0;
    const int64_t sstride = (int64_t)a.Hq * kD / 4;  // float4s between splits
    float4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float M = -INFINITY, lw = 0.0f;
    for (int s0 = 0; s0 < a.nsplit; s0 += kMergeBatch) {
        float2 st[kMergeBatch];
        float4 v[kMergeBatch][8];
#pragma unroll
        for (int u = 0; u < kMergeBatch; u++) {
            const int sp = min(s0 + u, a.nsplit - 1);
            st[u] = mlp[(int64_t)sp * a.Hq];
#pragma unroll
            for (int i = 0; i < 8; i++) v[u][i] = src[sp * sstride + 16 * i];
        }
        float mu[kMergeBatch], mb = M;
#pragma unroll
        for (int u = 0; u < kMergeBatch; u++) {
            mu[u] = s0 + u < a.nsplit && st[u].y > 0.0f ? st[u].x : -INFINITY;
            mb = fmaxf(mb, mu[u]);
        }
        const float alpha = M == -INFINITY ? 0.0f : exp2f((M - mb) * a.scale_log2);
        lw *= alpha;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            acc[i].x *= alpha;
            acc[i].y *= alpha;
            acc[i].z *= alpha;
            acc[i].w *= alpha;
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; u++) {
            const bool use = mu[u] != -INFINITY;
            const float e = use ? exp2f((mu[u] - mb) * a.scale_log2) : 0.0f;
            lw += use ? e * st[u].y : 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                acc[i].x += use ? e * v[u][i].x : 0.0f;
                acc[i].y += use ? e * v[u][i].y : 0.0f;
                acc[i].z += use ? e * v[u][i].z : 0.0f;
                acc[i].w += use ? e * v[u][i].w : 0.0f;
            }
        }
        M = mb;
    }
    const float inv = lw > 0.0f ? 1.0f / lw : 0.0f;
    float4 *dst = reinterpret_cast<float4 *>(a.out + ((int64_t)b * a.Hq + hg * 16 + h) * kD) + q;
#pragma unroll
    for (int i = 0; i < 8; i++)
        dst[16 * i] = make_float4(acc[i].x * inv, acc[i].y * inv, acc[i].z * inv, acc[i].w * inv);
    if (q == 0)
        a.lse[(int64_t)b * a.Hq + hg * 16 + h] = lw > 0.0f ? a.sm_scale * M + logf(lw) : -INFINITY;
}

__global__ __launch_bounds__(kAttnThreads, 2) void k_attn(AttnArgs a) {
    __shared__ __align__(16) AttnShared sh;

    const int s = blockIdx.x, b = blockIdx.y / a.HG, hg = blockIdx.y % a.HG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g4 = lane >> 4;

    // ---- this lane's query slice (head c16, dims g4*128 ..), the A operand of S = Q K^T;
    //      loaded first so that it overlaps the row-address chain
    bf16x8_t qa[16];
    {
        const bf16x8_t *qh = reinterpret_cast<const bf16x8_t *>(
            a.q + ((int64_t)b * a.Hq + hg * 16 + c16) * kD + g4 * 128);
#pragma unroll
        for (int t = 0; t < 16; t++) qa[t] = qh[t];
    }

    const int L = clamp_ctx(a.ctx_len ? a.ctx_len[b] : a.q_pos0 + b + 1, a.maxb);
    const int tl = max(0, min(a.topk_len[b], a.k));
    const int w0 = max(0, L - a.W), nwin = L - w0;
    const int r_loc = 16 * wave + c16;
    const int np_b = a.swa_new ? a.new_pos[b] : -1;

    // ---- an appended row outside the attended window is still written (split 0, hg 0)
    if (a.swa_new && s == 0 && hg == 0 && np_b >= 0 && !(np_b >= w0 && np_b < L && np_b - w0 < a.W) &&
        tid < kD / 32) {
        uint8_t *dst = a.swa_out + ((int64_t)b * a.rstride + np_b % a.C) * (kD + kD / 32);
        quant_fp8(a.swa_new + (int64_t)b * kD + 32 * tid, dst + 32 * tid, dst + kD + tid);
    }

    // running softmax state of heads 4*g4 + j (j = 0..3): max M (score units), sum l, and
    // the unnormalised output of this wave's 8 column tiles
    float M[4], lsum[4];
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        M[j] = -INFINITY;
        lsum[j] = 0.0f;
    }
#pragma unroll
    for (int n = 0; n < 8; n++) o[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int nchunk = attn_splits(a.k, a.W);
    const int c_end = min(nchunk, (s + 1) * a.cps);
    for (int c = s * a.cps; c < c_end; c++) {
        const int rg = c * kAttnRows + r_loc;
        // ---- locate this lane's row
        const uint8_t *rp = nullptr;
        bool fp8 = false, fresh = false;
        if (rg < a.k) {
            if (rg < tl) {
                const int p = a.topk[(int64_t)b * a.k + rg];
                if (p >= 0 && p < L) {
                    const int64_t phys = a.table[(int64_t)b * a.tstride + p / kBlk];
                    if (phys >= 0 && phys < a.n_blocks)
                        rp = a.kv + phys * (kBlk * (kD / 2 + kD / 32)) + (p % kBlk) * (kD / 2 + kD / 32);
                }
            }
        } else {
            const int wi = rg - a.k;
            if (wi < nwin && wi < a.W) {
                const int p = w0 + wi;
                rp = a.swa + ((int64_t)b * a.rstride + p % a.C) * (kD + kD / 32);
                fp8 = true;
                fresh = p == np_b;  // the appended row: quantised here, not read back
            }
        }
        const bool valid = rp != nullptr;
        if (tid == 0) {
            sh.any_valid = 0;
            sh.has_fresh = 0;
        }
        __syncthreads();  // also: the previous chunk is done with V^T, P and the reductions
        if (valid) sh.any_valid = 1;
        if (fresh) sh.has_fresh = 1;
        __syncthreads();
        if (!sh.any_valid) continue;  // uniform
        if (sh.has_fresh) {
            // the appended row: 16 threads quantise one group each into LDS (and, for the
            // first head group, into the ring); its lanes then read it from LDS
            if (tid < kD / 32) {
                float v[32];
                load_group(a.swa_new + (int64_t)b * kD + 32 * tid, v);
                uint32_t w[8];
                const uint32_t sc = quant_fp8_regs(v, w);
                uint4 *d4 = reinterpret_cast<uint4 *>(sh.fresh_row + 32 * tid);
                d4[0] = make_uint4(w[0], w[1], w[2], w[3]);
                d4[1] = make_uint4(w[4], w[5], w[6], w[7]);
                sh.fresh_row[kD + tid] = (uint8_t)sc;
                if (hg == 0) {
                    uint8_t *dst = a.swa_out + ((int64_t)b * a.rstride + np_b % a.C) * (kD + kD / 32);
                    uint4 *g4p = reinterpret_cast<uint4 *>(dst + 32 * tid);
                    g4p[0] = d4[0];
                    g4p[1] = d4[1];
                    dst[kD + tid] = (uint8_t)sc;
                }
            }
            __syncthreads();
            if (fresh) rp = sh.fresh_row;
        }

        // ---- gather + exact conversion to bf16: kb[t] = dims g4*128 + 8t .. +8 of the row
        bf16x8_t kb[16];
        if (valid && !fp8) {
            const uint4 *src = reinterpret_cast<const uint4 *>(rp + g4 * 64);
            const uint4 u0 = src[0], u1 = src[1], u2 = src[2], u3 = src[3];
            const uint32_t sc4 = *reinterpret_cast<const uint32_t *>(rp + kD / 2 + 4 * g4);
            const uint4 uu[4] = {u0, u1, u2, u3};
#pragma unroll
            for (int t = 0; t < 16; t++) {
                const uint32_t wd = word_of(uu[t >> 2], t & 3);
                const float sc = e8m0_to_f32((sc4 >> (8 * (t >> 2))) & 255u);
                kb[t] = join4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 0),
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 1),
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 2),
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 3));
            }
        } else if (valid) {
            const uint4 *src = reinterpret_cast<const uint4 *>(rp + g4 * 128);
            uint4 uu[8];
#pragma unroll
            for (int i = 0; i < 8; i++) uu[i] = src[i];
            const uint32_t sc4 = *reinterpret_cast<const uint32_t *>(rp + kD + 4 * g4);
#pragma unroll
            for (int t = 0; t < 16; t++) {
                const uint32_t w0d = word_of(uu[t >> 1], 2 * (t & 1)), w1d = word_of(uu[t >> 1], 2 * (t & 1) + 1);
                const float sc = e8m0_to_f32((sc4 >> (8 * (t >> 2))) & 255u);
                kb[t] = join4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0d, sc, false),
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0d, sc, true),
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1d, sc, false),
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1d, sc, true));
            }
        } else {
#pragma unroll
            for (int t = 0; t < 16; t++)
#pragma unroll
                for (int i = 0; i < 8; i++) kb[t][i] = (__bf16)0.0f;
        }

        // ---- V^T into LDS
#pragma unroll
        for (int t = 0; t < 16; t++)
#pragma unroll
            for (int i = 0; i < 8; i++) sh.vt[vt_index(g4 * 128 + 8 * t + i, r_loc)] = kb[t][i];

        // ---- S = Q K^T for this wave's 16 rows and the 16 heads
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 16; t++) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], kb[t], acc, 0, 0, 0);
        // lane holds S[head 4*g4 + j][row c16 of this wave]
        float sv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            sv[j] = valid ? acc[j] : -INFINITY;
            const float m = row16_max(sv[j]);
            if (c16 == 0) sh.red_m[wave][4 * g4 + j] = m;
        }
        __syncthreads();  // V^T and the row maxima are in LDS
        // new running maxima (finite: the chunk has a valid row, so every head has a finite
        // score), rescale factors, probabilities of this lane's row
        float alpha[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int h = 4 * g4 + j;
            const float mc = fmaxf(fmaxf(sh.red_m[0][h], sh.red_m[1][h]), fmaxf(sh.red_m[2][h], sh.red_m[3][h]));
            const float mn = fmaxf(M[j], mc);
            alpha[j] = exp2f((M[j] - mn) * a.scale_log2);  // 0 for the first chunk
            M[j] = mn;
            const float pv = valid ? exp2f((sv[j] - mn) * a.scale_log2) : 0.0f;
            const float l = row16_sum(pv);
            if (c16 == 0) sh.red_l[wave][h] = l;
            sh.ptile[h * kPStride + r_loc] = pv;
        }
        __syncthreads();  // P and the row sums are in LDS
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int h = 4 * g4 + j;
            lsum[j] = lsum[j] * alpha[j] + ((sh.red_l[0][h] + sh.red_l[1][h]) + (sh.red_l[2][h] + sh.red_l[3][h]));
        }

        // ---- O = alpha O + P V for this wave's 8 column tiles (128 dims)
        bf16x8_t ph[2], plo[2];
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            const float4 *pr = reinterpret_cast<const float4 *>(sh.ptile + c16 * kPStride + 32 * ks + 8 * g4);
            const float4 x0 = pr[0], x1 = pr[1];
            const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const __bf16 hi = (__bf16)f[i];
                ph[ks][i] = hi;
                plo[ks][i] = (__bf16)(f[i] - (float)hi);
            }
        }
#pragma unroll
        for (int n = 0; n < 8; n++) {
            const int nt = 8 * wave + n;
            const int d = 16 * nt + c16;
#pragma unroll
            for (int j = 0; j < 4; j++) o[n][j] *= alpha[j];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const int chunk = 4 * ks + g4;
                const bf16x8_t vb = *reinterpret_cast<const bf16x8_t *>(
                    &sh.vt[d * 64 + (((chunk ^ (d >> 1)) & 7) << 3)]);
                o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[ks], vb, o[n], 0, 0, 0);
                o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[ks], vb, o[n], 0, 0, 0);
            }
        }
    }

    // ---- one split: normalised output and log-sum-exp; several: the partial state
    if (a.nsplit == 1) {
#pragma unroll
        for (int n = 0; n < 8; n++) {
            const int d = 16 * (8 * wave + n) + c16;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int h = hg * 16 + 4 * g4 + j;
                a.out[((int64_t)b * a.Hq + h) * kD + d] = lsum[j] > 0.0f ? o[n][j] * (1.0f / lsum[j]) : 0.0f;
            }
        }
        if (wave == 0 && c16 == 0)
#pragma unroll
            for (int j = 0; j < 4; j++)
                a.lse[(int64_t)b * a.Hq + hg * 16 + 4 * g4 + j] =
                    lsum[j] > 0.0f ? a.sm_scale * M[j] + logf(lsum[j]) : -INFINITY;
    } else {
        const int64_t pbase = ((int64_t)b * a.nsplit + s) * a.Hq + hg * 16;
        if (wave == 0 && c16 == 0)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int64_t i = pbase + 4 * g4 + j;
                a.part_ml[2 * i] = lsum[j] > 0.0f ? M[j] : -INFINITY;
                a.part_ml[2 * i + 1] = lsum[j];
            }
        if (lsum[0] > 0.0f || lsum[1] > 0.0f || lsum[2] > 0.0f || lsum[3] > 0.0f) {
            float *po = a.part_o + pbase * kD;
#pragma unroll
            for (int n = 0; n < 8; n++) {
                const int d = 16 * (8 * wave + n) + c16;
#pragma unroll
                for (int j = 0; j < 4; j++) po[(4 * g4 + j) * kD + d] = o[n][j];
            }
        }
        // The last split of (b, hg) to arrive combines them all.  Every wave's stores are
        // ordered before the barrier; thread 0's agent-scope release then publishes them
        // device-wide and its acquire (for the last split) covers the other splits' partials.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        int32_t *cnt = a.count + (int64_t)b * a.HG + hg;
        if (tid == 0)
            sh.last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                      a.nsplit - 1;
        __syncthreads();
        if (!sh.last) return;  // uniform
        merge_splits(a, b, hg);
        if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace csa2

using namespace csa2;

namespace {

int sparse_attn(const csa2_config *c, const float *swa_new, const int32_t *new_pos,
                const uint16_t *q, const uint8_t *kv_cache, int64_t n_blocks,
                const int32_t *block_table, int32_t maxb, const uint8_t *swa_cache,
                uint8_t *swa_out, int32_t C, const int32_t *ctx_len, int32_t q_pos0,
                int32_t batch, const int32_t *topk, const int32_t *topk_len, float *out,
                float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!c || !q || !kv_cache || n_blocks <= 0 || !block_table || maxb <= 0 ||
        batch < 0 || !topk || !topk_len || !out || !lse || !ws || c->topk <= 0 ||
        c->swa_window < 0 || c->n_q_heads <= 0 || c->kv_dim <= 0)
        return CSA2_ERR_INVALID;
    if (c->swa_window > 0 && (!swa_cache || C < c->swa_window)) return CSA2_ERR_INVALID;
    if (swa_new && (!new_pos || !swa_out || C <= 0)) return CSA2_ERR_INVALID;
    if (c->kv_dim != kD || c->n_q_heads % 16 || c->n_q_heads > 128) return CSA2_ERR_UNSUPPORTED;
    if (attn_splits(c->topk, c->swa_window) > kMaxSplits) return CSA2_ERR_UNSUPPORTED;
    const AttnPlan plan = attn_plan(batch, c->n_q_heads, c->topk, c->swa_window);
    const int nsplit = plan.nsplit;
    const WsAttn wl = ws_attn(batch, c->n_q_heads, c->kv_dim, nsplit);
    if (ws_bytes < wl.total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    AttnArgs a{};
    a.q = q;
    a.kv = kv_cache;
    a.n_blocks = n_blocks;
    a.table = block_table;
    a.maxb = maxb;
    a.tstride = ctx_len ? maxb : 0;
    a.swa = swa_cache;
    a.C = C > 0 ? C : 1;
    a.rstride = ctx_len ? a.C : 0;
    a.ctx_len = ctx_len;
    a.q_pos0 = q_pos0;
    a.B = batch;
    a.topk = topk;
    a.topk_len = topk_len;
    a.k = c->topk;
    a.W = c->swa_window;
    a.Hq = c->n_q_heads;
    a.HG = c->n_q_heads / 16;
    a.sm_scale = c->sm_scale;
    a.scale_log2 = c->sm_scale * 1.4426950408889634f;
    a.nsplit = nsplit;
    a.cps = plan.cps;
    a.part_o = (float *)((uint8_t *)ws + wl.part_o);
    a.part_ml = (float *)((uint8_t *)ws + wl.part_ml);
    a.count = (int32_t *)((uint8_t *)ws + wl.count);
    a.out = out;
    a.lse = lse;
    a.swa_new = swa_new;
    a.new_pos = new_pos;
    a.swa_out = swa_out;
    k_attn<<<dim3(nsplit, batch * a.HG), kAttnThreads, 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

}  // namespace

extern "C" int csa2_sparse_attn(const csa2_config *c, const uint16_t *q, const uint8_t *kv_cache,
                                int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                                const uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                                int32_t batch, const int32_t *topk, const int32_t *topk_len,
                                float *out, float *lse, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
    if (!ctx_len) return CSA2_ERR_INVALID;
    return sparse_attn(c, nullptr, nullptr, q, kv_cache, n_blocks, block_table, maxb, swa_cache,
                       nullptr, C, ctx_len, 0, batch, topk, topk_len, out, lse, ws, ws_bytes,
                       stream);
}

extern "C" int csa2_sparse_attn_prefill(const csa2_config *c, const uint16_t *q,
                                        const uint8_t *kv_cache, int64_t n_blocks,
                                        const int32_t *block_table, int32_t maxb,
                                        const uint8_t *swa_ring, int32_t C, int32_t q_pos0,
                                        int32_t n_q, const int32_t *topk,
                                        const int32_t *topk_len, float *out, float *lse,
                                        void *ws, size_t ws_bytes, hipStream_t stream) {
    if (q_pos0 < 0 || n_q < 0 || (int64_t)q_pos0 + n_q > (int64_t)maxb * kBlk)
        return CSA2_ERR_INVALID;
    return sparse_attn(c, nullptr, nullptr, q, kv_cache, n_blocks, block_table, maxb, swa_ring,
                       nullptr, C, nullptr, q_pos0, n_q, topk, topk_len, out, lse, ws, ws_bytes,
                       stream);
}

extern "C" int csa2_sparse_attn_append(const csa2_config *c, const float *swa_rows,
                                       const int32_t *pos, const uint16_t *q,
                                       const uint8_t *kv_cache, int64_t n_blocks,
                                       const int32_t *block_table, int32_t maxb,
                                       uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                                       int32_t batch, const int32_t *topk,
                                       const int32_t *topk_len, float *out, float *lse, void *ws,
                                       size_t ws_bytes, hipStream_t stream) {
    if (!swa_rows || !pos || !swa_cache || !ctx_len) return CSA2_ERR_INVALID;
    return sparse_attn(c, swa_rows, pos, q, kv_cache, n_blocks, block_table, maxb, swa_cache,
                       swa_cache, C, ctx_len, 0, batch, topk, topk_len, out, lse, ws, ws_bytes,
                       stream);
}
