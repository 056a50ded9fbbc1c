// csa2_index.hip -- hierarchical sparse indexer of the CSA2 decode step.
//
// What runs (dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心"; and
// prism.simon-ai.net/article/7901, "层级稀疏索引器：精准筛选关键信息"): a Full layer scores
// every visible position with FP4 indexer keys, reduces the scores to 8-position blocks,
// keeps a pool of the K_blk best blocks, then the k best positions inside the pool; a
// Reindex layer rescores only the pool.
//
// Kernels of one Full call (all asynchronous on the caller's stream):
//   k_scan         HBM stream over every visible key: exact FP4 dot products (gfx950
//                  scaled FP4->f16 converts + v_dot2_f32_f16), fixed-order fp32 score,
//                  block max, 12-bit radix histogram of the block keys in LDS; the last
//                  workgroup of each sequence turns the histogram into the pool threshold
//                  and clears the histogram for the next call
//   k_pool_filter  blocks above the threshold digit -> selected list, at it -> candidates
//   k_pool_final   one workgroup per sequence: exact radix select among the candidates,
//                  bitonic sort -> ascending pool
//   k_rescore      scores of the <= 8*K_blk pool positions (shared with Reindex)
//   k_select_topk  one workgroup per sequence: exact radix select, ordered compaction
//
// Score (this library's definition; the pages give none): s(p) = sum_h w_h ReLU(q_h.k_{p,h})
// in a fixed fp32 order.  Per 32-group the dot of the unscaled E2M1 values is exact in
// fp32 (products are multiples of 1/4, |sum| <= 1152), so v_dot2_f32_f16 accumulates it
// exactly in any order; t_j = dot * 2^(E_j) is exact; the group sum, ReLU and the fma chain
// over heads then follow one fixed order, so the result is bit-reproducible.
#include <algorithm>

#include "csa2_common.h"

namespace csa2 {

constexpr int kScanThreads = 256;
constexpr int kChunkBlocks = 32;  // blocks per scan work unit

// ------------------------------------------------------------------ query + score core

__device__ __forceinline__ void cvt_fp4x8_f16(uint32_t w, half2_t *o) {
    o[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    o[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    o[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    o[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
}

template <int H, int G>
struct Query {
    half2_t q[G * 16];  // this lane's head: unscaled E2M1 value pairs of every group
    int e[G];           // unbiased scale exponents of those groups
    float w[H];         // head weights
};

template <int H, int G>
__device__ __forceinline__ void load_query(Query<H, G> &Q, const uint8_t *qc, const uint8_t *qs,
                                           const float *w, int h) {
    const uint4 *c4 = reinterpret_cast<const uint4 *>(qc + h * 16 * G);
#pragma unroll
    for (int g = 0; g < G; g++) {
        const uint4 c = c4[g];
        cvt_fp4x8_f16(c.x, Q.q + 16 * g + 0);
        cvt_fp4x8_f16(c.y, Q.q + 16 * g + 4);
        cvt_fp4x8_f16(c.z, Q.q + 16 * g + 8);
        cvt_fp4x8_f16(c.w, Q.q + 16 * g + 12);
        Q.e[g] = (int)qs[h * G + g] - 127;
    }
#pragma unroll
    for (int j = 0; j < H; j++) Q.w[j] = w[j];
}

// Exact dot of one 32-group (returns N/4 where N is the dot of doubled codes).
__device__ __forceinline__ float group_dot(const half2_t *q, uint4 c) {
    half2_t k[16];
    cvt_fp4x8_f16(c.x, k + 0);
    cvt_fp4x8_f16(c.y, k + 4);
    cvt_fp4x8_f16(c.z, k + 8);
    cvt_fp4x8_f16(c.w, k + 12);
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a0 = __builtin_amdgcn_fdot2(q[i], k[i], a0, false);
        a1 = __builtin_amdgcn_fdot2(q[8 + i], k[8 + i], a1, false);
    }
    return a0 + a1;  // both partials are exact multiples of 1/4 below 2^11: exact
}

template <int G>
__device__ __forceinline__ uint32_t load_scales(const uint8_t *p) {
    if constexpr (G == 1) return *p;
    else if constexpr (G == 2) return *reinterpret_cast<const uint16_t *>(p);
    else return *reinterpret_cast<const uint32_t *>(p);
}

// r_h = ReLU(D_h) for one (position, head): groups summed in order in fp32.
template <int H, int G>
__device__ __forceinline__ float head_relu(const Query<H, G> &Q, const uint4 (&kc)[G], uint32_t ks) {
    float D = 0.0f;
#pragma unroll
    for (int g = 0; g < G; g++) {
        const float acc = group_dot(Q.q + 16 * g, kc[g]);
        const int E = Q.e[g] + (int)((ks >> (8 * g)) & 255u) - 127;
        D = D + ldexpf(acc, E);
    }
    return D > 0.0f ? D : 0.0f;
}

// s = fma(w_{H-1}, r_{H-1}, ... fma(w_0, r_0, +0)); the H lanes of a position hold r_0..r_{H-1}.
template <int H, int G>
__device__ __forceinline__ float combine_heads(const Query<H, G> &Q, float r, int lane) {
    const int base = lane - (lane % H);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < H; j++) s = __builtin_fmaf(Q.w[j], __shfl(r, base + j, kWave), s);
    return s;
}

// Geometry of one indexer-key block as seen by a wave: 8 positions x H heads per block,
// 8/H blocks per wave; lane = (position in wave) * H + head.
template <int H, int G>
struct KeyBlock {
    static constexpr int BPW = 8 / H;             // blocks per wave step
    static constexpr int BPS = BPW * (kScanThreads / kWave);  // blocks per workgroup step
    static constexpr int CODES = kBlk * H * 16 * G;
    static constexpr int BYTES = CODES + kBlk * H * G;
};

template <int H, int G>
__device__ __forceinline__ float block_position_relu(const uint8_t *bp, int slot, int h,
                                                     const Query<H, G> &Q) {
    uint4 kc[G];
#pragma unroll
    for (int g = 0; g < G; g++)
        kc[g] = *reinterpret_cast<const uint4 *>(bp + ((g * kBlk + slot) * H + h) * 16);
    const uint32_t ks = load_scales<G>(bp + KeyBlock<H, G>::CODES + (slot * H + h) * G);
    return head_relu<H, G>(Q, kc, ks);
}

// ------------------------------------------------------------------ block-level helpers

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) t += sh[i];
    return t;
}

// Exclusive scan over the threads of the block (thread order), returns total via *tot.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh, uint32_t *tot) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == kWave - 1) sh[wave] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) {
        const uint32_t x = sh[i];
        before += (i < wave) ? x : 0u;
        all += x;
    }
    *tot = all;
    return before + incl - v;
}

template <int NT>
__device__ __forceinline__ void block_and_or(uint64_t &va, uint64_t &vo, uint64_t *sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        va &= __shfl_xor(va, o, kWave);
        vo |= __shfl_xor(vo, o, kWave);
    }
    __syncthreads();
    if (lane == 0) {
        sh[2 * wave] = va;
        sh[2 * wave + 1] = vo;
    }
    __syncthreads();
    va = ~0ull;
    vo = 0ull;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) {
        va &= sh[2 * i];
        vo |= sh[2 * i + 1];
    }
}

// ------------------------------------------------------------------ exact block-wide select
//
// Selects the `need` largest of a set of distinct 64-bit keys (score key << 32 | ~index, so
// ties in score go to the lower index).  Radix select with 8-bit digits over LDS
// histograms, starting at the first bit where the keys differ.  On return an item is
// selected iff (key >> shift) >= prefix.  `src.each(f)` calls f(key) for every item the
// calling thread owns.

template <int NT>
struct SelShared {
    uint32_t hist[256];
    uint64_t red[2 * (NT / kWave)];
    uint32_t chosen, above, count;
};

template <int NT, class Src>
__device__ void block_select(const Src &src, uint32_t need, SelShared<NT> &sh, uint64_t &prefix_out,
                             int &shift_out) {
    uint64_t va = ~0ull, vo = 0ull;
    src.each([&](uint64_t c) {
        va &= c;
        vo |= c;
    });
    block_and_or<NT>(va, vo, sh.red);
    const uint64_t diff = va ^ vo;
    if (diff == 0) {  // at most one distinct key
        prefix_out = va;
        shift_out = 0;
        return;
    }
    int shift = ((63 - __clzll((long long)diff)) / 8) * 8;
    uint64_t prefix = (shift + 8 >= 64) ? 0ull : (va >> (shift + 8));
    uint32_t remaining = need;
    const int tid = threadIdx.x;
    while (true) {
        for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
        __syncthreads();
        src.each([&](uint64_t c) {
            if (shift + 8 >= 64 || (c >> (shift + 8)) == prefix)
                atomicAdd(&sh.hist[(uint32_t)(c >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (tid < kWave) {
            const int l = tid;
            const uint32_t c0 = sh.hist[255 - 4 * l], c1 = sh.hist[254 - 4 * l],
                           c2 = sh.hist[253 - 4 * l], c3 = sh.hist[252 - 4 * l];
            const uint32_t tot = c0 + c1 + c2 + c3;
            const uint32_t incl = wave_incl_scan(tot);
            const uint32_t excl = incl - tot;
            if (excl < remaining && remaining <= incl) {
                uint32_t cum = excl, d = 255 - 4 * l, cnt = c0;
                if (cum + c0 < remaining) {
                    cum += c0; d -= 1; cnt = c1;
                    if (cum + c1 < remaining) {
                        cum += c1; d -= 1; cnt = c2;
                        if (cum + c2 < remaining) {
                            cum += c2; d -= 1; cnt = c3;
                        }
                    }
                }
                sh.chosen = d;
                sh.above = cum;
                sh.count = cnt;
            }
        }
        __syncthreads();
        const uint32_t d = sh.chosen, above = sh.above, cnt = sh.count;
        __syncthreads();  // everyone has read before the next pass rewrites
        prefix = (prefix << 8) | d;
        remaining -= above;
        if (cnt == remaining || shift == 0) break;
        shift -= 8;
    }
    prefix_out = prefix;
    shift_out = shift;
}

// ------------------------------------------------------------------ kernel arguments

struct IndexArgs {
    const uint8_t *q_codes;
    const uint8_t *q_scales;
    const float *w;
    const uint8_t *idx_cache;
    int64_t n_blocks;
    const int32_t *table;
    int32_t maxb;
    int32_t B;
    int32_t K_blk;
    int32_t k;
    const int32_t *ctx_len;
    SeqState *st;
    uint32_t *hist;
    float *bscore;
    int32_t *sel;
    uint2 *cand;
    float *pscore;
    float *scores_out;        // inspection only
    float *block_scores_out;  // inspection only
    const int32_t *pool_blocks;
    const int32_t *pool_len;
};

__device__ __forceinline__ int clamp_len(int32_t L, int maxb) {
    const int64_t cap = (int64_t)maxb * kBlk;
    return L < 0 ? 0 : (int)(L > cap ? cap : L);
}

// Work list of the scan: sequence b owns chunks [prefix[b], prefix[b+1]) of kChunkBlocks
// blocks.  Every scan workgroup rebuilds it in LDS from ctx_len (B <= kMaxBatch).
__device__ int build_chunk_prefix(const IndexArgs &a, int32_t *prefix, uint32_t *sh_scan) {
    uint32_t running = 0;
    for (int base = 0; base < a.B; base += kScanThreads) {
        const int b = base + (int)threadIdx.x;
        uint32_t v = 0;
        if (b < a.B) {
            const int nb = (clamp_len(a.ctx_len[b], a.maxb) + kBlk - 1) / kBlk;
            v = (uint32_t)((nb + kChunkBlocks - 1) / kChunkBlocks);
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan<kScanThreads>(v, sh_scan, &tot);
        if (b < a.B) prefix[b] = (int32_t)(running + ex);
        running += tot;
    }
    if (threadIdx.x == 0) prefix[a.B] = (int32_t)running;
    __syncthreads();
    return (int)running;
}

// ------------------------------------------------------------------ k_scan

__device__ __forceinline__ int seq_of_chunk(const int32_t *prefix, int B, int c) {
    int lo = 0, hi = B - 1;  // largest b with prefix[b] <= c
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The pool threshold of sequence b from its complete histogram: the digit d such that
// fewer than K_blk blocks have a larger digit and at least K_blk have d or larger (-1 when
// every block fits in the pool).  Then clears the histogram and the chunk counter.
__device__ void pool_threshold(const IndexArgs &a, int b, int nb, uint32_t *sh_scan) {
    SeqState *S = a.st + b;
    const int K = a.K_blk, tid = threadIdx.x;
    uint32_t *gh = a.hist + (size_t)b * kHistBins;
    if (nb <= K) {
        if (tid == 0) {
            S->thr = -1;
            S->above = 0;
        }
    } else {
        uint32_t cnt[16], tsum = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            cnt[i] = load_coherent(gh + (kHistBins - 1 - 16 * tid - i));
            tsum += cnt[i];
        }
        uint32_t tot;
        const uint32_t excl = block_excl_scan<kScanThreads>(tsum, sh_scan, &tot);
        const uint32_t incl = excl + tsum;
        if (excl < (uint32_t)K && (uint32_t)K <= incl) {
            uint32_t cum = excl;
            for (int i = 0; i < 16; i++) {
                if (cum + cnt[i] >= (uint32_t)K) {
                    S->thr = kHistBins - 1 - 16 * tid - i;
                    S->above = (int)cum;
                    break;
                }
                cum += cnt[i];
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < kHistBins; i += kScanThreads) gh[i] = 0;
    if (tid == 0) S->done = 0;
}

// FULL: block scores + histogram + pool threshold.  Otherwise: inspection outputs only.
template <int H, int G, bool FULL>
__global__ __launch_bounds__(kScanThreads) void k_scan(IndexArgs a) {
    using KB = KeyBlock<H, G>;
    __shared__ uint32_t sh_hist[FULL ? kHistBins : 1];
    __shared__ int32_t sh_prefix[kMaxBatch + 1];
    __shared__ uint32_t sh_scan[kScanThreads / kWave];
    __shared__ int sh_last;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int h = lane % H, pw = lane / H, bw = pw / kBlk, slot = pw % kBlk;
    const int total = build_chunk_prefix(a, sh_prefix, sh_scan);
    const int per = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    const int c0 = (int)blockIdx.x * per, c1 = min(total, c0 + per);
    if (c0 >= c1) return;
    if (FULL) {
        for (int i = tid; i < kHistBins; i += kScanThreads) sh_hist[i] = 0;
    }
    Query<H, G> Q;
    int cur = -1, credits = 0, L = 0, nb = 0;
    const int32_t *trow = nullptr;

    auto flush = [&](int b) {
        __syncthreads();
        uint32_t *gh = a.hist + (size_t)b * kHistBins;
        for (int i = tid; i < kHistBins; i += kScanThreads) {
            const uint32_t v = sh_hist[i];
            if (v) {
                atomicAdd(gh + i, v);
                sh_hist[i] = 0;
            }
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const int nch = sh_prefix[b + 1] - sh_prefix[b];
            const int old = atomicAdd(&a.st[b].done, credits);
            sh_last = (old + credits == nch);
        }
        __syncthreads();
        if (sh_last) {
            __threadfence();
            pool_threshold(a, b, nb, sh_scan);
        }
        __syncthreads();
    };

    for (int c = c0; c < c1; c++) {
        const int b = seq_of_chunk(sh_prefix, a.B, c);
        if (b != cur) {
            if (FULL && cur >= 0) flush(cur);
            cur = b;
            credits = 0;
            L = clamp_len(a.ctx_len[b], a.maxb);
            nb = (L + kBlk - 1) / kBlk;
            load_query<H, G>(Q, a.q_codes + (size_t)b * H * 16 * G, a.q_scales + (size_t)b * H * G,
                             a.w + (size_t)b * H, h);
            trow = a.table + (int64_t)b * a.maxb;
        }
        const int cb0 = (c - sh_prefix[b]) * kChunkBlocks;
        const int cb1 = min(nb, cb0 + kChunkBlocks);
        for (int base = cb0; base < cb1; base += KB::BPS) {
            const int blk = base + wave * KB::BPW + bw;
            const bool active = blk < cb1;
            float r = 0.0f;
            bool vis = false;
            if (active) {
                const int64_t phys = trow[blk];
                if (phys >= 0 && phys < a.n_blocks) {
                    r = block_position_relu<H, G>(a.idx_cache + phys * KB::BYTES, slot, h, Q);
                    vis = blk * kBlk + slot < L;
                }
            }
            const float s = combine_heads<H, G>(Q, r, lane);
            float m = vis ? s : -INFINITY;
            m = fmaxf(m, __shfl_xor(m, H, kWave));
            m = fmaxf(m, __shfl_xor(m, 2 * H, kWave));
            m = fmaxf(m, __shfl_xor(m, 4 * H, kWave));
            if (!FULL && a.scores_out && vis && h == 0)
                a.scores_out[(int64_t)b * a.maxb * kBlk + (int64_t)blk * kBlk + slot] = s;
            if (active && slot == 0 && h == 0) {
                if (FULL) {
                    a.bscore[(int64_t)b * a.maxb + blk] = m;
                    atomicAdd(&sh_hist[order_key(m) >> (32 - kHistBits)], 1u);
                } else if (a.block_scores_out) {
                    a.block_scores_out[(int64_t)b * a.maxb + blk] = m;
                }
            }
        }
        credits++;
    }
    if (FULL && cur >= 0) flush(cur);
}

// ------------------------------------------------------------------ k_pool_filter

__global__ __launch_bounds__(256) void k_pool_filter(IndexArgs a) {
    const int b = blockIdx.y, tid = threadIdx.x, lane = lane_id();
    SeqState *S = a.st + b;
    const int nb = (clamp_len(a.ctx_len[b], a.maxb) + kBlk - 1) / kBlk;
    const int j0 = blockIdx.x * 1024;
    if (j0 >= nb) return;
    const int thr = S->thr;
    for (int i = 0; i < 4; i++) {
        const int j = j0 + i * 256 + tid;
        const bool valid = j < nb;
        const uint32_t key = valid ? order_key(a.bscore[(int64_t)b * a.maxb + j]) : 0u;
        const int d = (int)(key >> (32 - kHistBits));
        const bool is_sel = valid && d > thr, is_cand = valid && d == thr;
        const uint64_t ms = ballot(is_sel), mc = ballot(is_cand);
        if (ms) {
            const int leader = __ffsll((long long)ms) - 1;
            int base = 0;
            if (lane == leader) base = atomicAdd(&S->n_sel, (int)__popcll(ms));
            base = __shfl(base, leader, kWave);
            const int off = base + (int)lanes_below(ms);
            if (is_sel && off < a.K_blk) a.sel[(int64_t)b * a.K_blk + off] = j;
        }
        if (mc) {
            const int leader = __ffsll((long long)mc) - 1;
            int base = 0;
            if (lane == leader) base = atomicAdd(&S->n_cand, (int)__popcll(mc));
            base = __shfl(base, leader, kWave);
            const int off = base + (int)lanes_below(mc);
            if (is_cand && off < a.maxb) a.cand[(int64_t)b * a.maxb + off] = make_uint2(key, (uint32_t)j);
        }
    }
}

// ------------------------------------------------------------------ k_pool_final

constexpr int kFinalThreads = 1024;
constexpr int kCandPerThread = 8;

struct CandRegs {
    uint64_t c[kCandPerThread];
    uint32_t valid;  // bit i: item i holds a candidate
    template <class F>
    __device__ void each(F f) const {
#pragma unroll
        for (int i = 0; i < kCandPerThread; i++)
            if (valid & (1u << i)) f(c[i]);
    }
};

struct CandGlobal {
    const uint2 *p;
    int n;
    template <class F>
    __device__ void each(F f) const {
        for (int i = threadIdx.x; i < n; i += kFinalThreads) {
            const uint2 v = p[i];
            f(((uint64_t)v.x << 32) | (uint64_t)(0xFFFFFFFFu - v.y));
        }
    }
};

__device__ __forceinline__ void bitonic_sort_lds(int32_t *v, int n_pow2) {
    for (int k = 2; k <= n_pow2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n_pow2 / 2; i += blockDim.x) {
                const int lo = 2 * i - (i & (j - 1));
                const int hi = lo + j;
                const bool up = ((lo & k) == 0);
                const int32_t x = v[lo], y = v[hi];
                if ((x > y) == up) {
                    v[lo] = y;
                    v[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(kFinalThreads) void k_pool_final(IndexArgs a, int32_t *pool_blocks,
                                                              int32_t *pool_len) {
    __shared__ int32_t out[CSA2_MAX_POOL_BLOCKS];
    __shared__ int out_n;
    __shared__ SelShared<kFinalThreads> sh;
    const int b = blockIdx.x, tid = threadIdx.x;
    const SeqState S = a.st[b];
    const int K = a.K_blk;
    const int nb = (clamp_len(a.ctx_len[b], a.maxb) + kBlk - 1) / kBlk;
    const int Kp = min(K, nb);
    const int n_sel = min(S.n_sel, Kp);
    const int n_cand = min(S.n_cand, a.maxb);
    const int need = Kp - n_sel;
    for (int i = tid; i < n_sel; i += kFinalThreads) out[i] = a.sel[(int64_t)b * K + i];
    if (tid == 0) out_n = n_sel;
    __syncthreads();
    const uint2 *cp = a.cand + (int64_t)b * a.maxb;
    if (need > 0 && need >= n_cand) {
        for (int i = tid; i < n_cand; i += kFinalThreads) out[n_sel + i] = (int32_t)cp[i].y;
    } else if (need > 0 && n_cand <= kFinalThreads * kCandPerThread) {
        CandRegs src;
        src.valid = 0;
#pragma unroll
        for (int i = 0; i < kCandPerThread; i++) {
            const int idx = tid + i * kFinalThreads;
            uint2 v = make_uint2(0u, 0u);
            if (idx < n_cand) {
                v = cp[idx];
                src.valid |= 1u << i;
            }
            src.c[i] = ((uint64_t)v.x << 32) | (uint64_t)(0xFFFFFFFFu - v.y);
        }
        uint64_t prefix;
        int shift;
        block_select<kFinalThreads>(src, (uint32_t)need, sh, prefix, shift);
        src.each([&](uint64_t c) {
            if ((c >> shift) >= prefix) {
                const int o = atomicAdd(&out_n, 1);
                if (o < Kp) out[o] = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
            }
        });
    } else if (need > 0) {
        CandGlobal src{cp, n_cand};
        uint64_t prefix;
        int shift;
        block_select<kFinalThreads>(src, (uint32_t)need, sh, prefix, shift);
        src.each([&](uint64_t c) {
            if ((c >> shift) >= prefix) {
                const int o = atomicAdd(&out_n, 1);
                if (o < Kp) out[o] = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
            }
        });
    }
    __syncthreads();
    int np2 = 1;
    while (np2 < Kp) np2 <<= 1;
    for (int i = Kp + tid; i < np2; i += kFinalThreads) out[i] = 0x7FFFFFFF;
    __syncthreads();
    bitonic_sort_lds(out, np2);
    for (int i = tid; i < K; i += kFinalThreads)
        pool_blocks[(int64_t)b * K + i] = i < Kp ? out[i] : -1;
    if (tid == 0) {
        pool_len[b] = Kp;
        a.st[b].n_sel = 0;  // leave the workspace counters cleared
        a.st[b].n_cand = 0;
    }
}

// ------------------------------------------------------------------ k_rescore

constexpr int kRescoreBlocks = 16;  // pool entries per workgroup (at least one step)

template <int H, int G>
__global__ __launch_bounds__(kScanThreads) void k_rescore(IndexArgs a) {
    using KB = KeyBlock<H, G>;
    constexpr int RB = kRescoreBlocks > KB::BPS ? kRescoreBlocks : KB::BPS;
    const int b = blockIdx.y, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int h = lane % H, pw = lane / H, bw = pw / kBlk, slot = pw % kBlk;
    const int plen = max(0, min(a.pool_len[b], a.K_blk));
    const int e0 = blockIdx.x * RB, e1 = min(plen, e0 + RB);
    if (e0 >= e1) return;
    const int L = clamp_len(a.ctx_len[b], a.maxb), nb = (L + kBlk - 1) / kBlk;
    Query<H, G> Q;
    load_query<H, G>(Q, a.q_codes + (size_t)b * H * 16 * G, a.q_scales + (size_t)b * H * G,
                     a.w + (size_t)b * H, h);
    const int32_t *trow = a.table + (int64_t)b * a.maxb;
    const int32_t *pool = a.pool_blocks + (int64_t)b * a.K_blk;
    for (int base = e0; base < e1; base += KB::BPS) {
        const int e = base + wave * KB::BPW + bw;
        const bool active = e < e1;
        float r = 0.0f;
        bool vis = false;
        if (active) {
            const int j = pool[e];
            if (j >= 0 && j < nb) {
                const int64_t phys = trow[j];
                if (phys >= 0 && phys < a.n_blocks) {
                    r = block_position_relu<H, G>(a.idx_cache + phys * KB::BYTES, slot, h, Q);
                    vis = j * kBlk + slot < L;
                }
            }
        }
        const float s = combine_heads<H, G>(Q, r, lane);
        if (active && h == 0)
            a.pscore[((int64_t)b * a.K_blk + e) * kBlk + slot] = vis ? s : -INFINITY;
    }
}

// ------------------------------------------------------------------ k_select_topk

constexpr int kSelItems = 16;  // pool slots per thread (1024 * 16 = 8 * 2048)

struct SlotRegs {
    uint64_t c[kSelItems];
    uint32_t valid;  // bit i: item i is a visible candidate
    template <class F>
    __device__ void each(F f) const {
#pragma unroll
        for (int i = 0; i < kSelItems; i++)
            if (valid & (1u << i)) f(c[i]);
    }
};

__global__ __launch_bounds__(kFinalThreads) void k_select_topk(IndexArgs a, int32_t *topk,
                                                               int32_t *topk_len) {
    __shared__ SelShared<kFinalThreads> sh;
    __shared__ uint32_t sh_scan[kFinalThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int plen = max(0, min(a.pool_len[b], a.K_blk));
    const int n = plen * kBlk;
    const int s0 = tid * kSelItems;
    const float *ps = a.pscore + (int64_t)b * a.K_blk * kBlk;
    SlotRegs src;
    src.valid = 0;
#pragma unroll
    for (int i = 0; i < kSelItems; i += 4) {
        float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (s0 + i < n) v = *reinterpret_cast<const float4 *>(ps + s0 + i);
        const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int slot = s0 + i + t;
            const bool ok = slot < n && f[t] != -INFINITY;
            src.c[i + t] = ((uint64_t)order_key(f[t]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)slot);
            if (ok) src.valid |= 1u << (i + t);
        }
    }
    const uint32_t n_valid = block_sum<kFinalThreads>((uint32_t)__popc(src.valid), sh_scan);
    const uint32_t need = min((uint32_t)a.k, n_valid);
    uint32_t selmask = 0;
    if (need == n_valid) {
        selmask = src.valid;
    } else if (need > 0) {
        uint64_t prefix;
        int shift;
        block_select<kFinalThreads>(src, need, sh, prefix, shift);
#pragma unroll
        for (int i = 0; i < kSelItems; i++)
            if ((src.valid & (1u << i)) && (src.c[i] >> shift) >= prefix) selmask |= 1u << i;
    }
    uint32_t tot;
    const uint32_t off = block_excl_scan<kFinalThreads>((uint32_t)__popc(selmask), sh_scan, &tot);
    const int32_t *pool = a.pool_blocks + (int64_t)b * a.K_blk;
    int32_t *out = topk + (int64_t)b * a.k;
    uint32_t o = off;
#pragma unroll
    for (int i = 0; i < kSelItems; i++) {
        if (selmask & (1u << i)) {
            const int slot = s0 + i;
            if (o < (uint32_t)a.k) out[o] = pool[slot / kBlk] * kBlk + slot % kBlk;
            o++;
        }
    }
    for (int i = (int)need + tid; i < a.k; i += kFinalThreads) out[i] = -1;
    if (tid == 0) topk_len[b] = (int32_t)need;
}

// ------------------------------------------------------------------ dispatch

template <int H, int G>
struct Kern {
    static void scan_full(dim3 g, hipStream_t s, const IndexArgs &a) {
        k_scan<H, G, true><<<g, kScanThreads, 0, s>>>(a);
    }
    static void scan_inspect(dim3 g, hipStream_t s, const IndexArgs &a) {
        k_scan<H, G, false><<<g, kScanThreads, 0, s>>>(a);
    }
    static void rescore(dim3 g, hipStream_t s, const IndexArgs &a) {
        k_rescore<H, G><<<g, kScanThreads, 0, s>>>(a);
    }
    static int rescore_blocks() {
        return kRescoreBlocks > KeyBlock<H, G>::BPS ? kRescoreBlocks : KeyBlock<H, G>::BPS;
    }
};

typedef void (*LaunchFn)(dim3, hipStream_t, const IndexArgs &);
struct KernSet {
    LaunchFn scan_full, scan_inspect, rescore;
    int rescore_blocks;
};

template <int H, int G>
KernSet kern_set() {
    return {Kern<H, G>::scan_full, Kern<H, G>::scan_inspect, Kern<H, G>::rescore,
            Kern<H, G>::rescore_blocks()};
}

bool pick(int H, int dI, KernSet *ks) {
    const int G = dI / 32;
#define CSA2_CASE(h, g) \
    if (H == h && G == g) { *ks = kern_set<h, g>(); return true; }
    CSA2_CASE(1, 1) CSA2_CASE(1, 2) CSA2_CASE(1, 4)
    CSA2_CASE(2, 1) CSA2_CASE(2, 2) CSA2_CASE(2, 4)
    CSA2_CASE(4, 1) CSA2_CASE(4, 2) CSA2_CASE(4, 4)
    CSA2_CASE(8, 1) CSA2_CASE(8, 2) CSA2_CASE(8, 4)
#undef CSA2_CASE
    return false;
}

}  // namespace csa2

using namespace csa2;

namespace {

int check_cfg(const csa2_config *c) {
    if (!c) return CSA2_ERR_INVALID;
    if (c->n_idx_heads <= 0 || c->idx_dim <= 0 || c->idx_dim % 32 || c->kv_dim <= 0 ||
        c->kv_dim % 32 || c->n_q_heads <= 0 || c->swa_window < 0 || c->pool_blocks <= 0 ||
        c->topk <= 0 || (int64_t)c->topk > 8 * (int64_t)c->pool_blocks)
        return CSA2_ERR_INVALID;
    if (c->pool_blocks > CSA2_MAX_POOL_BLOCKS) return CSA2_ERR_UNSUPPORTED;
    KernSet ks;
    if (!pick(c->n_idx_heads, c->idx_dim, &ks)) return CSA2_ERR_UNSUPPORTED;
    return CSA2_OK;
}

int launched() { return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

IndexArgs make_args(const csa2_config *c, const uint8_t *qc, const uint8_t *qs, const float *w,
                    const uint8_t *idx, int64_t n_blocks, const int32_t *table, int32_t maxb,
                    const int32_t *ctx, int32_t B, void *ws) {
    const WsIndex L = ws_index(B, maxb, c->pool_blocks);
    uint8_t *base = (uint8_t *)ws;
    IndexArgs a{};
    a.q_codes = qc;
    a.q_scales = qs;
    a.w = w;
    a.idx_cache = idx;
    a.n_blocks = n_blocks;
    a.table = table;
    a.maxb = maxb;
    a.B = B;
    a.K_blk = c->pool_blocks;
    a.k = c->topk;
    a.ctx_len = ctx;
    a.st = (SeqState *)(base + L.st);
    a.hist = (uint32_t *)(base + L.hist);
    a.bscore = (float *)(base + L.bscore);
    a.sel = (int32_t *)(base + L.sel);
    a.cand = (uint2 *)(base + L.cand);
    a.pscore = (float *)(base + L.pscore);
    return a;
}

int scan_grid(int B, int maxb) {
    const int64_t chunks = (int64_t)B * ((maxb + kChunkBlocks - 1) / kChunkBlocks);
    return (int)std::max<int64_t>(1, std::min<int64_t>(chunks, 2048));
}

}  // namespace

extern "C" int csa2_layout(const csa2_config *c, csa2_layout_info *out) {
    if (!c || !out || c->n_idx_heads <= 0 || c->idx_dim <= 0 || c->idx_dim % 32 ||
        c->kv_dim <= 0 || c->kv_dim % 32)
        return CSA2_ERR_INVALID;
    out->idx_block_bytes = (size_t)kBlk * c->n_idx_heads * (c->idx_dim / 2 + c->idx_dim / 32);
    out->kv_row_bytes = (size_t)c->kv_dim / 2 + c->kv_dim / 32;
    out->kv_block_bytes = kBlk * out->kv_row_bytes;
    out->swa_row_bytes = (size_t)c->kv_dim + c->kv_dim / 32;
    return CSA2_OK;
}

extern "C" int csa2_workspace_bytes(const csa2_config *c, int op, int32_t batch, int32_t maxb,
                                    size_t *bytes) {
    if (!c || !bytes || batch < 0 || maxb <= 0) return CSA2_ERR_INVALID;
    if (op == CSA2_OP_INDEX_FULL || op == CSA2_OP_INDEX_REINDEX) {
        const int st = check_cfg(c);
        if (st) return st;
        *bytes = ws_index(batch, maxb, c->pool_blocks).total;
        return CSA2_OK;
    }
    if (op == CSA2_OP_SPARSE_ATTN) {
        if (c->n_q_heads <= 0 || c->kv_dim <= 0 || c->topk <= 0 || c->swa_window < 0)
            return CSA2_ERR_INVALID;
        *bytes = ws_attn(batch, c->n_q_heads, c->kv_dim, attn_splits(c->topk, c->swa_window)).total;
        return CSA2_OK;
    }
    return CSA2_ERR_INVALID;
}

extern "C" const char *csa2_status_str(int s) {
    switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported shape";
    case CSA2_ERR_WORKSPACE: return "workspace too small";
    case CSA2_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
    }
}

namespace {

#define CSA2_CHECK_INDEX_ARGS()                                                              \
    do {                                                                                    \
        const int st_ = check_cfg(c);                                                       \
        if (st_) return st_;                                                                \
        if (!q_codes || !q_scales || !w || !idx_cache || n_blocks <= 0 || !block_table ||   \
            maxb <= 0 || !ctx_len || batch < 0)                                             \
            return CSA2_ERR_INVALID;                                                        \
        if (batch > kMaxBatch) return CSA2_ERR_UNSUPPORTED;                                 \
    } while (0)

}  // namespace

extern "C" int csa2_index_scores(const csa2_config *c, const uint8_t *q_codes,
                                 const uint8_t *q_scales, const float *w,
                                 const uint8_t *idx_cache, int64_t n_blocks,
                                 const int32_t *block_table, int32_t maxb,
                                 const int32_t *ctx_len, int32_t batch, float *scores,
                                 float *block_scores, hipStream_t stream) {
    CSA2_CHECK_INDEX_ARGS();
    if (batch == 0 || (!scores && !block_scores)) return CSA2_OK;
    KernSet ks;
    pick(c->n_idx_heads, c->idx_dim, &ks);
    IndexArgs a{};
    a.q_codes = q_codes;
    a.q_scales = q_scales;
    a.w = w;
    a.idx_cache = idx_cache;
    a.n_blocks = n_blocks;
    a.table = block_table;
    a.maxb = maxb;
    a.B = batch;
    a.K_blk = c->pool_blocks;
    a.k = c->topk;
    a.ctx_len = ctx_len;
    a.scores_out = scores;
    a.block_scores_out = block_scores;
    ks.scan_inspect(dim3(scan_grid(batch, maxb)), stream, a);
    return launched();
}

extern "C" int csa2_index_full_scan(const csa2_config *c, const uint8_t *q_codes,
                                    const uint8_t *q_scales, const float *w,
                                    const uint8_t *idx_cache, int64_t n_blocks,
                                    const int32_t *block_table, int32_t maxb,
                                    const int32_t *ctx_len, int32_t batch, void *ws,
                                    size_t ws_bytes, hipStream_t stream) {
    CSA2_CHECK_INDEX_ARGS();
    if (!ws) return CSA2_ERR_INVALID;
    if (ws_bytes < ws_index(batch, maxb, c->pool_blocks).total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    KernSet ks;
    pick(c->n_idx_heads, c->idx_dim, &ks);
    const IndexArgs a = make_args(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table,
                                  maxb, ctx_len, batch, ws);
    ks.scan_full(dim3(scan_grid(batch, maxb)), stream, a);
    return launched();
}

extern "C" int csa2_index_full_finish(const csa2_config *c, const uint8_t *q_codes,
                                      const uint8_t *q_scales, const float *w,
                                      const uint8_t *idx_cache, int64_t n_blocks,
                                      const int32_t *block_table, int32_t maxb,
                                      const int32_t *ctx_len, int32_t batch,
                                      int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                                      int32_t *topk_len, void *ws, size_t ws_bytes,
                                      hipStream_t stream) {
    CSA2_CHECK_INDEX_ARGS();
    if (!pool_blocks || !pool_len || !topk || !topk_len || !ws) return CSA2_ERR_INVALID;
    if (ws_bytes < ws_index(batch, maxb, c->pool_blocks).total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    KernSet ks;
    pick(c->n_idx_heads, c->idx_dim, &ks);
    IndexArgs a = make_args(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table, maxb,
                            ctx_len, batch, ws);
    k_pool_filter<<<dim3((maxb + 1023) / 1024, batch), 256, 0, stream>>>(a);
    k_pool_final<<<batch, kFinalThreads, 0, stream>>>(a, pool_blocks, pool_len);
    a.pool_blocks = pool_blocks;
    a.pool_len = pool_len;
    const int rb = ks.rescore_blocks;
    ks.rescore(dim3((c->pool_blocks + rb - 1) / rb, batch), stream, a);
    k_select_topk<<<batch, kFinalThreads, 0, stream>>>(a, topk, topk_len);
    return launched();
}

extern "C" int csa2_index_full(const csa2_config *c, const uint8_t *q_codes,
                               const uint8_t *q_scales, const float *w, const uint8_t *idx_cache,
                               int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                               const int32_t *ctx_len, int32_t batch, int32_t *pool_blocks,
                               int32_t *pool_len, int32_t *topk, int32_t *topk_len, void *ws,
                               size_t ws_bytes, hipStream_t stream) {
    CSA2_CHECK_INDEX_ARGS();
    if (!pool_blocks || !pool_len || !topk || !topk_len || !ws) return CSA2_ERR_INVALID;
    int st = csa2_index_full_scan(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table,
                                  maxb, ctx_len, batch, ws, ws_bytes, stream);
    if (st) return st;
    return csa2_index_full_finish(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table,
                                  maxb, ctx_len, batch, pool_blocks, pool_len, topk, topk_len,
                                  ws, ws_bytes, stream);
}

extern "C" int csa2_index_reindex(const csa2_config *c, const uint8_t *q_codes,
                                  const uint8_t *q_scales, const float *w,
                                  const uint8_t *idx_cache, int64_t n_blocks,
                                  const int32_t *block_table, int32_t maxb,
                                  const int32_t *ctx_len, int32_t batch,
                                  const int32_t *pool_blocks, const int32_t *pool_len,
                                  int32_t *topk, int32_t *topk_len, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
    CSA2_CHECK_INDEX_ARGS();
    if (!pool_blocks || !pool_len || !topk || !topk_len || !ws) return CSA2_ERR_INVALID;
    if (ws_bytes < ws_index(batch, maxb, c->pool_blocks).total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    KernSet ks;
    pick(c->n_idx_heads, c->idx_dim, &ks);
    IndexArgs a = make_args(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table, maxb,
                            ctx_len, batch, ws);
    a.pool_blocks = pool_blocks;
    a.pool_len = pool_len;
    const int rb = ks.rescore_blocks;
    ks.rescore(dim3((c->pool_blocks + rb - 1) / rb, batch), stream, a);
    k_select_topk<<<batch, kFinalThreads, 0, stream>>>(a, topk, topk_len);
    return launched();
}
