// csa2_index.hip -- hierarchical sparse indexer of the CSA2 decode step.
//
// What runs (dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心"; and
// prism.simon-ai.net/article/7901, "层级稀疏索引器：精准筛选关键信息"): a Full layer scores
// every visible position with FP4 indexer keys, reduces the scores to 8-position blocks,
// keeps a pool of the K_blk best blocks, then the k best positions inside the pool; a
// Reindex layer rescores only the pool.
//
// Kernels (all asynchronous on the caller's stream, no atomics on shared counters):
//   k_scan<.., false>  HBM stream over every visible key.  Exact FP4 dot products (gfx950
//                      scaled FP4->f16 converts + v_dot2_f32_f16), fixed-order fp32 score,
//                      written per position; block maxima; and the maximum of every group
//                      of 8 consecutive blocks.
//   k_scan<.., true>   the same arithmetic over the 8 positions of every pool block
//                      (Reindex rescoring).
//   k_select           (csa2_select.hip) one workgroup per sequence.  Full: the pool from
//                      the block and group maxima, then the top-k inside the pool from the
//                      stored position scores.  Reindex: the top-k from the rescored pool.
//
// Score (this library's definition; the pages give none): s(p) = sum_h w_h ReLU(q_h.k_{p,h})
// in a fixed fp32 order.  Per 32-group the dot of the unscaled E2M1 values is exact in
// fp32 (products are multiples of 1/4, |sum| <= 1152), so v_dot2_f32_f16 accumulates it
// exactly in any order; t_j = dot * 2^(E_j) is exact; the group sum, ReLU and the fma chain
// over heads then follow one fixed order, so the result is bit-reproducible.

#include <algorithm>

#include "csa2_block.h"
#include "csa2_layer.h"
#include "csa2_quant.h"
#include "csa2_select.h"

namespace csa2 {

constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kHold = 8;  // item outputs a scan wave holds in LDS before storing them
constexpr int kScanGridMax = 512;   // workgroups of a scan (grid-stride over waves): two per
                                    // CU, so that each wave runs enough steps to amortise its
                                    // pipeline fill

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

// The query bytes of head h as loaded (codes, scales, weights), decoded by decode_query;
// split so that the loads can be issued long before the values are needed.
template <int H, int G>
struct QueryRaw {
    uint4 c[G];
    uint32_t s;  // the G scale bytes of the head (byte g: group g)
    float w[H];
};

template <int H, int G>
__device__ __forceinline__ void load_query_raw(QueryRaw<H, G> &R, const uint8_t *qc,
                                               const uint8_t *qs, const float *w, int h) {
    const uint4 *c4 = reinterpret_cast<const uint4 *>(qc + h * 16 * G);
#pragma unroll
    for (int g = 0; g < G; g++) R.c[g] = c4[g];
    if constexpr (G == 1) R.s = qs[h];
    else if constexpr (G == 2) R.s = *reinterpret_cast<const uint16_t *>(qs + h * 2);
    else R.s = *reinterpret_cast<const uint32_t *>(qs + h * 4);
#pragma unroll
    for (int j = 0; j < H; j++) R.w[j] = w[j];
}

// (the raw values are pinned here, so that their first use -- and the wait for the loads --
// is not hoisted up to the loads)
template <int H, int G>
__device__ __forceinline__ void decode_query(Query<H, G> &Q, QueryRaw<H, G> R) {
    asm volatile("" : "+v"(R.s));
#pragma unroll
    for (int g = 0; g < G; g++) {
        asm volatile("" : "+v"(R.c[g].x), "+v"(R.c[g].y), "+v"(R.c[g].z), "+v"(R.c[g].w));
        cvt_fp4x8_f16(R.c[g].x, Q.q + 16 * g + 0);
        cvt_fp4x8_f16(R.c[g].y, Q.q + 16 * g + 4);
        cvt_fp4x8_f16(R.c[g].z, Q.q + 16 * g + 8);
        cvt_fp4x8_f16(R.c[g].w, Q.q + 16 * g + 12);
        Q.e[g] = (int)((R.s >> (8 * g)) & 255u) - 127;
    }
#pragma unroll
    for (int j = 0; j < H; j++) Q.w[j] = R.w[j];
}

template <int H, int G>
__device__ __forceinline__ void load_query(Query<H, G> &Q, const uint8_t *qc, const uint8_t *qs,
                                           const float *w, int h) {
    QueryRaw<H, G> R;
    load_query_raw(R, qc, qs, w, h);
    decode_query(Q, R);
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
__device__ __forceinline__ float head_relu(const Query<H, G> &Q, const uint4 *kc, uint32_t ks) {
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

// Block-level helpers (wave and block reductions, scans, clamp_len): csa2_block.h

// ------------------------------------------------------------------ k_scan

struct ScanArgs {
    const uint8_t *q_codes;
    const uint8_t *q_scales;
    const float *q_f32;  // the unquantised query [B][H*dI] (non-null: quantised in the kernel)
    const float *w;
    const uint8_t *idx_cache;
    int64_t n_blocks;
    const int32_t *table;
    int32_t maxb;
    const int32_t *ctx_len;
    int32_t B;
    // scan outputs (any may be null): position scores [B][maxb*8], block maxima [B][maxb],
    // group maxima [B][ngmax]
    float *pscore;
    float *bscore;
    float *gmax;
    int32_t *arrive;  // [B] arrival counters of the two-phase selection, zeroed here (or null)
    int32_t ngmax;
    int32_t bstride;  // row stride of bscore (floats)
    // rescore mode: pool [B][K_blk], pool_len [B] -> pool scores [B][K_blk*8]
    const int32_t *pool;
    const int32_t *pool_len;
    int32_t K_blk;
    float *poolsc;
    float *poolbmax;  // rescore: pool block maxima [B][K_blk]
    // fused append of each sequence's current token, position ctx_len[b] - 1 (Full scan
    // only; new_key null: none): its indexer key [B][H*dI] and main latent [B][kAppD] fp32
    // (new_lat may be null), quantised into the caches by the wave that scores its block
    const float *new_key;
    const float *new_lat;
    uint8_t *idx_w;  // the indexer-key cache (the same bytes as idx_cache)
    uint8_t *kv_w;   // the main-KV cache
};

constexpr int kAppD = 512;  // main latent dim of the fused append

// MXFP4 quantisation of 32-groups spread over 8 lanes: lane l holds elements 4(l%8)..+3 of
// group l/8.  Returns the group's E8M0 code in every lane and, in the even lane of each
// lane pair, the code word of the pair's 8 elements (element 8i+j in bits 4j..4j+3, i =
// (l%8)/2), the word layout of quant_fp4_regs.  The amax is a max (exact in any order) and
// each element is encoded by fp4_code, so the codes equal quant_fp4's.
__device__ __forceinline__ void coop_fp4(float4 v, uint32_t &word, uint32_t &scale) {
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    am = fmaxf(am, dpp(am, std::integral_constant<int, 0xB1>{}));   // quad [1,0,3,2]
    am = fmaxf(am, dpp(am, std::integral_constant<int, 0x4E>{}));   // quad [2,3,0,1]
    am = fmaxf(am, dpp(am, std::integral_constant<int, 0x141>{}));  // row_half_mirror (8 lanes)
    const int e = group_exponent(am, 2);
    const uint32_t c = fp4_code(v.x, e) | fp4_code(v.y, e) << 4 | fp4_code(v.z, e) << 8 |
                       fp4_code(v.w, e) << 12;
    const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)c, 0xB1, 0xf, 0xf, false);
    word = c | nb << 16;
    scale = (uint32_t)(e + 127);
}

// The new token's inputs of one sequence as one wave loads them: key float4 chunk 64r + lane
// in key[r], latent chunk 64r + lane in lat[r], and the table entry of its block.
template <int H, int G>
struct AppendRegs {
    static constexpr int KR = (H * G * 8 + kWave - 1) / kWave;  // rounds of key chunks
    static constexpr int LR = kAppD / 4 / kWave;                // rounds of latent chunks
    float4 key[KR];
    float4 lat[LR];
    int ph;
};

// The unquantised query of one sequence as one wave loads it: float4 chunk 64r + lane in
// f[r] (every element loaded once per wave).
template <int H, int G>
struct QueryF32 {
    static constexpr int R = (H * G * 8 + kWave - 1) / kWave;  // rounds of chunks
    float4 f[R];
};

template <int H, int G>
__device__ __forceinline__ void load_query_f32(QueryF32<H, G> &F, const float *qf) {
    const float4 *src = reinterpret_cast<const float4 *>(qf);
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < F.R; r++) F.f[r] = src[min(r * kWave + lane, H * G * 8 - 1)];
}

// MXFP4 codes and scales of the loaded query for head h, in the layout load_query_raw reads:
// every 32-group is encoded by 8 lanes (coop_fp4, the encoder of the append kernels, so the
// codes equal csa2_quantize_mxfp4's), then each lane gathers its head's groups.
template <int H, int G>
__device__ __forceinline__ void quant_query(QueryRaw<H, G> &R, const QueryF32<H, G> &F,
                                            const float *w, int h) {
    uint32_t kw[F.R], ksc[F.R];
#pragma unroll
    for (int r = 0; r < F.R; r++) coop_fp4(F.f[r], kw[r], ksc[r]);
    R.s = 0u;
#pragma unroll
    for (int g = 0; g < G; g++) {
        const int q = h * G + g, rq = q / 8, src = 8 * (q % 8);
        uint32_t wv[4], sv = 0u;
#pragma unroll
        for (int rr = 0; rr < F.R; rr++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (src + 2 * i), (int)kw[rr]);
                wv[i] = rr == rq ? x : (rr == 0 ? x : wv[i]);
            }
            const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)ksc[rr]);
            sv = rr == rq ? y : (rr == 0 ? y : sv);
        }
        R.c[g] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        R.s |= sv << (8 * g);
    }
#pragma unroll
    for (int j = 0; j < H; j++) R.w[j] = w[j];
}

// Items (8 blocks or 8 pool entries) of sequence b.
template <bool RESCORE>
__device__ __forceinline__ int items_of(const ScanArgs &a, int b) {
    if (RESCORE) {
        const int pl = max(0, min(a.pool_len[b], a.K_blk));
        return (pl + kItemBlocks - 1) / kItemBlocks;
    }
    const int nb = (clamp_len(a.ctx_len[b], a.maxb) + kBlk - 1) / kBlk;
    return (nb + kItemBlocks - 1) / kItemBlocks;
}

// Exclusive prefix of items per sequence in LDS (prefix[0..B]), the clamped lengths
// (lens[0..B-1]) and the lengths as given (raw[0..B-1]); returns the total.  Each length
// (and pool length) is loaded once.
template <bool RESCORE>
__device__ int build_item_prefix(const ScanArgs &a, int32_t *prefix, int32_t *lens, int32_t *raw,
                                 uint32_t *sh_scan) {
    uint32_t running = 0;
    for (int base = 0; base < a.B; base += kScanThreads) {
        const int b = base + (int)threadIdx.x;
        uint32_t v = 0u;
        if (b < a.B) {
            const int32_t Lr = a.ctx_len[b];
            const int L = clamp_len(Lr, a.maxb);
            lens[b] = L;
            raw[b] = Lr;
            if (RESCORE) {
                const int pl = max(0, min(a.pool_len[b], a.K_blk));
                v = (uint32_t)((pl + kItemBlocks - 1) / kItemBlocks);
            } else {
                v = (uint32_t)((((L + kBlk - 1) / kBlk) + kItemBlocks - 1) / kItemBlocks);
            }
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

__device__ __forceinline__ int seq_of_item(const int32_t *prefix, int B, int it) {
    int lo = 0, hi = B - 1;  // largest b with prefix[b] <= it
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= it) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// s = fma(w_{H-1}, r_{H-1}, ... fma(w_0, r_0, +0)) where lane base+j holds r_j; quad
// broadcasts (DPP) for H <= 4, a permute otherwise.
template <int H, int G>
__device__ __forceinline__ float combine_heads_dpp(const Query<H, G> &Q, float r, int lane) {
    if constexpr (H == 1) {
        return __builtin_fmaf(Q.w[0], r, 0.0f);
    } else if constexpr (H == 2) {
        const float r0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0xA0, 0xf, 0xf, false));
        const float r1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0xF5, 0xf, 0xf, false));
        return __builtin_fmaf(Q.w[1], r1, __builtin_fmaf(Q.w[0], r0, 0.0f));
    } else if constexpr (H == 4) {
        float s = __builtin_fmaf(Q.w[0], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0x00, 0xf, 0xf, false)), 0.0f);
        s = __builtin_fmaf(Q.w[1], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0x55, 0xf, 0xf, false)), s);
        s = __builtin_fmaf(Q.w[2], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0xAA, 0xf, 0xf, false)), s);
        s = __builtin_fmaf(Q.w[3], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0xFF, 0xf, 0xf, false)), s);
        return s;
    } else {
        return combine_heads<H, G>(Q, r, lane);
    }
}

__device__ __forceinline__ float fmax_sel(float a, float b) { return a > b ? a : b; }

// Key bytes of one position-head as one lane loads them: G chunks of 16 code bytes and G
// scale bytes.
template <int G>
struct KeyRegs {
    uint4 kc[G];
    uint32_t ks;
};

// DPP max of x with the lane selected by `ctrl` (lanes outside row_mask keep x).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_max(float x) {
    const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
    return __builtin_elementwise_maximum(x, __int_as_float(y));
}

// Maximum over the 8*H lanes of a block (the H lanes of a position hold the same value);
// the block's last lane (lane % (8H) == 8H - 1) holds it.
template <int H>
__device__ __forceinline__ float block_max_lanes(float m) {
    if constexpr (H == 1) {
        m = dpp_max<0xB1>(m);          // quad [1,0,3,2]
        m = dpp_max<0x4E>(m);          // quad [2,3,0,1]
        m = dpp_max<0x141>(m);         // row_half_mirror
    } else if constexpr (H == 2) {
        m = dpp_max<0x4E>(m);
        m = dpp_max<0x141>(m);
        m = dpp_max<0x140>(m);         // row_mirror
    } else if constexpr (H == 4) {
        m = dpp_max<0x141>(m);
        m = dpp_max<0x140>(m);
        m = dpp_max<0x142, 0xa>(m);    // row_bcast:15 into rows 1, 3
    } else {
        m = dpp_max<0x140>(m);
        m = dpp_max<0x142, 0xa>(m);
        m = dpp_max<0x143, 0xc>(m);    // row_bcast:31 into rows 2, 3
    }
    return m;
}

// Maximum over the blocks' last lanes into lane 63.
template <int H>
__device__ __forceinline__ float blocks_to_lane63(float m) {
    if constexpr (H == 1) m = dpp_max<0x140>(m);
    if constexpr (H <= 2) m = dpp_max<0x142, 0xa>(m);
    if constexpr (H <= 4) m = dpp_max<0x143, 0xc>(m);
    return m;
}

// Uniform load through the scalar data cache (read-only data; waits count on lgkmcnt, so they
// never wait for the vector loads in flight).
template <class T>
__device__ __forceinline__ T sload(const T *p, int64_t i) {
    return ((const __attribute__((address_space(4))) T *)(uintptr_t)p)[i];
}

// Per-step block bookkeeping of one wave: the entry index of the step's first block
// (uniform) and, per lane, the logical and physical block of the lane's own block (-1: none).
// Block-table and pool entries are per-lane vector loads: vector loads complete in issue
// order, so waiting for the entries of an earlier step never waits for later ones (scalar
// loads complete out of order, and a wait for any one of them is a wait for all).
struct StepMeta {
    int e0;    // entry index (block or pool entry) of the step's first block
    int jraw;  // rescore: the loaded pool entry (validated when the block is looked up)
    int j;     // logical block (-1: none)
    int ph;    // physical block as loaded (validated where it is used)
};

// One wave processes a contiguous range of items; an item is 8 consecutive blocks (scan)
// or 8 consecutive pool entries (rescore) of one sequence, BPW blocks per step, lane =
// (position in step) * H + head.  Software pipeline: step k issues the pool entries of step
// k+6 (rescoring), the block-table entries of step k+4 and the keys of step k+2, in that
// order, then computes step k.  Every value step k uses was requested by step k-2 or
// earlier, and vector loads complete in issue order, so no wait covers a load of step k-1.
// An item's scores and maxima leave in two stores at its last step, masked to the lanes
// that hold output.  Loads never branch: an absent block reads physical block 0 and its
// positions are masked.  OFF32: every key byte lies within 4 GiB of the cache base, so
// addresses are a scalar base plus a 32-bit lane offset.
template <int H, int G, bool RESCORE, bool OFF32, bool APPEND>
__global__ __launch_bounds__(kScanThreads, 2) void k_scan(ScanArgs a) {
    if (a.arrive && blockIdx.x == 0)  // (read by the selection, which runs after this kernel)
        for (int i = (int)threadIdx.x; i < a.B; i += kScanThreads) a.arrive[i] = 0;
    constexpr int BPW = 8 / H;                         // blocks per wave step
    constexpr int NSTEP = kItemBlocks / BPW;           // steps per item
    constexpr int CODES = kBlk * H * 16 * G;
    constexpr int BYTES = CODES + kBlk * H * G;
    extern __shared__ int32_t sh_dyn[];  // item prefix [B + 1], clamped lengths [B], lengths [B]
    __shared__ __align__(16) uint32_t sh_scan[kScanWaves];
    int32_t *sh_prefix = sh_dyn, *sh_len = sh_dyn + a.B + 1, *sh_raw = sh_dyn + 2 * a.B + 1;
    // Item outputs are held in LDS and stored after the wave's key loads (every kHold items):
    // stores count with the loads in the in-order vmcnt, and interleaved with the stream of
    // key loads they measured ~3.5 us per scan at 1M positions.  Per held item: the 64
    // position scores, the block and group maxima (lanes 0..7, 63) and (sequence, first
    // entry, in segment, entry limit).
    __shared__ __align__(16) float sh_hold[kScanWaves][kHold][2][kWave];
    __shared__ __align__(16) int4 sh_hmeta[kScanWaves][kHold];
    int nhold = 0;  // uniform

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int h = lane % H, pw = lane / H, bw = pw / kBlk, slot = pw % kBlk;
    const int nwaves = (int)gridDim.x * kScanWaves;
    const int gw = (int)blockIdx.x * kScanWaves + wave;
    // Items of a wave: one sequence -> items gw, gw + nwaves, ... (all resident waves read
    // one contiguous window of the cache at a time, spread over every HBM channel);
    // several sequences -> a contiguous range, so each wave meets few sequences.
    const bool inter = a.B == 1;
    // pipeline depth: bookkeeping of steps k .. k+DM-1, block-table entries of steps k .. k+DPH-1
    constexpr int DM = 7, DPH = 4, DK = 2;  // (and keys of steps k .. k+DK-1)
    // One sequence: the query and the first steps' entries (scan: block-table entries;
    // rescoring: pool entries) depend on no length and are requested before the item prefix,
    // whose length load and barriers they overlap (entries read clamped into the row and
    // masked once the length is known).
    auto entry0 = [&](int k2) {  // first entry of step k2 of an interleaved wave
        return (gw + (k2 / NSTEP) * nwaves) * kItemBlocks + (k2 % NSTEP) * BPW;
    };
    Query<H, G> Q;
    QueryRaw<H, G> QR;
    QueryF32<H, G> QF;
    const bool qf32 = a.q_f32 != nullptr;
    int pre[DM - 1] = {};
    if (inter) {
#pragma unroll
        for (int i = 0; i < (RESCORE ? DM - 1 : DPH); i++) {
            const int e = entry0(i) + bw;
            pre[i] = RESCORE ? a.pool[min(e, a.K_blk - 1)] : a.table[min(e, a.maxb - 1)];
        }
        if (qf32) {
            load_query_f32<H, G>(QF, a.q_f32);
            // a query of several rounds is encoded at once (its floats would stay live across
            // the prefix); one round is encoded after it, overlapping the load with the prefix
            if constexpr (QueryF32<H, G>::R > 1) quant_query<H, G>(QR, QF, a.w, h);
        } else {
            load_query_raw<H, G>(QR, a.q_codes, a.q_scales, a.w, h);
        }
    }
    const int total = __builtin_amdgcn_readfirstlane(build_item_prefix<RESCORE>(a, sh_prefix, sh_len, sh_raw, sh_scan));
    const int per = (total + nwaves - 1) / nwaves;
    const int it_begin = inter ? gw : gw * per;
    const int it_end = inter ? total : min(total, it_begin + per);
    if (it_begin >= it_end) return;
    const int nsteps = inter ? (total - gw + nwaves - 1) / nwaves * NSTEP : (it_end - it_begin) * NSTEP;
    const uint32_t lane_off = (uint32_t)((slot * H + h) * 16);
    // the lane's G scale bytes, read as the aligned dword that holds them (blocks are
    // multiples of 8 bytes) and shifted where they are used, so that nothing in the loading
    // step consumes the value
    const uint32_t sc_byte = (uint32_t)(CODES + (slot * H + h) * G);
    const uint32_t sc_off = sc_byte & ~3u, sc_sh = 8u * (sc_byte & 3u);

    constexpr int PPS = kBlk * BPW;                    // positions per step
    constexpr int STEPS = NSTEP >= 4 ? NSTEP : 4;      // steps per loop iteration (whole items)
    // gather sources: position l of an item is computed in lane (l % PPS) * H of step l / PPS;
    // block i of an item ends in lane (i % BPW + 1) * 8H - 1 of step i / BPW
    const int src_p = (lane % PPS) * H;
    const int src_b = ((lane % BPW) + 1) * kBlk * H - 1;

    // a lane's physical block: the loaded table entry when its logical block exists and the
    // entry lies in the cache, else -1
    auto phys_of = [&](const StepMeta &m) -> int {
        return m.j >= 0 && m.ph >= 0 && (int64_t)m.ph < a.n_blocks ? m.ph : -1;
    };
    auto load_keys = [&](const StepMeta &m, KeyRegs<G> &kr) {
        const int ph = phys_of(m);
        const uint32_t p = (uint32_t)(ph >= 0 ? ph : 0);
        if constexpr (OFF32) {
            const uint32_t base = p * (uint32_t)BYTES;
#pragma unroll
            for (int g = 0; g < G; g++)
                kr.kc[g] = *reinterpret_cast<const uint4 *>(a.idx_cache + (base + lane_off + (uint32_t)(g * kBlk * H * 16)));
            kr.ks = *reinterpret_cast<const uint32_t *>(a.idx_cache + (base + sc_off));
        } else {
            const uint8_t *bp = a.idx_cache + (int64_t)p * BYTES;
#pragma unroll
            for (int g = 0; g < G; g++)
                kr.kc[g] = *reinterpret_cast<const uint4 *>(bp + lane_off + g * kBlk * H * 16);
            kr.ks = *reinterpret_cast<const uint32_t *>(bp + sc_off);
        }
    };
    float gm = -INFINITY;
    const bool ps_on = RESCORE || a.pscore, pb_on = RESCORE || a.bscore, pg_on = !RESCORE && a.gmax;
    // the held items' stores (lanes without output are masked off: no store of theirs reaches
    // memory)
    auto flush = [&] {
        for (int i = 0; i < nhold; i++) {
            const int4 m = sh_hmeta[wave][i];
            const int hb = __builtin_amdgcn_readfirstlane(m.x), he = __builtin_amdgcn_readfirstlane(m.y);
            const bool hok = __builtin_amdgcn_readfirstlane(m.z) != 0;
            const int hlim = __builtin_amdgcn_readfirstlane(m.w);
            const float vp = sh_hold[wave][i][0][lane], vs = sh_hold[wave][i][1][lane];
            float *ps = (RESCORE ? a.poolsc + (int64_t)hb * a.K_blk * kBlk : a.pscore + (int64_t)hb * a.maxb * kBlk) +
                        (int64_t)he * kBlk + lane;
            float *pb = (RESCORE ? a.poolbmax + (int64_t)hb * a.K_blk : a.bscore + (int64_t)hb * a.bstride) + he + lane;
            const bool pos_ok = hok && he + lane / kBlk < hlim;
            bool pb_ok = lane < kBlk && hok && he + lane < hlim && pb_on;
            if (!RESCORE && lane == kWave - 1) {
                pb_ok = hok && pg_on;
                pb = a.gmax + (int64_t)hb * a.ngmax + he / kItemBlocks;
            }
            if (pos_ok && ps_on) *ps = vp;
            if (pb_ok) *pb = vs;
        }
        nhold = 0;
    };

    // The wave's steps split into segments of one sequence each (items are 8-aligned, so a
    // segment starts at an item boundary).  Per segment: the query, row bases and lengths;
    // per step only an entry index that advances by BPW.
    int cur_b = 0;
    int k = 0;
    while (k < nsteps) {
        const int it0 = it_begin + k / NSTEP;
        if (a.B > 1)
            while (cur_b + 1 < a.B && __builtin_amdgcn_readfirstlane(sh_prefix[cur_b + 1]) <= it0) cur_b++;
        const int b = cur_b;
        const int kend = b + 1 < a.B
            ? min(nsteps, (__builtin_amdgcn_readfirstlane(sh_prefix[b + 1]) - it_begin) * NSTEP)
            : nsteps;
        const int kseg = k;
        const int e_start = (it0 - __builtin_amdgcn_readfirstlane(sh_prefix[b])) * kItemBlocks;
        const int L = __builtin_amdgcn_readfirstlane(sh_len[b]);
        const int nb = (L + kBlk - 1) / kBlk;
        const int32_t *table_row = a.table + (int64_t)b * a.maxb;
        const int32_t *pool_row = RESCORE ? a.pool + (int64_t)b * a.K_blk : nullptr;
        const int n_ent = RESCORE ? max(0, min(sload(a.pool_len, b), a.K_blk)) : 0;

        // entries of step k2 of this segment (-1 past its end); rescoring loads the lane's pool
        // entry (read clamped into the row, checked by meta_phys a step later) unless it was
        // requested already (`have`: its value is hv)
        auto meta_entries = [&](int k2, StepMeta &m, bool have = false, int hv = 0) {
            m.e0 = inter ? entry0(k2) : e_start + (k2 - kseg) * BPW;
            const int e = m.e0 + bw;
            const bool live = k2 < kend && e < (RESCORE ? n_ent : nb);
            if (RESCORE) {
                m.jraw = have ? hv : pool_row[live ? e : 0];
                m.j = live ? 0 : -1;
            } else {
                m.j = live ? e : -1;
            }
            m.ph = -1;
        };
        // the lane's block-table entry (its use comes at least a step later)
        auto meta_phys = [&](StepMeta &m) {
            if (RESCORE) m.j = m.j >= 0 && m.jraw >= 0 && m.jraw < nb ? m.jraw : -1;
            m.ph = table_row[m.j >= 0 ? m.j : 0];
        };

        if (inter) {
            if constexpr (QueryF32<H, G>::R == 1)
                if (qf32) quant_query<H, G>(QR, QF, a.w, h);
            decode_query<H, G>(Q, QR);
        } else if (qf32) {
            load_query_f32<H, G>(QF, a.q_f32 + (size_t)b * H * 32 * G);
            quant_query<H, G>(QR, QF, a.w + (size_t)b * H, h);
            decode_query<H, G>(Q, QR);
        } else {
            load_query<H, G>(Q, a.q_codes + (size_t)b * H * 16 * G, a.q_scales + (size_t)b * H * G,
                             a.w + (size_t)b * H, h);
        }

        // ---- fused append: does this segment score the block of the new token (position
        //      pn = L_b - 1, unclamped)?  k_new: that step (uniform; -1: not here).  Its inputs
        //      are requested now; before the keys of step k_new are loaded, the wave quantises
        //      them and the lane that loads each key chunk of the new slot writes it first, so
        //      that lane's own load reads its own store (the latent goes to the main-KV cache).
        int k_new = -1, pn = -1;
        AppendRegs<H, G> ar;
        if (APPEND) {
            pn = __builtin_amdgcn_readfirstlane(sh_raw[b]) - 1;
            if (pn >= 0 && pn / kBlk < a.maxb) {
                const int jn = pn / kBlk, itn = jn / kItemBlocks, stn = (jn % kItemBlocks) / BPW;
                if (inter) {
                    if (itn >= gw && (itn - gw) % nwaves == 0) k_new = (itn - gw) / nwaves * NSTEP + stn;
                } else {
                    const int kk = (__builtin_amdgcn_readfirstlane(sh_prefix[b]) + itn - it_begin) * NSTEP + stn;
                    if (kk >= kseg && kk < kend) k_new = kk;
                }
            }
            if (k_new >= 0) {
                const float4 *kb = reinterpret_cast<const float4 *>(a.new_key + (size_t)b * H * G * 32);
#pragma unroll
                for (int r = 0; r < ar.KR; r++) ar.key[r] = kb[min(r * kWave + lane, H * G * 8 - 1)];
                if (a.new_lat) {
                    const float4 *lb = reinterpret_cast<const float4 *>(a.new_lat + (size_t)b * kAppD);
#pragma unroll
                    for (int r = 0; r < ar.LR; r++) ar.lat[r] = lb[r * kWave + lane];
                }
                ar.ph = table_row[pn / kBlk];
            }
        }
        auto append_write = [&] {
            const int ph = ar.ph >= 0 && (int64_t)ar.ph < a.n_blocks ? ar.ph : -1;
            const int sn = pn % kBlk;
            // key: groups q = h*G + g in rounds of 8; lane (pair) words, group scales
            uint32_t kw[ar.KR], ksc[ar.KR];
#pragma unroll
            for (int r = 0; r < ar.KR; r++) coop_fp4(ar.key[r], kw[r], ksc[r]);
            const bool writer = ph >= 0 && bw == (pn / kBlk) % BPW && slot == sn;
#pragma unroll
            for (int g = 0; g < G; g++) {
                const int q = h * G + g, r = q / 8, src = 8 * (q % 8);
                uint32_t wv[4], sv = 0u;
#pragma unroll
                for (int rr = 0; rr < ar.KR; rr++) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (src + 2 * i), (int)kw[rr]);
                        wv[i] = rr == r ? x : (rr == 0 ? x : wv[i]);
                    }
                    const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)ksc[rr]);
                    sv = rr == r ? y : (rr == 0 ? y : sv);
                }
                if (writer) {
                    uint8_t *blk = a.idx_w + (int64_t)ph * BYTES;
                    *reinterpret_cast<uint4 *>(blk + ((g * kBlk + sn) * H + h) * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                    blk[CODES + (sn * H + h) * G + g] = (uint8_t)sv;
                }
            }
            if (a.new_lat && ph >= 0) {
                uint8_t *row = a.kv_w + ((int64_t)ph * kBlk + sn) * (kAppD / 2 + kAppD / 32);
#pragma unroll
                for (int r = 0; r < ar.LR; r++) {
                    uint32_t lw, lsc;
                    coop_fp4(ar.lat[r], lw, lsc);
                    const int c = r * kWave + lane, gl = c / 8;
                    if ((c & 1) == 0) *reinterpret_cast<uint32_t *>(row + 16 * gl + 2 * (c % 8)) = lw;
                    if (c % 8 == 0) row[kAppD / 2 + gl] = (uint8_t)lsc;
                }
            }
        };
        if (APPEND && k_new >= 0 && k_new < k + DK) {  // before the prologue's key loads
            append_write();
            k_new = -1;
        }
        // pipeline state at step k: entries of steps k..k+5 (rescoring: pool entries loaded),
        // table entries of steps k..k+3 loaded, keys of steps k and k+1 loaded (one sequence:
        // k = 0 here, and the early requests above stand in for the first loads)
        StepMeta mt[DM];
#pragma unroll
        for (int i = 0; i < DM - 1; i++) meta_entries(k + i, mt[i], RESCORE && inter, pre[i]);
#pragma unroll
        for (int i = 0; i < DPH; i++) {
            if (!RESCORE && inter) mt[i].ph = pre[i];
            else meta_phys(mt[i]);
        }
        KeyRegs<G> K[4];
        load_keys(mt[0], K[0]);
        load_keys(mt[1], K[1]);

        const int n_lim = RESCORE ? n_ent : nb;  // entries of the segment's row

        // scores and block maxima of the current item, gathered so that lane l holds position
        // l (acc_p) and lanes 0..7 the maxima of blocks 0..7 (acc_b)
        float acc_p = 0.0f, acc_b = 0.0f;
        auto body = [&](int k2, int si, KeyRegs<G> &cur, KeyRegs<G> &nxt2) {
            meta_entries(k2 + 6, mt[6]);
            meta_phys(mt[4]);
            load_keys(mt[2], nxt2);
            const float r = head_relu<H, G>(Q, cur.kc, cur.ks >> sc_sh);
            const float sc = combine_heads_dpp<H, G>(Q, r, lane);
            const int j = mt[0].j, ph = phys_of(mt[0]);
            const bool vis = ph >= 0 && j * kBlk + slot < L;
            const float val = vis ? sc : -INFINITY;
            const float m = block_max_lanes<H>(val);
            const float vp = __shfl(val, src_p, kWave);
            const float vb = __shfl(m, src_b, kWave);
            acc_p = lane / PPS == si ? vp : acc_p;
            acc_b = lane / BPW == si ? vb : acc_b;
            if (!RESCORE) {
                // the item's group maximum so far, in lane 63
                gm = __builtin_elementwise_maximum(si == 0 ? -INFINITY : gm, m);
            }
            if (si == NSTEP - 1) {
                // the item's outputs (64 position scores, 8 block maxima, the group maximum
                // in lane 63) wait in LDS
                const int e_item = mt[0].e0 - (NSTEP - 1) * BPW;
                float vstore = acc_b;
                if (!RESCORE) {
                    const float g63 = blocks_to_lane63<H>(gm);
                    if (lane == kWave - 1) vstore = g63;
                }
                sh_hold[wave][nhold][0][lane] = acc_p;
                sh_hold[wave][nhold][1][lane] = vstore;
                if (lane == 0) sh_hmeta[wave][nhold] = make_int4(b, e_item, k2 < kend ? 1 : 0, n_lim);
                nhold++;
            }
#pragma unroll
            for (int i = 0; i < DM - 1; i++) mt[i] = mt[i + 1];
        };
        // iterations of STEPS steps (whole items); steps past the segment end are masked
        for (; k < kend; k += STEPS) {
            if (nhold + STEPS / NSTEP > kHold) flush();  // room for this iteration's items
            if (APPEND && k_new >= 0 && k_new - DK < k + STEPS) {  // before this iteration's key loads
                append_write();
                k_new = -1;
            }
#pragma unroll
            for (int st = 0; st < STEPS; st++) body(k + st, st % NSTEP, K[st % 4], K[(st + 2) % 4]);
        }
    }
    flush();
}

// ------------------------------------------------------------------ k_scan_shared
//
// The shared-key variant of the scan (one d_I key per position scored by all H query
// heads).  Per 16-position tile one scaled-FP4 matrix instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4) forms every (head, position) dot: operand A holds the
// query heads (rows), operand B the tile's keys (columns), each lane one 32-group of one row
// or column with its E8M0 scale, so that lane (column c, g) reads the 16 code bytes of group
// g of position c straight from the block layout.  The result lane (position c, g) holds
// heads 4g .. 4g+3.  Exactness as in the prefill kernel: the matrix core adds the scaled
// group products in an undisclosed order, which equals the defined fp32 group order whenever
// every partial sum is representable -- |N_g| <= 4608 < 2^13, so an exponent span
// max_g E_g - min_g E_g <= 9 keeps every partial inside 24 bits.  An item whose key span plus
// the query's exceeds that takes one instruction per group (the other groups' key lanes
// zeroed, each product exact) and adds the groups in order.  Epilogue: ReLU, the fma chain
// over heads in head order, block and group maxima -- the outputs k_scan writes, read by the
// same selection.  Pipeline per wave over its items: pool entries three items ahead
// (rescoring), block-table entries two ahead, keys one ahead.

typedef int v8i_t __attribute__((ext_vector_type(8)));
constexpr int kSpanExactShared = 9;

__device__ __forceinline__ f32x4_t mfma_fp4_sk(const uint4 &a, const uint4 &b, uint32_t sa,
                                               uint32_t sb) {
    const v8i_t av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    // formats 4/4: both operands FP4 E2M1; scales in byte 0 of sa and sb
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 4, 0, (int)sa, 0, (int)sb);
}

// max(x, +0) exactly as defined (every negative value and -0 give +0) in one integer max.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Largest minus smallest of the n low bytes of w.
template <int N>
__device__ __forceinline__ int byte_span(uint32_t w) {
    int lo = 255, hi = 0;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const int v = (int)((w >> (8 * i)) & 255u);
        lo = min(lo, v);
        hi = max(hi, v);
    }
    return hi - lo;
}

__device__ __forceinline__ int wave_max_i(int v) {
    return (int)wave_reduce_to63((uint32_t)v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}

// The MXFP4 codes and E8M0 scale of query group q (head-major index, runtime per lane) from
// the loaded fp32 query: every group encoded by 8 lanes (coop_fp4), then this lane's group
// gathered with ds_bpermute.
template <int H, int G>
__device__ __forceinline__ void quant_query_group(const QueryF32<H, G> &F, int q, uint4 &codes,
                                                  uint32_t &scale) {
    constexpr int R = QueryF32<H, G>::R;
    uint32_t kw[R], ksc[R];
#pragma unroll
    for (int r = 0; r < R; r++) coop_fp4(F.f[r], kw[r], ksc[r]);
    const int rq = q / 8, src = 8 * (q % 8);
    uint32_t wv[4], sv = 0u;
#pragma unroll
    for (int rr = 0; rr < R; rr++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (src + 2 * i), (int)kw[rr]);
            wv[i] = rr == rq ? x : (rr == 0 ? x : wv[i]);
        }
        const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)ksc[rr]);
        sv = rr == rq ? y : (rr == 0 ? y : sv);
    }
    codes = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    scale = sv;
}

template <int H, int G, bool RESCORE>
__global__ __launch_bounds__(kScanThreads, 2) void k_scan_shared(ScanArgs a) {
    if (a.arrive && blockIdx.x == 0)  // (read by the selection, which runs after this kernel)
        for (int i = (int)threadIdx.x; i < a.B; i += kScanThreads) a.arrive[i] = 0;
    constexpr int CODES = kBlk * 16 * G;  // code bytes of a block (one key per position)
    constexpr int BYTES = CODES + kBlk * G;
    constexpr int T = 4;                  // 16-position tiles per item
    extern __shared__ int32_t sh_dyn[];   // item prefix [B + 1], clamped lengths [B], lengths [B]
    __shared__ __align__(16) uint32_t sh_scan[kScanWaves];
    int32_t *sh_prefix = sh_dyn, *sh_len = sh_dyn + a.B + 1, *sh_raw = sh_dyn + 2 * a.B + 1;

    const int lane = lane_id(), col = lane & 15, g = lane >> 4, slot = col & 7;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int nwaves = (int)gridDim.x * kScanWaves;
    const int gw = (int)blockIdx.x * kScanWaves + wave;
    const bool inter = a.B == 1;
    const int total = __builtin_amdgcn_readfirstlane(build_item_prefix<RESCORE>(a, sh_prefix, sh_len, sh_raw, sh_scan));
    const int per = (total + nwaves - 1) / nwaves;
    const int it_begin = inter ? gw : gw * per;
    const int it_end = inter ? total : min(total, it_begin + per);
    if (it_begin >= it_end) return;
    const int n_items = inter ? (total - gw + nwaves - 1) / nwaves : it_end - it_begin;

    // the uniform part of item k of this wave: sequence, first entry, existence
    struct ItemU {
        int b, e0;
        bool ok;
    };
    auto item_u = [&](int k) -> ItemU {
        ItemU u;
        u.ok = k < n_items;
        const int it = inter ? gw + (u.ok ? k : 0) * nwaves : it_begin + (u.ok ? k : 0);
        u.b = a.B > 1 ? __builtin_amdgcn_readfirstlane(seq_of_item(sh_prefix, a.B, it)) : 0;
        u.e0 = (it - __builtin_amdgcn_readfirstlane(sh_prefix[u.b])) * kItemBlocks;
        return u;
    };
    auto nb_of = [&](int b) { return (__builtin_amdgcn_readfirstlane(sh_len[b]) + kBlk - 1) / kBlk; };
    auto nent_of = [&](int b) {
        return RESCORE ? max(0, min(sload(a.pool_len, b), a.K_blk)) : 0;
    };
    // per lane and tile t: the item's entry of this lane's position, 2t + col/8
    auto entry = [&](const ItemU &u, int t) { return u.e0 + 2 * t + (col >> 3); };

    // Pipeline rings (indices static: the loop is unrolled by 4 and items advance by 4):
    // pool entries of items k+1 .. k+3 (rescoring), logical block (-1: none) and table entry
    // of items k+1, k+2, key codes, scale words and visibility of items k, k+1.  Loads never
    // branch: items past the wave's last read its first item's entries and are not stored.
    int praw[4][T];
    int lj[2][T], lph[2][T];
    uint4 kc[2][T];
    uint32_t ksw[2][T];  // the position's G scale bytes from byte 0
    int vis[2][T];       // logical block of the key (-1: no key)

    auto load_pool = [&](int k, int (&pr)[T]) {
        if constexpr (RESCORE) {
            const ItemU u = item_u(k);
            const int32_t *pool_row = a.pool + (int64_t)u.b * a.K_blk;
#pragma unroll
            for (int t = 0; t < T; t++) pr[t] = pool_row[min(entry(u, t), a.K_blk - 1)];
        }
    };
    auto load_table = [&](int k, const int (&pr)[T], int (&j_out)[T], int (&ph_out)[T]) {
        const ItemU u = item_u(k);
        const int nb = nb_of(u.b);
        const int n_ent = nent_of(u.b);
        const int32_t *table_row = a.table + (int64_t)u.b * a.maxb;
#pragma unroll
        for (int t = 0; t < T; t++) {
            const int e = entry(u, t);
            int j;
            if constexpr (RESCORE) {
                const int jr = pr[t];
                j = u.ok && e < n_ent && jr >= 0 && jr < nb ? jr : -1;
            } else {
                j = u.ok && e < nb ? e : -1;
            }
            j_out[t] = j;
            ph_out[t] = table_row[j >= 0 ? j : 0];
        }
    };
    auto load_keys = [&](const int (&jj)[T], const int (&pp)[T], uint4 (&kc_out)[T],
                         uint32_t (&ks_out)[T], int (&vis_out)[T]) {
#pragma unroll
        for (int t = 0; t < T; t++) {
            const int j = jj[t], ph = pp[t];
            const bool ok = j >= 0 && ph >= 0 && (int64_t)ph < a.n_blocks;
            const uint8_t *blk = a.idx_cache + (int64_t)(ok ? ph : 0) * BYTES;
            kc_out[t] = *reinterpret_cast<const uint4 *>(blk + 16 * (min(g, G - 1) * kBlk + slot));
            const uint32_t sb = (uint32_t)(CODES + slot * G);
            ks_out[t] = *reinterpret_cast<const uint32_t *>(blk + (sb & ~3u)) >> (8 * (sb & 3u));
            vis_out[t] = ok ? j : -1;
        }
    };

    // the query of the current sequence: operand A lanes (head col, group g), head weights,
    // and the query's largest scale span
    int cur_b = -1;
    uint4 qa = make_uint4(0u, 0u, 0u, 0u);
    uint32_t qsc = 127u;
    float W[H];
    int qspan = 0;
    auto load_query_for = [&](int b) {
        const int hq = min(col, H - 1), gq = min(g, G - 1);
        uint4 c;
        uint32_t sc;
        if (a.q_f32) {
            QueryF32<H, G> F;
            load_query_f32<H, G>(F, a.q_f32 + (size_t)b * H * 32 * G);
            quant_query_group<H, G>(F, hq * G + gq, c, sc);
        } else {
            c = *reinterpret_cast<const uint4 *>(a.q_codes + ((size_t)b * H * G + hq * G + gq) * 16);
            sc = a.q_scales[(size_t)b * H * G + hq * G + gq];
        }
        const bool real = col < H && g < G;
        qa = real ? c : make_uint4(0u, 0u, 0u, 0u);
        qsc = real ? sc : 127u;
#pragma unroll
        for (int h = 0; h < H; h++) W[h] = a.w[(size_t)b * H + h];
        // the query's largest scale span: lanes (head, group) of the real groups
        int lo = real ? (int)sc : 255, hi = real ? (int)sc : 0;
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {  // over the groups of a head (lanes col + 16 i)
            lo = min(lo, __shfl_xor(lo, o, kWave));
            hi = max(hi, __shfl_xor(hi, o, kWave));
        }
        qspan = __builtin_amdgcn_readlane((int)wave_max_i(col < H ? hi - lo : 0), 63);
    };

    // one item: scores of its 64 positions, block maxima, its maximum; stored if it exists
    auto compute = [&](int k, const uint4 (&kk)[T], const uint32_t (&kw)[T], const int (&vv)[T]) {
        const ItemU u = item_u(k);
        if (!u.ok) return;  // uniform
        if (u.b != cur_b) {  // uniform: a new sequence's query
            load_query_for(u.b);
            cur_b = u.b;
        }
        const int L = __builtin_amdgcn_readfirstlane(sh_len[u.b]);
        const int n_lim = RESCORE ? nent_of(u.b) : nb_of(u.b);
        // exact single products for the whole item, unless some key's span is too wide
        int ksp = 0;
#pragma unroll
        for (int t = 0; t < T; t++) ksp = max(ksp, vv[t] >= 0 ? byte_span<G>(kw[t]) : 0);
        const bool single = __builtin_amdgcn_readlane((int)wave_max_i(ksp), 63) + qspan <= kSpanExactShared;
        float acc_p = -INFINITY;
#pragma unroll
        for (int t = 0; t < T; t++) {
            const uint4 kb = g < G ? kk[t] : make_uint4(0u, 0u, 0u, 0u);
            const uint32_t ksb = g < G ? (kw[t] >> (8 * g)) & 255u : 127u;
            f32x4_t d;
            if (single) {
                d = mfma_fp4_sk(qa, kb, qsc, ksb);
            } else {
                d = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g2 = 0; g2 < G; g2++) {
                    const f32x4_t tg = mfma_fp4_sk(qa, g == g2 ? kb : make_uint4(0u, 0u, 0u, 0u), qsc, ksb);
#pragma unroll
                    for (int e = 0; e < 4; e++) d[e] = d[e] + tg[e];
                }
            }
            // lane (position col, g): heads 4g .. 4g+3; s = fma(w_{H-1}, r_{H-1}, ... fma(w_0, r_0, +0))
            float sc;
            if constexpr (H <= 4) {
                sc = 0.0f;
#pragma unroll
                for (int e = 0; e < H; e++) sc = __builtin_fmaf(W[e], relu_bits(d[e]), sc);
            } else {
                float lo = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; e++) lo = __builtin_fmaf(W[e], relu_bits(d[e]), lo);
                sc = __shfl(lo, max(lane - 16, 0), kWave);  // heads 0..3 of the position
#pragma unroll
                for (int e = 0; e < 4; e++) sc = __builtin_fmaf(W[4 + e], relu_bits(d[e]), sc);
            }
            const int jv = vv[t];
            const float val = jv >= 0 && jv * kBlk + slot < L ? sc : -INFINITY;
            // position 16t + c of the item into lane 16t + c
            const float v = __shfl(val, (H > 4 ? 16 : 0) + col, kWave);
            acc_p = g == t ? v : acc_p;
        }
        // block maxima (every lane of an 8-lane group), the item's maximum into lane 63
        const float m = block_max_lanes<1>(acc_p);
        const float bmax = __shfl(m, 8 * (lane & 7), kWave);
        const float g63 = blocks_to_lane63<1>(m);
        float *ps_row = RESCORE ? a.poolsc + (int64_t)u.b * a.K_blk * kBlk : a.pscore + (int64_t)u.b * a.maxb * kBlk;
        float *pb_row = RESCORE ? a.poolbmax + (int64_t)u.b * a.K_blk : a.bscore + (int64_t)u.b * a.bstride;
        if ((RESCORE || a.pscore) && u.e0 + lane / kBlk < n_lim) ps_row[(int64_t)u.e0 * kBlk + lane] = acc_p;
        if ((RESCORE || a.bscore) && lane < kBlk && u.e0 + lane < n_lim) pb_row[u.e0 + lane] = bmax;
        if (!RESCORE && a.gmax && lane == kWave - 1) a.gmax[(int64_t)u.b * a.ngmax + u.e0 / kItemBlocks] = g63;
    };

    // prologue: pool entries of items 0..2, table entries of items 0 and 1, keys of item 0
    load_pool(0, praw[0]);
    load_pool(1, praw[1]);
    load_pool(2, praw[2]);
    load_table(0, praw[0], lj[0], lph[0]);
    load_table(1, praw[1], lj[1], lph[1]);
    load_keys(lj[0], lph[0], kc[0], ksw[0], vis[0]);
    for (int k0 = 0; k0 < n_items; k0 += 4) {
#pragma unroll
        for (int st = 0; st < 4; st++) {
            const int k = k0 + st;
            load_pool(k + 3, praw[(st + 3) % 4]);
            load_table(k + 2, praw[(st + 2) % 4], lj[st % 2], lph[st % 2]);
            load_keys(lj[(st + 1) % 2], lph[(st + 1) % 2], kc[(st + 1) % 2], ksw[(st + 1) % 2],
                      vis[(st + 1) % 2]);
            compute(k, kc[st % 2], ksw[st % 2], vis[st % 2]);
        }
    }
}

// ------------------------------------------------------------------ dispatch

typedef void (*ScanFn)(dim3, size_t, hipStream_t, const ScanArgs &);
struct KernSet {
    ScanFn scan, rescore;
};

template <int H, int G>
bool off32(const ScanArgs &a) {
    constexpr int64_t BYTES = kBlk * H * 17 * G;
    return a.n_blocks * BYTES <= ((int64_t)1 << 32);
}
// Layouts whose scan takes the global append without spilling registers (with four groups
// per head and two or more heads the append's key and latent registers do not fit beside the
// pipeline's; those layouts append in a launch of their own before the scan).
constexpr bool fuse_append(int H, int G) { return G <= 2 || H == 1; }

template <int H, int G>
void launch_scan(dim3 g, size_t sh, hipStream_t s, const ScanArgs &a) {
    const bool o32 = off32<H, G>(a);
    if constexpr (fuse_append(H, G)) {
        if (a.new_key) {  // the fused append keeps its own registers out of the plain scan
            if (o32) k_scan<H, G, false, true, true><<<g, kScanThreads, sh, s>>>(a);
            else k_scan<H, G, false, false, true><<<g, kScanThreads, sh, s>>>(a);
            return;
        }
    }
    if (o32) k_scan<H, G, false, true, false><<<g, kScanThreads, sh, s>>>(a);
    else k_scan<H, G, false, false, false><<<g, kScanThreads, sh, s>>>(a);
}
template <int H, int G>
void launch_rescore(dim3 g, size_t sh, hipStream_t s, const ScanArgs &a) {
    if (off32<H, G>(a)) k_scan<H, G, true, true, false><<<g, kScanThreads, sh, s>>>(a);
    else k_scan<H, G, true, false, false><<<g, kScanThreads, sh, s>>>(a);
}

template <int H, int G>
void launch_scan_shared(dim3 g, size_t sh, hipStream_t s, const ScanArgs &a) {
    k_scan_shared<H, G, false><<<g, kScanThreads, sh, s>>>(a);
}
template <int H, int G>
void launch_rescore_shared(dim3 g, size_t sh, hipStream_t s, const ScanArgs &a) {
    k_scan_shared<H, G, true><<<g, kScanThreads, sh, s>>>(a);
}

bool pick_shared(int H, int dI, KernSet *ks) {
    const int G = dI / 32;
#define CSA2_CASE(h, g) \
    if (H == h && G == g) { *ks = {launch_scan_shared<h, g>, launch_rescore_shared<h, g>}; return true; }
    CSA2_CASE(1, 1) CSA2_CASE(1, 2) CSA2_CASE(1, 4)
    CSA2_CASE(2, 1) CSA2_CASE(2, 2) CSA2_CASE(2, 4)
    CSA2_CASE(4, 1) CSA2_CASE(4, 2) CSA2_CASE(4, 4)
    CSA2_CASE(8, 1) CSA2_CASE(8, 2) CSA2_CASE(8, 4)
#undef CSA2_CASE
    return false;
}

bool pick(int H, int dI, KernSet *ks) {
    const int G = dI / 32;
#define CSA2_CASE(h, g) \
    if (H == h && G == g) { *ks = {launch_scan<h, g>, launch_rescore<h, g>}; return true; }
    CSA2_CASE(1, 1) CSA2_CASE(1, 2) CSA2_CASE(1, 4)
    CSA2_CASE(2, 1) CSA2_CASE(2, 2) CSA2_CASE(2, 4)
    CSA2_CASE(4, 1) CSA2_CASE(4, 2) CSA2_CASE(4, 4)
    CSA2_CASE(8, 1) CSA2_CASE(8, 2) CSA2_CASE(8, 4)
#undef CSA2_CASE
    return false;
}

// The kernels of a configuration: per-head keys or one shared key per position.
bool pick_cfg(const csa2_config *c, KernSet *ks) {
    return c->shared_key ? pick_shared(c->n_idx_heads, c->idx_dim, ks)
                         : pick(c->n_idx_heads, c->idx_dim, ks);
}

int check_index_cfg(const csa2_config *c) {
    if (!c) return CSA2_ERR_INVALID;
    if (c->n_idx_heads <= 0 || c->idx_dim <= 0 || c->idx_dim % 32 || c->kv_dim <= 0 ||
        c->kv_dim % 32 || c->n_q_heads <= 0 || c->swa_window < 0 || c->pool_blocks <= 0 ||
        c->topk <= 0 || (int64_t)c->topk > 8 * (int64_t)c->pool_blocks ||
        (c->shared_key != 0 && c->shared_key != 1))
        return CSA2_ERR_INVALID;
    if (c->pool_blocks > CSA2_MAX_POOL_BLOCKS) return CSA2_ERR_UNSUPPORTED;
    KernSet ks;
    if (!pick_cfg(c, &ks)) return CSA2_ERR_UNSUPPORTED;
    return CSA2_OK;
}

// Row stride of the group maxima (rounded to 4 floats for 16-byte loads).
int ngmax_of(int maxb) { return (((maxb + kItemBlocks - 1) / kItemBlocks) + 3) & ~3; }

}  // namespace csa2

using namespace csa2;

namespace {

int check_cfg(const csa2_config *c) { return check_index_cfg(c); }

int launched() { return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

ScanArgs scan_args(const csa2_config *c, const uint8_t *qc, const uint8_t *qs, const float *w,
                   const uint8_t *idx, int64_t n_blocks, const int32_t *table, int32_t maxb,
                   const int32_t *ctx, int32_t B, const float *q_f32 = nullptr) {
    ScanArgs a{};
    a.q_codes = qc;
    a.q_scales = qs;
    a.q_f32 = q_f32;
    a.w = w;
    a.idx_cache = idx;
    a.n_blocks = n_blocks;
    a.table = table;
    a.maxb = maxb;
    a.ctx_len = ctx;
    a.B = B;
    a.ngmax = ngmax_of(maxb);
    a.bstride = maxb;
    a.K_blk = c->pool_blocks;
    return a;
}

int scan_grid(int64_t items) {
    const int64_t wgs = (items + kScanWaves - 1) / kScanWaves;
    return (int)std::max<int64_t>(1, std::min<int64_t>(wgs, kScanGridMax));
}

size_t prefix_bytes(int B) { return sizeof(int32_t) * (3 * (size_t)B + 1); }

}  // namespace

// Workspace of the index calls: position scores, block maxima, group maxima (Full) and
// pool scores (Reindex).  No initialisation is needed.
namespace csa2 {

int sel2_workgroups(const csa2_config *c, int32_t maxb) {
    // below 2 K_blk groups most groups hold candidates and the last workgroup would select
    // from nearly every block: the one-workgroup selection is faster there (measured at
    // 64K-128K contexts; the two-phase form wins from 256K on)
    const int ng = (maxb + kItemBlocks - 1) / kItemBlocks;
    if (ng < 2 * c->pool_blocks || c->pool_blocks < c->topk) return 0;
    const int nw = (ng + kSel2GroupsPerW - 1) / kSel2GroupsPerW;
    return nw <= kSel2MaxW ? nw : 0;
}

struct WsIdx {
    size_t pscore, bscore, gmax, poolsc, poolbmax;
    size_t cand, mu_sc, mu_blk, cnt, arrive;  // two-phase Full selection (nw > 0)
    int nw;
    size_t total;
};
static WsIdx ws_idx(const csa2_config *c, int B, int maxb) {
    const int K_blk = c->pool_blocks;
    WsIdx w;
    size_t o = 0;
    w.pscore = o;  o = align256(o + sizeof(float) * (size_t)B * maxb * kBlk);
    w.bscore = o;  o = align256(o + sizeof(float) * (size_t)B * ngmax_of(maxb) * kItemBlocks);
    w.gmax = o;    o = align256(o + sizeof(float) * (size_t)B * ngmax_of(maxb));
    w.poolsc = o;  o = align256(o + sizeof(float) * (size_t)B * K_blk * kBlk);
    w.poolbmax = o; o = align256(o + sizeof(float) * (size_t)B * K_blk);
    w.nw = sel2_workgroups(c, maxb);
    const size_t regs = (size_t)B * w.nw;
    w.cand = o;    o = align256(o + sizeof(uint2) * regs * kSel2GroupsPerW * kItemBlocks);
    w.mu_sc = o;   o = align256(o + sizeof(float) * regs * kSel2MuCap * kBlk);
    w.mu_blk = o;  o = align256(o + sizeof(int32_t) * regs * kSel2MuCap);
    w.cnt = o;     o = align256(o + sizeof(int32_t) * regs * 2);
    w.arrive = o;  o = align256(o + sizeof(int32_t) * (w.nw ? (size_t)B : 0));
    w.total = o;
    return w;
}
}  // namespace csa2

extern "C" int csa2_layout(const csa2_config *c, csa2_layout_info *out) {
    if (!c || !out || c->n_idx_heads <= 0 || c->idx_dim <= 0 || c->idx_dim % 32 ||
        c->kv_dim <= 0 || c->kv_dim % 32 || (c->shared_key != 0 && c->shared_key != 1))
        return CSA2_ERR_INVALID;
    out->idx_block_bytes = (size_t)kBlk * key_heads(c) * (c->idx_dim / 2 + c->idx_dim / 32);
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
        *bytes = ws_idx(c, batch, maxb).total;
        return CSA2_OK;
    }
    if (op == CSA2_OP_INDEX_PREFILL) {
        const int st = check_cfg(c);
        if (st) return st;
        *bytes = prefill_ws_bytes(c, batch, maxb);
        return CSA2_OK;
    }
    if (op == CSA2_OP_SPARSE_ATTN) {
        if (const int st = attn_cfg_status(c)) return st;
        *bytes = ws_attn(batch, c->n_q_heads, c->kv_dim,
                         attn_plan(batch, c->n_q_heads, c->topk, c->swa_window).nsplit).total;
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
    case CSA2_ERR_SCRATCH: return "shape needs more than the 16 MiB static scratch";
    default: return "unknown status";
    }
}

namespace {

#define CSA2_CHECK_INDEX_ARGS()                                                              \
    do {                                                                                    \
        const int st_ = check_cfg(c);                                                       \
        if (st_) return st_;                                                                \
        if (((!q_codes || !q_scales) && !q_f32) || !w || !idx_cache || n_blocks <= 0 ||     \
            !block_table || maxb <= 0 || !ctx_len || batch < 0)                             \
            return CSA2_ERR_INVALID;                                                        \
        if (batch > kMaxBatch) return CSA2_ERR_UNSUPPORTED;                                 \
    } while (0)

SelectArgs select_args(const csa2_config *c, const int32_t *ctx, int32_t maxb, int32_t B,
                       void *ws) {
    const WsIdx L = ws_idx(c, B, maxb);
    uint8_t *base = (uint8_t *)ws;
    SelectArgs s{};
    s.ctx_len = ctx;
    s.maxb = maxb;
    s.B = B;
    s.K_blk = c->pool_blocks;
    s.k = c->topk;
    s.pscore = (const float *)(base + L.pscore);
    s.bscore = (const float *)(base + L.bscore);
    s.ps_b = (int64_t)maxb * kBlk;
    s.ps_j = kBlk;
    s.bs_b = (int64_t)ngmax_of(maxb) * kItemBlocks;
    s.bs_g = kItemBlocks;
    s.gmax = (const float *)(base + L.gmax);
    s.ngmax = ngmax_of(maxb);
    s.poolsc = (const float *)(base + L.poolsc);
    s.poolbmax = (const float *)(base + L.poolbmax);
    s.sel2.nw = L.nw;
    if (L.nw) {
        s.sel2.cand = (uint2 *)(base + L.cand);
        s.sel2.mu_sc = (float *)(base + L.mu_sc);
        s.sel2.mu_blk = (int32_t *)(base + L.mu_blk);
        s.sel2.cnt = (int32_t *)(base + L.cnt);
        s.sel2.arrive = (int32_t *)(base + L.arrive);
    }
    return s;
}

// The Full selection: two-phase where it serves, else one workgroup per sequence.
int launch_full_select(const SelectArgs &s, hipStream_t stream) {
    return s.sel2.nw ? launch_select_full2(s, stream) : launch_select(s, false, stream);
}

}  // namespace

extern "C" int csa2_index_scores(const csa2_config *c, const uint8_t *q_codes,
                                 const uint8_t *q_scales, const float *w,
                                 const uint8_t *idx_cache, int64_t n_blocks,
                                 const int32_t *block_table, int32_t maxb,
                                 const int32_t *ctx_len, int32_t batch, float *scores,
                                 float *block_scores, hipStream_t stream) {
    const float *q_f32 = nullptr;
    CSA2_CHECK_INDEX_ARGS();
    if (batch == 0 || (!scores && !block_scores)) return CSA2_OK;
    KernSet ks;
    pick_cfg(c, &ks);
    ScanArgs a = scan_args(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table, maxb,
                           ctx_len, batch);
    a.pscore = scores;
    a.bscore = block_scores;
    ks.scan(dim3(scan_grid((int64_t)batch * ngmax_of(maxb))), prefix_bytes(batch), stream, a);
    return launched();
}

extern "C" int csa2_index_full_scan(const csa2_config *c, const uint8_t *q_codes,
                                    const uint8_t *q_scales, const float *w,
                                    const uint8_t *idx_cache, int64_t n_blocks,
                                    const int32_t *block_table, int32_t maxb,
                                    const int32_t *ctx_len, int32_t batch, void *ws,
                                    size_t ws_bytes, hipStream_t stream) {
    const float *q_f32 = nullptr;
    CSA2_CHECK_INDEX_ARGS();
    if (!ws) return CSA2_ERR_INVALID;
    const WsIdx L = ws_idx(c, batch, maxb);
    if (ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    KernSet ks;
    pick_cfg(c, &ks);
    ScanArgs a = scan_args(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table, maxb,
                           ctx_len, batch);
    uint8_t *base = (uint8_t *)ws;
    a.pscore = (float *)(base + L.pscore);
    a.bscore = (float *)(base + L.bscore);
    a.bstride = ngmax_of(maxb) * kItemBlocks;
    a.gmax = (float *)(base + L.gmax);
    a.arrive = L.nw ? (int32_t *)(base + L.arrive) : nullptr;
    ks.scan(dim3(scan_grid((int64_t)batch * ngmax_of(maxb))), prefix_bytes(batch), stream, a);
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
    const float *q_f32 = nullptr;
    CSA2_CHECK_INDEX_ARGS();
    if (!pool_blocks || !pool_len || !topk || !topk_len || !ws) return CSA2_ERR_INVALID;
    if (ws_bytes < ws_idx(c, batch, maxb).total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    SelectArgs s = select_args(c, ctx_len, maxb, batch, ws);
    s.pool_blocks = pool_blocks;
    s.pool_len = pool_len;
    s.topk = topk;
    s.topk_len = topk_len;
    return launch_full_select(s, stream);
}

extern "C" int csa2_index_full(const csa2_config *c, const uint8_t *q_codes,
                               const uint8_t *q_scales, const float *w, const uint8_t *idx_cache,
                               int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                               const int32_t *ctx_len, int32_t batch, int32_t *pool_blocks,
                               int32_t *pool_len, int32_t *topk, int32_t *topk_len, void *ws,
                               size_t ws_bytes, hipStream_t stream) {
    const float *q_f32 = nullptr;
    CSA2_CHECK_INDEX_ARGS();
    if (!pool_blocks || !pool_len || !topk || !topk_len || !ws) return CSA2_ERR_INVALID;
    int st = csa2_index_full_scan(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table,
                                  maxb, ctx_len, batch, ws, ws_bytes, stream);
    if (st) return st;
    return csa2_index_full_finish(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table,
                                  maxb, ctx_len, batch, pool_blocks, pool_len, topk, topk_len,
                                  ws, ws_bytes, stream);
}

namespace csa2 {

int index_full_append(const csa2_config *c, const float *latent, const float *idx_k,
                      const uint8_t *q_codes, const uint8_t *q_scales, const float *q_f32,
                      const float *w, uint8_t *kv_cache, uint8_t *idx_cache, int64_t n_blocks,
                      const int32_t *block_table, int32_t maxb, const int32_t *ctx_len,
                      int32_t batch, int32_t *pool_blocks, int32_t *pool_len, int32_t *topk,
                      int32_t *topk_len, void *ws, size_t ws_bytes, hipStream_t stream) {
    CSA2_CHECK_INDEX_ARGS();
    if (!idx_k || (latent && !kv_cache) || !pool_blocks || !pool_len || !topk || !topk_len || !ws)
        return CSA2_ERR_INVALID;
    if (latent && c->kv_dim != kAppD) return CSA2_ERR_UNSUPPORTED;
    const WsIdx L = ws_idx(c, batch, maxb);
    if (ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    const bool fused = !c->shared_key && fuse_append(c->n_idx_heads, c->idx_dim / 32);
    if (!fused) {
        const int st = launch_append_global(c, latent, idx_k, block_table, maxb, n_blocks,
                                            ctx_len, -1, batch, 1, kv_cache, idx_cache, stream);
        if (st) return st;
    }
    KernSet ks;
    pick_cfg(c, &ks);
    ScanArgs a = scan_args(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table, maxb,
                           ctx_len, batch, q_f32);
    uint8_t *base = (uint8_t *)ws;
    a.pscore = (float *)(base + L.pscore);
    a.bscore = (float *)(base + L.bscore);
    a.bstride = ngmax_of(maxb) * kItemBlocks;
    a.gmax = (float *)(base + L.gmax);
    a.arrive = L.nw ? (int32_t *)(base + L.arrive) : nullptr;
    if (fused) {
        a.new_key = idx_k;
        a.new_lat = latent;
        a.idx_w = idx_cache;
        a.kv_w = kv_cache;
    }
    ks.scan(dim3(scan_grid((int64_t)batch * ngmax_of(maxb))), prefix_bytes(batch), stream, a);
    const int st = launched();
    if (st) return st;
    SelectArgs sa = select_args(c, ctx_len, maxb, batch, ws);
    sa.pool_blocks = pool_blocks;
    sa.pool_len = pool_len;
    sa.topk = topk;
    sa.topk_len = topk_len;
    return launch_full_select(sa, stream);
}

int index_reindex(const csa2_config *c, const uint8_t *q_codes, const uint8_t *q_scales,
                  const float *q_f32, const float *w, const uint8_t *idx_cache, int64_t n_blocks,
                  const int32_t *block_table, int32_t maxb, const int32_t *ctx_len, int32_t batch,
                  const int32_t *pool_blocks, const int32_t *pool_len, int32_t *topk,
                  int32_t *topk_len, void *ws, size_t ws_bytes, hipStream_t stream) {
    CSA2_CHECK_INDEX_ARGS();
    if (!pool_blocks || !pool_len || !topk || !topk_len || !ws) return CSA2_ERR_INVALID;
    const WsIdx L = ws_idx(c, batch, maxb);
    if (ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
    if (batch == 0) return CSA2_OK;
    KernSet ks;
    pick_cfg(c, &ks);
    ScanArgs a = scan_args(c, q_codes, q_scales, w, idx_cache, n_blocks, block_table, maxb,
                           ctx_len, batch, q_f32);
    a.pool = pool_blocks;
    a.pool_len = pool_len;
    a.poolsc = (float *)((uint8_t *)ws + L.poolsc);
    a.poolbmax = (float *)((uint8_t *)ws + L.poolbmax);
    const int64_t items = (int64_t)batch * ((c->pool_blocks + kItemBlocks - 1) / kItemBlocks);
    ks.rescore(dim3(scan_grid(items)), prefix_bytes(batch), stream, a);
    const int st = launched();
    if (st) return st;
    SelectArgs s = select_args(c, ctx_len, maxb, batch, ws);
    s.pool_blocks = const_cast<int32_t *>(pool_blocks);
    s.pool_len = const_cast<int32_t *>(pool_len);
    s.topk = topk;
    s.topk_len = topk_len;
    return launch_select(s, true, stream);
}

}  // namespace csa2

extern "C" int csa2_index_full_append(const csa2_config *c, const float *latent,
                                      const float *idx_k, const uint8_t *q_codes,
                                      const uint8_t *q_scales, const float *w, uint8_t *kv_cache,
                                      uint8_t *idx_cache, int64_t n_blocks,
                                      const int32_t *block_table, int32_t maxb,
                                      const int32_t *ctx_len, int32_t batch, int32_t *pool_blocks,
                                      int32_t *pool_len, int32_t *topk, int32_t *topk_len,
                                      void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!q_codes || !q_scales) return CSA2_ERR_INVALID;
    return index_full_append(c, latent, idx_k, q_codes, q_scales, nullptr, w, kv_cache, idx_cache,
                             n_blocks, block_table, maxb, ctx_len, batch, pool_blocks, pool_len,
                             topk, topk_len, ws, ws_bytes, stream);
}

extern "C" int csa2_index_reindex(const csa2_config *c, const uint8_t *q_codes,
                                  const uint8_t *q_scales, const float *w,
                                  const uint8_t *idx_cache, int64_t n_blocks,
                                  const int32_t *block_table, int32_t maxb,
                                  const int32_t *ctx_len, int32_t batch,
                                  const int32_t *pool_blocks, const int32_t *pool_len,
                                  int32_t *topk, int32_t *topk_len, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
    if (!q_codes || !q_scales) return CSA2_ERR_INVALID;
    return index_reindex(c, q_codes, q_scales, nullptr, w, idx_cache, n_blocks, block_table, maxb,
                         ctx_len, batch, pool_blocks, pool_len, topk, topk_len, ws, ws_bytes,
                         stream);
}
