// csa2_prefill.hip -- the indexer of a prefill chunk: n_q consecutive query tokens of one
// sequence, query i at position t_i = q_pos0 + i, each scoring the positions p <= t_i and
// selecting its own pool and top-k exactly as a Full-mode decode step on that prefix
// (dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心": the Full layer's scan, pool
// of 2048 blocks of 8 and top-512; the per-layer kernel counts quoted there cover prefill).
//
// With many queries against the same keys the score is a dense contraction, so the products
// run on the gfx950 scaled FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4): per head
// one 16 positions x 16 queries tile consumes the head's 128 (4 groups of 32) FP4 elements,
// each lane carrying one 32-group and its E8M0 scale.  The library's score definition is a
// fixed-order fp32 sum of exact per-group terms t_g = N_g * 2^(E_g - 2); the matrix core
// instead adds the scaled group dot products in an undisclosed order.  Both give the exact
// sum D_h whenever every partial sum is representable: with |N_g| <= 4608 < 2^13, the four
// terms are multiples of 2^(min E - 2) below 2^(max E - 2 + 15), so an exponent span
// max_g E_g - min_g E_g <= 9 keeps every partial inside 24 bits.  Tiles whose key and query
// scale spans could exceed that take an exact path instead: one matrix instruction per
// group (the other groups' operands zeroed) and the fp32 group sum in the defined order.
// The epilogue (ReLU, fma chain over heads in head order, causal mask, block and group
// maxima) runs on the vector ALUs and writes what the Full-mode selection reads.
//
// With more than 16 queries no position score is stored by the scoring pass: it keeps the
// block and group maxima, the selection takes the pools from them, and a second pass
// recomputes only the scores the top-k can need (the pool blocks whose maximum reaches the
// k-th largest pool block maximum, about k per query), block by block for the queries that
// flagged each block.
//
// Kernels:
//   k_prefill_span    per logical block: the largest exponent span of any key head vector.
//   k_prefill<H,G,.,MODE>  a workgroup = 128 queries x 2048 positions; keys staged through
//                     LDS in stages of 8 blocks (double-buffered), queries and head weights
//                     held in registers, 4 waves x 2 query tiles of 16.  MODE: scores and
//                     maxima (at most 16 queries), or maxima only.
//   k_prefill_rescore (more than 16 queries) one workgroup per stage of 8 blocks: the
//                     flagged blocks' scores for the queries that flagged them.
//   k_select          (at most 16 queries, shared with Full mode) one workgroup per query;
//   k_select_pf_pool / k_select_pf_topk  (more queries) the two selection phases around
//                     the rescoring pass.
#include <algorithm>

#include "csa2_block.h"
#include "csa2_select.h"

namespace csa2 {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr int kPfNQ = 2;                          // 16-query tiles per wave
constexpr int kPfStageBlocks = 8;                 // blocks per LDS stage (one group maximum)
constexpr int kPfChunkStages = 32;                // stages per workgroup (2048 positions)
constexpr int kPfChunkBlocks = kPfChunkStages * kPfStageBlocks;
constexpr int kSpanExact = 9;                     // largest exact exponent span
constexpr int kBlockPad = 128;                    // LDS bytes between staged blocks

// MODE: kPfAll, scores and maxima (at most 16 queries); kPfMaxima, block and group maxima
// only.
constexpr int kPfAll = 0, kPfMaxima = 1;

// A scoring workgroup: 4 waves, each holding kPfNQ query tiles of 16 and sharing the staged
// keys (two workgroups per CU, whose waves share SIMDs without a common barrier).
template <int MODE>
struct PfShape {
    static constexpr int waves = 4;
    static constexpr int threads = waves * kWave;
    static constexpr int qt = waves * kPfNQ * 16;  // queries per workgroup
};

struct PrefillArgs {
    const uint8_t *q_codes;   // [n_q][H*G*16]
    const uint8_t *q_scales;  // [n_q][H*G]
    const float *w;           // [n_q][H]
    int32_t q_pos0, n_q;
    const uint8_t *idx_cache;
    int64_t n_blocks;
    const int32_t *table;  // one row of maxb entries
    int32_t maxb;
    int32_t nb;            // logical blocks touched: ceil((q_pos0 + n_q) / 8)
    uint8_t *kspan;        // [round8(nb)]
    float *pscore;         // block-major: (q, p) at ((p/8)*n_q + q)*8 + p%8
    float *bscore;         // group-major: (q, j) at ((j/8)*n_q + q)*8 + j%8
    float *gmax;           // [n_q][ngmax]
    int32_t ngmax;
    uint32_t *need;        // flags of the blocks to rescore: word w of chunk c, query q at (c*8 + w)*n_q + q
    uint8_t *qspan;        // [n_q] largest scale-exponent span of any head vector of the query
    int32_t *arrive;       // [n_q] arrivals of the two-phase selection (null: not used)
    int32_t n_qt, n_pc;    // query tiles, position chunks
};

__device__ __forceinline__ int64_t phys_block(const PrefillArgs &a, int j) {
    if (j >= a.nb) return -1;
    const int32_t ph = a.table[j];
    return (ph >= 0 && ph < a.n_blocks) ? ph : -1;
}

// Key span of physical block ph (0 when absent): max over the 8 positions and H heads of
// (largest - smallest E8M0 code among the head's G groups), from its scale bytes
// (position-major, then head, then group), read as dwords.
template <int H, int G>
__device__ __forceinline__ int block_span(const PrefillArgs &a, int64_t ph) {
    constexpr int CODES = kBlk * H * 16 * G;
    constexpr int BYTES = CODES + kBlk * H * G;
    constexpr int NW = kBlk * H * G / 4;
    if (ph < 0) return 0;
    const uint32_t *sw = reinterpret_cast<const uint32_t *>(a.idx_cache + ph * BYTES + CODES);
    uint32_t w[NW];
#pragma unroll
    for (int i = 0; i < NW; i++) w[i] = sw[i];
    int span = 0;
#pragma unroll
    for (int sh = 0; sh < kBlk * H; sh++) {
        int lo = 255, hi = 0;
#pragma unroll
        for (int g = 0; g < G; g++) {
            const int k = sh * G + g;
            const int e = (int)((w[k >> 2] >> (8 * (k & 3))) & 0xffu);
            lo = min(lo, e);
            hi = max(hi, e);
        }
        span = max(span, hi - lo);
    }
    return span;
}

// kspan[j] = max over the 8 positions and H heads of block j of
// (largest - smallest E8M0 code among the head's G groups); 0 for absent blocks.
template <int H, int G>
__global__ __launch_bounds__(256) void k_prefill_span(PrefillArgs a) {
    constexpr int CODES = kBlk * H * 16 * G;
    constexpr int BYTES = CODES + kBlk * H * G;
    const int gid = blockIdx.x * 256 + threadIdx.x;  // (block, slot)
    const int j = gid / kBlk, s = gid % kBlk;
    const int nbr = (a.nb + kBlk - 1) / kBlk * kBlk;
    int span = 0;
    const int64_t ph = j < a.nb ? phys_block(a, j) : -1;
    if (ph >= 0) {
        const uint8_t *sc = a.idx_cache + ph * BYTES + CODES + s * H * G;
#pragma unroll
        for (int h = 0; h < H; h++) {
            int lo = 255, hi = 0;
#pragma unroll
            for (int g = 0; g < G; g++) {
                const int e = sc[h * G + g];
                lo = min(lo, e);
                hi = max(hi, e);
            }
            span = max(span, hi - lo);
        }
    }
    span = max(span, __shfl_xor(span, 1, kWave));
    span = max(span, __shfl_xor(span, 2, kWave));
    span = max(span, __shfl_xor(span, 4, kWave));
    if (s == 0 && j < nbr) a.kspan[j] = (uint8_t)span;
}

// One key stage in LDS: the code bytes of 8 blocks (rows of H 16-byte chunks, chunk h of
// row R stored at position h ^ (R mod H), blocks kBlockPad apart, the whole region a
// multiple of 1 KB) and their scale bytes (a multiple of 256 B).
template <int H, int G>
struct PfStage {
    static constexpr int CODES = kBlk * H * 16 * G;  // code bytes per block
    static constexpr int SCB = kBlk * H * G;         // scale bytes per block
    static constexpr int BSTR = CODES + kBlockPad;   // LDS bytes per staged block
    static constexpr int SLOTS = (kPfStageBlocks * BSTR / 16 + kWave - 1) / kWave * kWave;
    static constexpr int SDW = (kPfStageBlocks * SCB / 4 + kWave - 1) / kWave * kWave;
    __align__(16) uint8_t codes[SLOTS * 16];
    __align__(16) uint32_t scales[SDW];
};

// Block-table entries and key spans of a workgroup's position chunk, staged once in LDS so
// that no per-stage lookup waits on global memory.
struct __align__(16) PfMeta {
    int32_t phys[kPfChunkBlocks];  // physical block, -1 when absent
    uint8_t kspan[kPfChunkBlocks];
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Byte offset, inside a block's codes, of the 16-byte chunk that lane `lane` of a 1 KB LDS
// DMA row fetches: LDS slot c holds global chunk (c/H)*H + ((c%H) ^ ((c/H) mod H)); for a row
// starting at a multiple of 64 slots, (c/H) mod H depends on the lane only.
template <int H>
__device__ __forceinline__ uint32_t pf_swizzle16(int lane) {
    const int hs = lane % H, row = lane / H;
    return (uint32_t)((lane - hs + (hs ^ (row & (H - 1)))) * 16);
}

// Stage the keys of blocks jrel .. jrel+7 of the chunk into dst with LDS DMA
// (global_load_lds): one instruction moves 64 lanes x 16 (or 4) bytes into 1 KB (256 B) of
// consecutive LDS, lane i to byte 16*i (4*i), so each lane fetches the global chunk that the
// swizzled layout puts at its slot.  Absent blocks read physical block 0.
// When a block's codes and scale bytes are whole rows (at least 8 heads x 32-groups), every
// row lies inside one block: its physical block is wave-uniform (a scalar base) and each lane
// adds a fixed offset (sw16, from pf_swizzle16).  Otherwise rows span blocks and each lane
// looks its block up.
template <int H, int G, int kPfWaves>
__device__ __forceinline__ void pf_dma(const PrefillArgs &a, const PfMeta &meta, int jrel,
                                       PfStage<H, G> &dst, uint32_t sw16) {
    using S = PfStage<H, G>;
    constexpr int BYTES = S::CODES + S::SCB;
    constexpr int CPB = S::CODES / 16;  // code chunks per block
    constexpr int SPB = S::BSTR / 16;   // LDS slots per staged block
    constexpr int DPB = S::SCB / 4;     // scale dwords per block
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    if constexpr (S::CODES % 1024 == 0 && S::SCB % 256 == 0) {
        // wave w stages blocks BPW*w .. BPW*w + BPW - 1 of the stage, all of their rows
        constexpr int CR = S::CODES / 1024, SR = S::SCB / 256;
        constexpr int BPW = kPfStageBlocks / kPfWaves;
        static_assert(BPW * kPfWaves == kPfStageBlocks, "whole blocks per wave");
#pragma unroll
        for (int i = 0; i < BPW; i++) {
            const int blk = BPW * wave + i;
            const int32_t ph = __builtin_amdgcn_readfirstlane(meta.phys[jrel + blk]);
            const uint8_t *base = a.idx_cache + (int64_t)(ph >= 0 ? ph : 0) * BYTES;
#pragma unroll
            for (int k = 0; k < CR; k++)
                __builtin_amdgcn_global_load_lds(base + k * 1024 + sw16,
                                                 (lds_ptr_t)(dst.codes + blk * S::BSTR + k * 1024), 16, 0, 0);
#pragma unroll
            for (int k = 0; k < SR; k++)
                __builtin_amdgcn_global_load_lds(base + S::CODES + k * 256 + lane * 4,
                                                 (lds_ptr_t)(dst.scales + (blk * S::SCB + k * 256) / 4), 4, 0, 0);
        }
        return;
    }
#pragma unroll
    for (int r = wave; r < S::SLOTS / kWave; r += kPfWaves) {
        const int slot = kWave * r + lane;
        const int blk = min(slot / SPB, kPfStageBlocks - 1), c = slot - blk * SPB;
        int chunk = 0;
        if (c < CPB) {
            const int row = c / H, hs = c % H;
            chunk = row * H + (hs ^ (row & (H - 1)));
        }
        const int64_t ph = meta.phys[jrel + blk];
        const uint8_t *src = a.idx_cache + (ph >= 0 ? ph : 0) * BYTES + chunk * 16;
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst.codes + kWave * 16 * r), 16, 0, 0);
    }
#pragma unroll
    for (int r = wave; r < S::SDW / kWave; r += kPfWaves) {
        const int d = kWave * r + lane;
        const int blk = min(d / DPB, kPfStageBlocks - 1), k = min(d - blk * DPB, DPB - 1);
        const int64_t ph = meta.phys[jrel + blk];
        const uint8_t *src = a.idx_cache + (ph >= 0 ? ph : 0) * BYTES + S::CODES + k * 4;
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst.scales + kWave * r), 4, 0, 0);
    }
}

// One 16x16x128 FP4 tile product; the scale of operand A is byte 0 of sa, that of B byte
// SB of sb (operand selects are immediates).
template <int SB>
__device__ __forceinline__ f32x4_t mfma_fp4(const uint4 &a, const uint4 &b, uint32_t sa, uint32_t sb) {
    const v8i_t av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    // formats 4/4: both operands FP4 E2M1
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 4, 0, (int)sa, SB, (int)sb);
}

// mfma_fp4 with the B scale in byte i (0..3, unrolled) of sb.
__device__ __forceinline__ f32x4_t mfma_pick(const uint4 &a, const uint4 &b, uint32_t sa, uint32_t sb, int i) {
    switch (i) {
    case 0: return mfma_fp4<0>(a, b, sa, sb);
    case 1: return mfma_fp4<1>(a, b, sa, sb);
    case 2: return mfma_fp4<2>(a, b, sa, sb);
    default: return mfma_fp4<3>(a, b, sa, sb);
    }
}

// max(x, +0) exactly as defined (every negative value and -0 give +0) in one integer max:
// finite floats with the sign bit clear order like their bit patterns, and every float with
// the sign bit set is a negative integer.
__device__ __forceinline__ float relu0(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Maximum of scores (finite or -inf, never NaN) without the IEEE-mode canonicalisation.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(x, x of lane ^ 16) in the vector unit: the row swap of v_permlane16_swap leaves x of
// lanes l and l ^ 16 in the two results of every lane.
__device__ __forceinline__ float smax_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return smax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max(x, x of lane ^ 32), likewise with v_permlane32_swap.
__device__ __forceinline__ float smax_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return smax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Query tile held by a lane: column q (16 queries), group g = lane / 16 of every head.
template <int H>
struct PfQuery {
    uint4 c[H];                // FP4 codes of group g of head h
    uint32_t s[(H + 3) / 4];   // E8M0 code of group g of head h in byte h % 4 of s[h / 4]
    float w[H];
};

// Blocks per position chunk of a scoring workgroup.  At most 16 queries the scoring kernel
// streams the keys with little work per byte, so its chunks are halved: twice the
// workgroups are resident, and twice the staged bytes are in flight.
template <bool SMALL>
__host__ __device__ constexpr int pf_chunk_blocks() { return SMALL ? kPfChunkBlocks / 2 : kPfChunkBlocks; }

template <int H, int G, bool SMALL, int MODE>
__global__ __launch_bounds__(PfShape<MODE>::threads, 8 / PfShape<MODE>::waves) void k_prefill(PrefillArgs a) {
    using S = PfStage<H, G>;
    constexpr int kPfWaves = PfShape<MODE>::waves, kPfThreads = PfShape<MODE>::threads;
    constexpr int kPfQT = PfShape<MODE>::qt;
    // two stage buffers as distinct objects, so that the reads of one are known not to
    // alias the DMA into the other
    __shared__ S stA, stB;
    __shared__ PfMeta meta;
    if (SMALL && a.arrive && blockIdx.x == 0 && (int)threadIdx.x < a.n_q)  // (read by the selection)
        a.arrive[threadIdx.x] = 0;
    // workgroup -> (position chunk, query tile); the workgroups of one chunk are consecutive
    // on one XCD (dispatch places workgroup i on XCD i % 8) so its keys are fetched once
    const int T = a.n_qt * a.n_pc;
    const int bid = (int)blockIdx.x, x = bid % 8, i8 = bid / 8, per = T / 8, rem = T % 8;
    const int lin = x < rem ? x * (per + 1) + i8 : rem * (per + 1) + (x - rem) * per + i8;
    const int pc = lin / a.n_qt, qt = lin % a.n_qt;
    const int Q0 = qt * kPfQT;
    const int qlast = min(a.n_q, Q0 + kPfQT) - 1;
    const int Jbeg = pc * pf_chunk_blocks<SMALL>();
    // blocks this tile can see: j*8 <= q_pos0 + qlast
    const int Jend = min(min(a.nb, Jbeg + pf_chunk_blocks<SMALL>()), (a.q_pos0 + qlast) / kBlk + 1);
    // the flags of this (chunk, query tile), set by the pool selection and read by the
    // rescoring pass: cleared here by every workgroup, including those that see nothing of
    // the chunk
    if constexpr (MODE == kPfMaxima) {
        for (int i = (int)threadIdx.x; i < 8 * kPfQT; i += kPfThreads) {
            const int qi = Q0 + i % kPfQT;
            if (qi < a.n_q) a.need[((int64_t)pc * 8 + i / kPfQT) * a.n_q + qi] = 0u;
        }
    }
    if (Jbeg >= Jend) return;  // uniform per workgroup (no query of the tile sees the chunk)
    const int nstage = (Jend - Jbeg + kPfStageBlocks - 1) / kPfStageBlocks;

    const int lane = lane_id(), wave = (int)threadIdx.x / kWave;
    const int col = lane & 15, g = lane >> 4;
    const bool gl = g < G;  // lanes of groups >= G carry zeros (d_I < 128)

    // the chunk's table entries and key spans (blocks past Jend: absent, span 0)
    // (at most 16 queries: one workgroup per position chunk, which computes the spans of its
    // own blocks here instead of reading them from the span pass)
    for (int i = (int)threadIdx.x; i < pf_chunk_blocks<SMALL>(); i += kPfThreads) {
        const int j = Jbeg + i;
        const int32_t ph = j < Jend ? (int32_t)phys_block(a, j) : -1;
        meta.phys[i] = ph;
        if constexpr (SMALL) meta.kspan[i] = (uint8_t)block_span<H, G>(a, ph);
        else meta.kspan[i] = j < Jend ? a.kspan[j] : (uint8_t)0;
    }
    __syncthreads();
    const uint32_t sw16 = pf_swizzle16<H>(lane_id());
    pf_dma<H, G, kPfWaves>(a, meta, 0, stA, sw16);

    // At most 16 queries (a verification step): every wave takes the one query tile and a
    // quarter of each stage's positions (16-position tile u = wave) instead of a query tile
    // pair of its own, which would leave three of the four waves idle.  The stage's group
    // maxima are then combined across the waves through LDS.
    constexpr bool small = SMALL;  // the host sets it when n_q <= 16
    const int u_beg = small ? wave : 0, u_end = small ? wave + 1 : kPfStageBlocks / 2;
    __shared__ float sm_gm[2][kPfWaves][16];
    // group maxima of the current run of 8 stages (lane g: stages g and 4 + g of the run)
    float gbuf[kPfNQ][2];
#pragma unroll
    for (int jq = 0; jq < kPfNQ; jq++) gbuf[jq][0] = gbuf[jq][1] = -INFINITY;
    // queries of this wave's tiles, their scale spans and causal limits
    PfQuery<H> Q[kPfNQ];
    int qspan[kPfNQ], qb[kPfNQ];
#pragma unroll
    for (int jq = 0; jq < kPfNQ; jq++) {
        qb[jq] = small ? (jq == 0 ? Q0 : a.n_q) : Q0 + (wave * kPfNQ + jq) * 16;
        const int q = min(qb[jq] + col, a.n_q - 1);
        const uint8_t *qc = a.q_codes + (int64_t)q * H * G * 16;
        const uint8_t *qs = a.q_scales + (int64_t)q * H * G;
        int span = 0;
#pragma unroll
        for (int i = 0; i < (H + 3) / 4; i++) Q[jq].s[i] = 0u;
#pragma unroll
        for (int h = 0; h < H; h++) {
            Q[jq].c[h] = gl ? *reinterpret_cast<const uint4 *>(qc + (h * G + (gl ? g : 0)) * 16)
                            : make_uint4(0u, 0u, 0u, 0u);
            Q[jq].s[h / 4] |= (gl ? (uint32_t)qs[h * G + g] : 127u) << (8 * (h % 4));
            Q[jq].w[h] = a.w[(int64_t)q * H + h];
            int lo = 255, hi = 0;
#pragma unroll
            for (int gg = 0; gg < G; gg++) {
                lo = min(lo, (int)qs[h * G + gg]);
                hi = max(hi, (int)qs[h * G + gg]);
            }
            span = max(span, hi - lo);
        }
        // the query's own span, for the rescoring pass (from the first position chunk)
        if (MODE == kPfMaxima && pc == 0 && g == 0 && qb[jq] + col < a.n_q) a.qspan[qb[jq] + col] = (uint8_t)span;
        // wave maximum (queries past n_q repeat query n_q - 1)
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) span = max(span, __shfl_xor(span, o, kWave));
        qspan[jq] = __builtin_amdgcn_readfirstlane(span);
    }

    // the lane's byte offset, inside a stage, of head h's 16-byte chunk of its key row in
    // 16-position tile 0 (tile u adds 2u blocks): fixed for the kernel, so every LDS read
    // of the keys is this register plus an immediate
    uint32_t koff[H];
#pragma unroll
    for (int h = 0; h < H; h++) {
        const int row = g * kBlk + (col & 7);
        koff[h] = (uint32_t)((col >> 3) * S::BSTR + (row * H + (h ^ (row & (H - 1)))) * 16);
    }
    // scores of one staged stage: 4 tiles of 16 positions x the wave's 2 tiles of 16 queries
    auto compute = [&](const S &cur, int sidx) {
        const int J0 = Jbeg + sidx * kPfStageBlocks;
        const int jrel = sidx * kPfStageBlocks;
        uint32_t present = 0;
#pragma unroll
        for (int b = 0; b < kPfStageBlocks; b++)
            if (meta.phys[jrel + b] >= 0) present |= 1u << b;
        const uint2 ks8 = *reinterpret_cast<const uint2 *>(meta.kspan + jrel);
        float *ps_stage = a.pscore + (int64_t)J0 * a.n_q * kBlk;
        float *bs_stage = a.bscore + (int64_t)(J0 >> 3) * a.n_q * kBlk;
        float gm[kPfNQ];
        // maxima pass: the block maxima of the stage, one per 16-position tile (lane g < 2:
        // block 2u, else 2u + 1), stored once at the end of the stage (32 contiguous bytes
        // per query, so no line of the array is written back part-filled)
        f32x4_t bmv[kPfNQ];
#pragma unroll
        for (int jq = 0; jq < kPfNQ; jq++) {
            gm[jq] = -INFINITY;
            bmv[jq] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
        // 16-position tiles, unrolled (LDS offsets become immediates and the per-tile maxima
        // stay in place; a verification step runs one tile per wave)
#pragma unroll
        for (int u = u_beg; u < u_end; u++) {
            if constexpr (MODE == kPfMaxima) {
#pragma unroll
                for (int jq = 0; jq < kPfNQ; jq++) bmv[jq] = f32x4_t{bmv[jq][1], bmv[jq][2], bmv[jq][3], -INFINITY};
            }
            const int p0 = (J0 + 2 * u) * kBlk;
            // this lane's key row: position p0 + col, group g
            const int bi = 2 * u + (col >> 3), s = col & 7;
            const int row = g * kBlk + s;
            uint4 kc[H];
            uint32_t ksc[H];
            {
                const uint8_t *cb = cur.codes + 2 * u * S::BSTR;
#pragma unroll
                for (int h = 0; h < H; h++)
                    kc[h] = gl ? *reinterpret_cast<const uint4 *>(cb + koff[h]) : make_uint4(0u, 0u, 0u, 0u);
                if constexpr (H * G >= 4) {
                    // the position's H*G scale bytes start on a dword; byte h*G + g of
                    // them is byte ((h*G) & 3) + g of dword (h*G) / 4
                    const uint32_t *sd = cur.scales + (bi * S::SCB + s * H * G) / 4;
#pragma unroll
                    for (int h = 0; h < H; h++) {
                        const uint32_t dw = sd[(h * G) / 4];
                        ksc[h] = gl ? (dw >> (8 * (((h * G) & 3) + g))) : 127u;
                    }
                } else {
                    const int boff = bi * S::SCB + s * H * G + (gl ? g : 0);
#pragma unroll
                    for (int h = 0; h < H; h++) {
                        const int o = boff + h * G;
                        ksc[h] = gl ? (cur.scales[o >> 2] >> (8 * (o & 3))) : 127u;
                    }
                }
            }
            // largest key span of the tile's two blocks (bytes 2u, 2u + 1)
            const uint32_t ksp_w = u < 2 ? ks8.x : ks8.y;
            const uint32_t kspan_t = max((ksp_w >> (16 * (u & 1))) & 0xffu, (ksp_w >> (16 * (u & 1) + 8)) & 0xffu);
            const bool pres0 = (present >> (2 * u)) & 1u, pres1 = (present >> (2 * u + 1)) & 1u;
            // query tile jq takes part in this position tile (uniform)
            auto active = [&](int jq) {
                if (qb[jq] >= a.n_q) return false;                                  // no queries
                if (p0 > a.q_pos0 + min(qb[jq] + 15, a.n_q - 1)) return false;      // all masked
                return true;
            };
            // causal / presence mask, block maxima and stores of tile jq's scores
            auto tail = [&](int jq, f32x4_t sc) {
                // lane: query qb + col, positions p0 + 4*g + e
                const int tmin = a.q_pos0 + qb[jq];
                const int q = qb[jq] + col;
                const int t = a.q_pos0 + q;
                const int pl = p0 + 4 * g;
                const bool pres = g < 2 ? pres0 : pres1;
                if (p0 + 15 > tmin || !pres0 || !pres1) {
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        if (!pres || pl + e > t) sc[e] = -INFINITY;
                }
                const float m = smax_xor16(smax(smax(sc[0], sc[1]), smax(sc[2], sc[3])));
                gm[jq] = smax(gm[jq], m);
                // uniform stage bases, 32-bit lane offsets (< 8 blocks of n_q rows); lanes g and
                // g ^ 1 hold the same block maximum and store it to the same address
                const uint32_t po = (uint32_t)(((2 * u + (g >> 1)) * a.n_q + q) * kBlk + 4 * (g & 1));
                const uint32_t bo = (uint32_t)(q * kBlk + 2 * u + (g >> 1));
                if constexpr (MODE == kPfMaxima) {
                    bmv[jq][3] = m;
                } else if (qb[jq] + 15 < a.n_q && J0 + 2 * u + 1 < a.nb) {  // every lane's (query, block) exists
                    *reinterpret_cast<f32x4_t *>(ps_stage + po) = sc;
                    bs_stage[bo] = m;
                } else if (q < a.n_q && J0 + 2 * u + (g >> 1) < a.nb) {
                    // blocks past nb (the tile's second block when nb is odd) are not stored:
                    // the score arrays hold blocks 0 .. nb - 1 only
                    *reinterpret_cast<f32x4_t *>(ps_stage + po) = sc;
                    bs_stage[bo] = m;
                }
            };
            if constexpr (kPfNQ == 2 && H % 4 == 0) {
                // both query tiles on the one-product path: the second tile's products are
                // issued between the first tile's epilogue steps, so the matrix core works
                // while the vector unit runs the ReLU / fma chain
                if (active(0) && active(1) && (int)kspan_t + max(qspan[0], qspan[1]) <= kSpanExact) {
                    f32x4_t d0[H], d1[H];
                    f32x4_t sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int h = 0; h < H; h++) d0[h] = mfma_pick(kc[h], Q[0].c[h], ksc[h], Q[0].s[h / 4], h % 4);
#pragma unroll
                    for (int h = 0; h < H; h++) {
                        d1[h] = mfma_pick(kc[h], Q[1].c[h], ksc[h], Q[1].s[h / 4], h % 4);
#pragma unroll
                        for (int e = 0; e < 4; e++) sc0[e] = __builtin_fmaf(Q[0].w[h], relu0(d0[h][e]), sc0[e]);
                    }
#pragma unroll
                    for (int h = 0; h < H; h++)
#pragma unroll
                        for (int e = 0; e < 4; e++) sc1[e] = __builtin_fmaf(Q[1].w[h], relu0(d1[h][e]), sc1[e]);
                    __builtin_amdgcn_sched_group_barrier(0x008, H, 0);
#pragma unroll
                    for (int h = 0; h < H; h++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    }
                    // both chains end here, before the stores' branches (nothing sinks below)
                    asm volatile("" : "+v"(sc0), "+v"(sc1));
                    tail(0, sc0);
                    tail(1, sc1);
                    continue;
                }
            }
#pragma unroll
            for (int jq = 0; jq < kPfNQ; jq++) {
                if (!active(jq)) continue;                           // uniform
                const bool exact = (int)kspan_t + qspan[jq] <= kSpanExact;
                f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
                // four heads at a time: their products are issued before the epilogue
                // consumes them
#pragma unroll
                for (int h0 = 0; h0 < H; h0 += 4) {
                    constexpr int NH = H < 4 ? H : 4;
                    f32x4_t d[NH];
                    if (exact) {
#pragma unroll
                        for (int i = 0; i < NH; i++)
                            d[i] = mfma_pick(kc[h0 + i], Q[jq].c[h0 + i], ksc[h0 + i], Q[jq].s[h0 / 4], i);
                    } else {
                        // exact by construction: one product per group (the other groups'
                        // key lanes zeroed), summed in group order
#pragma unroll
                        for (int i = 0; i < NH; i++) {
                            d[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int g2 = 0; g2 < G; g2++) {
                                const uint4 kz = g == g2 ? kc[h0 + i] : make_uint4(0u, 0u, 0u, 0u);
                                const f32x4_t t = mfma_pick(kz, Q[jq].c[h0 + i], ksc[h0 + i], Q[jq].s[h0 / 4], i);
#pragma unroll
                                for (int e = 0; e < 4; e++) d[i][e] = d[i][e] + t[e];
                            }
                        }
                    }
#pragma unroll
                    for (int i = 0; i < NH; i++)
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            sc[e] = __builtin_fmaf(Q[jq].w[h0 + i], relu0(d[i][e]), sc[e]);
                }
                tail(jq, sc);
            }
        }
        if constexpr (MODE == kPfMaxima) {
            // lane g = 0 holds the maxima of blocks 0, 2, 4, 6 and lane g = 2 those of 1, 3, 5,
            // 7 (the same query): they swap and store blocks 0..3 and 4..7.  A group past nb
            // (the stage's tail) holds -inf there; the array covers whole groups.
#pragma unroll
            for (int jq = 0; jq < kPfNQ; jq++) {
                f32x4_t o;
#pragma unroll
                for (int i = 0; i < 4; i++) o[i] = __shfl_xor(bmv[jq][i], 32, kWave);
                const int q = qb[jq] + col;
                if (q < a.n_q && (g & 1) == 0) {
                    const f32x4_t v = g == 0 ? f32x4_t{bmv[jq][0], o[0], bmv[jq][1], o[1]}
                                             : f32x4_t{o[2], bmv[jq][2], o[3], bmv[jq][3]};
                    *reinterpret_cast<f32x4_t *>(bs_stage + q * kBlk + (g == 0 ? 0 : 4)) = v;
                }
            }
        }
#pragma unroll
        for (int jq = 0; jq < kPfNQ; jq++) {
            const float v = smax_xor32(gm[jq]);  // every lane of query col holds it
            const int q = qb[jq] + col;
            if (small) {
                if (jq == 0 && g == 0) sm_gm[sidx & 1][wave][col] = v;
                continue;
            }
            // group maxima leave in runs of 8 stages, 32 contiguous bytes per query: lane g
            // keeps stages s0 + g and s0 + 4 + g of the run; groups past the query's causal
            // end (uncomputed or masked) hold -inf, which the selection never reads
            const bool mine = (sidx & 3) == g, hi = (sidx >> 2) & 1;
            gbuf[jq][0] = mine && !hi ? v : gbuf[jq][0];
            gbuf[jq][1] = mine && hi ? v : gbuf[jq][1];
            if ((sidx & 7) == 7 || sidx == nstage - 1) {  // uniform
                const int s0 = sidx & ~7;
                float vals[8];
#pragma unroll
                for (int r = 0; r < 2; r++)
#pragma unroll
                    for (int gg = 0; gg < 4; gg++) vals[4 * r + gg] = __shfl(gbuf[jq][r], col + 16 * gg, kWave);
#pragma unroll
                for (int i = 0; i < 8; i++) if (s0 + i > sidx) vals[i] = -INFINITY;
                gbuf[jq][0] = gbuf[jq][1] = -INFINITY;
                const int G0 = Jbeg / kPfStageBlocks + s0;  // a multiple of 8 (rows: multiples of 4)
                if (g == 0 && q < a.n_q) {
                    float *dst = a.gmax + (int64_t)q * a.ngmax + G0;
                    if (G0 < a.ngmax) *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{vals[0], vals[1], vals[2], vals[3]};
                    if (G0 + 4 < a.ngmax) *reinterpret_cast<f32x4_t *>(dst + 4) = f32x4_t{vals[4], vals[5], vals[6], vals[7]};
                }
            }
        }
    };
    // small: group maxima of stage sidx from the four waves' parts (after the barrier that
    // ends the stage; the buffer of stage sidx is next written two stages later)
    auto combine_gm = [&](int sidx) {
        if (!small || sidx < 0 || wave != 0 || g != 0) return;
        const int J0 = Jbeg + sidx * kPfStageBlocks;
        const int q = Q0 + col;
        float v = sm_gm[sidx & 1][0][col];
#pragma unroll
        for (int w = 1; w < kPfWaves; w++) v = smax(v, sm_gm[sidx & 1][w][col]);
        if (q < a.n_q && J0 * kBlk <= a.q_pos0 + q)
            a.gmax[(int64_t)q * a.ngmax + J0 / kPfStageBlocks] = v;
    };

    // pipeline: the DMA of stage s+1 runs while stage s is computed; a stage ends with every
    // wave's DMA complete (vmcnt 0) and a barrier
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int sidx = 0; sidx < nstage; sidx += 2) {
        if (sidx + 1 < nstage) pf_dma<H, G, kPfWaves>(a, meta, (sidx + 1) * kPfStageBlocks, stB, sw16);
        combine_gm(sidx - 1);
        compute(stA, sidx);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (sidx + 1 >= nstage) break;
        if (sidx + 2 < nstage) pf_dma<H, G, kPfWaves>(a, meta, (sidx + 2) * kPfStageBlocks, stA, sw16);
        combine_gm(sidx);
        compute(stB, sidx + 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    combine_gm(nstage - 1);
}


// ------------------------------------------------------------------ rescoring pass
//
// With more than 16 queries the selection flags, per query, the pool blocks whose maximum
// reaches the k-th largest pool block maximum (about k of them); their position scores are
// recomputed here, block-major: one workgroup per stage of 8 blocks stages the stage's keys
// in LDS once, lists from the flag words the queries that flagged a block of each of its
// four 16-position tiles, and wave u computes tile u for its listed queries, 16 at a time
// (each lane's query gathered into the B operand), storing the scores of the flagged blocks
// only.  Tile products, the ReLU / fma chain over heads and the causal mask are those of the
// scoring pass, so the scores are bit-identical to the ones it would have stored.
constexpr int kRsWaves = 4, kRsThreads = kRsWaves * kWave;
constexpr int kRsBatch = 4096;  // queries listed per round (16-bit list entries: 12 + 2 bits)

// Query q as the B operand of a 16 x 16 tile (lane column: the query, group g of every head):
// codes, E8M0 codes packed as PfQuery::s and head weights, from whole-row vector loads.
template <int H, int G>
__device__ __forceinline__ void pf_gather_query(const PrefillArgs &a, int q, int g, PfQuery<H> &Q) {
    const bool gl = g < G;
    const int gg = gl ? g : 0;
    const uint8_t *qc = a.q_codes + (int64_t)q * H * G * 16;
#pragma unroll
    for (int h = 0; h < H; h++)
        Q.c[h] = gl ? *reinterpret_cast<const uint4 *>(qc + (h * G + gg) * 16) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < (H + 3) / 4; i++) Q.s[i] = 0u;
    if constexpr (H * G >= 4) {
        // byte h*G + g of the query's H*G scale bytes is byte ((h*G) & 3) + g of dword (h*G)/4
        const uint32_t *qs = reinterpret_cast<const uint32_t *>(a.q_scales + (int64_t)q * H * G);
        uint32_t dw[H * G / 4];
#pragma unroll
        for (int i = 0; i < H * G / 4; i++) dw[i] = qs[i];
#pragma unroll
        for (int h = 0; h < H; h++) {
            const uint32_t e = gl ? (dw[(h * G) / 4] >> (8 * (((h * G) & 3) + gg))) & 0xffu : 127u;
            Q.s[h / 4] |= e << (8 * (h % 4));
        }
    } else {
        const uint8_t *qs = a.q_scales + (int64_t)q * H * G;
#pragma unroll
        for (int h = 0; h < H; h++) Q.s[h / 4] |= (gl ? (uint32_t)qs[h * G + gg] : 127u) << (8 * (h % 4));
    }
#pragma unroll
    for (int h = 0; h < H; h++) Q.w[h] = a.w[(int64_t)q * H + h];
}

template <int H, int G>
__global__ __launch_bounds__(kRsThreads, 2) void k_prefill_rescore(PrefillArgs a) {
    using S = PfStage<H, G>;
    __shared__ S st;
    __shared__ PfMeta meta;  // entries 0..7: the stage's blocks
    __shared__ uint16_t lst[kRsWaves][kRsBatch];  // (query - batch start) << 2 | flags of the tile's two blocks
    __shared__ uint32_t cnt[kRsWaves];
    const int pc = (int)blockIdx.x / (kPfChunkBlocks / kPfStageBlocks);
    const int sg = (int)blockIdx.x % (kPfChunkBlocks / kPfStageBlocks);
    const int J0 = pc * kPfChunkBlocks + sg * kPfStageBlocks;
    if (J0 >= a.nb) return;  // uniform: no block of the stage is visible to any query
    const int tid = (int)threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col = lane & 15, g = lane >> 4;
    const bool gl = g < G;
    if (tid < kPfStageBlocks) {
        const int j = J0 + tid;
        meta.phys[tid] = (int32_t)phys_block(a, j);
        meta.kspan[tid] = j < a.nb ? a.kspan[j] : (uint8_t)0;
    }
    __syncthreads();
    pf_dma<H, G, kRsWaves>(a, meta, 0, st, pf_swizzle16<H>(lane));

    // this wave's 16-position tile: blocks 2u, 2u + 1 of the stage
    const int u = wave;
    const int p0 = (J0 + 2 * u) * kBlk;
    const int bi = 2 * u + (col >> 3), sl = col & 7;
    const int row = g * kBlk + sl;
    const uint32_t kspan_t = max((uint32_t)meta.kspan[2 * u], (uint32_t)meta.kspan[2 * u + 1]);
    const bool pres = meta.phys[2 * u + (g >> 1)] >= 0;  // the block of the lane's output rows
    const uint32_t *nw = a.need + ((int64_t)pc * 8 + sg / 4) * a.n_q;
    const int nsh = 8 * (sg % 4);

    for (int qb = 0; qb < a.n_q; qb += kRsBatch) {
        // list the batch's queries per tile: each lane counts its entries per tile, a wave
        // scan places them, and one LDS atomic per tile and wave reserves the wave's range
        constexpr int NI = kRsBatch / kRsThreads;
        uint32_t m8[NI / 4];  // the flag bytes of the thread's NI queries, four per word
#pragma unroll
        for (int i = 0; i < NI / 4; i++) m8[i] = 0u;
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const int q = qb + i * kRsThreads + tid;
            m8[i / 4] |= (q < a.n_q ? (nw[q] >> nsh) & 0xffu : 0u) << (8 * (i % 4));
        }
        if (tid < kRsWaves) cnt[tid] = 0u;
        // per-lane counts of tiles (0, 1) and (2, 3) in 16-bit fields (wave sums <= 1024)
        uint32_t c2[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
            for (int t = 0; t < kRsWaves; t++)
                c2[t / 2] += (((m8[i / 4] >> (8 * (i % 4) + 2 * t)) & 3u) != 0u) ? 1u << (16 * (t % 2)) : 0u;
        __syncthreads();
        uint32_t o[kRsWaves];
#pragma unroll
        for (int t2 = 0; t2 < 2; t2++) {
            const uint32_t incl = wave_incl_scan(c2[t2]);
            const uint32_t tot = __shfl(incl, kWave - 1, kWave);
            const uint32_t ex = incl - c2[t2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int t = 2 * t2 + h;
                const uint32_t tt = (tot >> (16 * h)) & 0xffffu;
                uint32_t base = 0u;
                if (lane == 0 && tt) base = atomicAdd(&cnt[t], tt);
                o[t] = __builtin_amdgcn_readfirstlane(base) + ((ex >> (16 * h)) & 0xffffu);
            }
        }
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
            for (int t = 0; t < kRsWaves; t++) {
                const uint32_t f = (m8[i / 4] >> (8 * (i % 4) + 2 * t)) & 3u;
                if (f != 0u) lst[t][o[t]++] = (uint16_t)(((uint32_t)(i * kRsThreads + tid) << 2) | f);
            }
        if (qb == 0) __builtin_amdgcn_s_waitcnt(0);  // the stage's keys
        __syncthreads();
        const int n = (int)cnt[u];
        if (n == 0) {  // uniform
            __syncthreads();
            continue;
        }
        // the tile's key rows, as the scoring pass reads them
        uint4 kc[H];
        uint32_t ksc[H];
        {
            const uint8_t *cb = st.codes + bi * S::BSTR;
#pragma unroll
            for (int h = 0; h < H; h++)
                kc[h] = gl ? *reinterpret_cast<const uint4 *>(cb + (row * H + (h ^ (row & (H - 1)))) * 16)
                           : make_uint4(0u, 0u, 0u, 0u);
            const int boff = bi * S::SCB + sl * H * G + (gl ? g : 0);
#pragma unroll
            for (int h = 0; h < H; h++) {
                const int o = boff + h * G;
                ksc[h] = gl ? (st.scales[o >> 2] >> (8 * (o & 3))) : 127u;
            }
        }
        // tiles of 16 listed queries; the next tile's queries are fetched while this one
        // is computed
#pragma unroll 1
        for (int e0 = 0; e0 < n; e0 += 16) {
            const bool live = e0 + col < n;
            const uint32_t ent = lst[u][live ? e0 + col : e0];
            const int q = qb + (int)(ent >> 2);
            PfQuery<H> Q;
            pf_gather_query<H, G>(a, q, g, Q);
            int span = (int)a.qspan[q];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) span = max(span, __shfl_xor(span, o, kWave));
            const int qspan_t = __builtin_amdgcn_readfirstlane(span);
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
            if ((int)kspan_t + qspan_t <= kSpanExact) {
#pragma unroll
                for (int h0 = 0; h0 < H; h0 += 4) {
                    constexpr int NH = H < 4 ? H : 4;
                    f32x4_t d[NH];
#pragma unroll
                    for (int i = 0; i < NH; i++) d[i] = mfma_pick(kc[h0 + i], Q.c[h0 + i], ksc[h0 + i], Q.s[h0 / 4], i);
#pragma unroll
                    for (int i = 0; i < NH; i++)
#pragma unroll
                        for (int r = 0; r < 4; r++) sc[r] = __builtin_fmaf(Q.w[h0 + i], relu0(d[i][r]), sc[r]);
                }
            } else {
                // exact by construction: one product per group (the other groups' key lanes
                // zeroed), summed in group order; one head at a time (a rare path, kept small)
#pragma unroll
                for (int h = 0; h < H; h++) {
                    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int g2 = 0; g2 < G; g2++) {
                        uint4 kz = g == g2 ? kc[h] : make_uint4(0u, 0u, 0u, 0u);
                        // (formed here, not hoisted out of the tile loop for every head and group)
                        asm volatile("" : "+v"(kz.x), "+v"(kz.y), "+v"(kz.z), "+v"(kz.w));
                        const f32x4_t t = mfma_pick(kz, Q.c[h], ksc[h], Q.s[h / 4], h % 4);
#pragma unroll
                        for (int r = 0; r < 4; r++) d[r] = d[r] + t[r];
                    }
#pragma unroll
                    for (int r = 0; r < 4; r++) sc[r] = __builtin_fmaf(Q.w[h], relu0(d[r]), sc[r]);
                }
            }
            // lane: query q, positions p0 + 4g .. p0 + 4g + 3 (block 2u + g/2 of the stage)
            const int t = a.q_pos0 + q, pl = p0 + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; r++)
                if (!pres || pl + r > t) sc[r] = -INFINITY;
            if (live && ((ent >> (g >> 1)) & 1u)) {
                const int j = J0 + 2 * u + (g >> 1);
                *reinterpret_cast<f32x4_t *>(a.pscore + ((int64_t)j * a.n_q + q) * kBlk + 4 * (g & 1)) = sc;
            }
        }
        __syncthreads();  // the lists are rewritten by the next round
    }
}

typedef void (*PfFn)(const PrefillArgs &, int, hipStream_t);

// Launch of one scoring kernel: query tiles of the mode's workgroup size x position chunks.
template <int H, int G, bool SMALL, int MODE>
void launch_mode(PrefillArgs a, hipStream_t s) {
    using P = PfShape<MODE>;
    a.n_qt = (a.n_q + P::qt - 1) / P::qt;
    a.n_pc = (a.nb + pf_chunk_blocks<SMALL>() - 1) / pf_chunk_blocks<SMALL>();
    k_prefill<H, G, SMALL, MODE><<<a.n_qt * a.n_pc, P::threads, 0, s>>>(a);
}

// pass 0: scores and maxima (at most 16 queries: spans computed inside the scoring kernel),
// or spans and maxima; pass 1: the rescoring of the flagged blocks (more than 16 queries).
template <int H, int G>
void launch_prefill(const PrefillArgs &a, int pass, hipStream_t s) {
    if (a.n_q <= 16) {
        if (pass == 0) launch_mode<H, G, true, kPfAll>(a, s);
        return;
    }
    if (pass == 0) {
        const int spans = (a.nb * kBlk + 255) / 256;
        k_prefill_span<H, G><<<spans, 256, 0, s>>>(a);
        launch_mode<H, G, false, kPfMaxima>(a, s);
    } else {
        k_prefill_rescore<H, G><<<a.n_pc * (kPfChunkBlocks / kPfStageBlocks), kRsThreads, 0, s>>>(a);
    }
}

bool pick_prefill(int H, int dI, PfFn *fn) {
    const int G = dI / 32;
#define CSA2_PF_CASE(h, g) \
    if (H == h && G == g) { *fn = launch_prefill<h, g>; return true; }
    CSA2_PF_CASE(1, 1) CSA2_PF_CASE(1, 2) CSA2_PF_CASE(1, 4)
    CSA2_PF_CASE(2, 1) CSA2_PF_CASE(2, 2) CSA2_PF_CASE(2, 4)
    CSA2_PF_CASE(4, 1) CSA2_PF_CASE(4, 2) CSA2_PF_CASE(4, 4)
    CSA2_PF_CASE(8, 1) CSA2_PF_CASE(8, 2) CSA2_PF_CASE(8, 4)
#undef CSA2_PF_CASE
    return false;
}

// Workspace of a prefill chunk: position scores (block-major), block and group maxima, key
// spans; with more than 16 queries also the block flags (8 words per chunk of 256 blocks and
// query, word-major), the flagged blocks (K_blk per query), their per-query bounds and the
// queries' scale spans; with at most 16
// queries over a long table, the regions of the two-phase Full selection.
struct WsPrefill {
    size_t pscore, bscore, gmax, kspan, need, list, meta, qspan;
    int nw;
    size_t cand, mu_sc, mu_blk, cnt, arrive, total;
};
WsPrefill ws_prefill(const csa2_config *c, int n_q, int maxb) {
    const int K_blk = c->pool_blocks;
    WsPrefill w;
    const int ng = ngmax_of(maxb);
    const int npc = (maxb + kPfChunkBlocks - 1) / kPfChunkBlocks;
    const bool two = n_q > 16;
    size_t o = 0;
    w.pscore = o; o = align256(o + sizeof(float) * (size_t)n_q * maxb * kBlk);
    w.bscore = o; o = align256(o + sizeof(float) * (size_t)n_q * ng * kPfStageBlocks);
    w.gmax = o;   o = align256(o + sizeof(float) * (size_t)n_q * ng);
    w.kspan = o;  o = align256(o + (size_t)ng * kPfStageBlocks);
    w.need = o;   o = align256(o + (two ? sizeof(uint32_t) * 8 * (size_t)npc * n_q : 0));
    w.list = o;   o = align256(o + (two ? sizeof(int32_t) * (size_t)K_blk * n_q : 0));
    w.meta = o;   o = align256(o + (two ? sizeof(uint4) * (size_t)n_q : 0));
    w.qspan = o;  o = align256(o + (two ? (size_t)n_q : 0));
    w.nw = two ? 0 : sel2_workgroups(c, maxb);
    const size_t regs = (size_t)n_q * w.nw;
    w.cand = o;   o = align256(o + sizeof(uint2) * regs * kSel2GroupsPerW * kItemBlocks);
    w.mu_sc = o;  o = align256(o + sizeof(float) * regs * kSel2MuCap * kBlk);
    w.mu_blk = o; o = align256(o + sizeof(int32_t) * regs * kSel2MuCap);
    w.cnt = o;    o = align256(o + sizeof(int32_t) * regs * 2);
    w.arrive = o; o = align256(o + sizeof(int32_t) * (w.nw ? (size_t)n_q : 0));
    w.total = o;
    return w;
}

}  // namespace

size_t prefill_ws_bytes(const csa2_config *c, int32_t n_q, int32_t maxb) {
    return ws_prefill(c, std::max(n_q, 0), maxb).total;
}

}  // namespace csa2

using namespace csa2;

namespace {

// Arguments of both prefill phases; returns a status (CSA2_OK: *a / *sel filled).
int prefill_setup(const csa2_config *c, const uint8_t *q_codes, const uint8_t *q_scales,
                  const float *w, int32_t q_pos0, int32_t n_q, const uint8_t *idx_cache,
                  int64_t n_blocks, const int32_t *block_table, int32_t maxb, void *ws,
                  size_t ws_bytes, PrefillArgs *a, PfFn *fn) {
    const int st = check_index_cfg(c);
    if (st) return st;
    if (!q_codes || !q_scales || !w || !idx_cache || n_blocks <= 0 || !block_table ||
        maxb <= 0 || q_pos0 < 0 || n_q < 0 || !ws)
        return CSA2_ERR_INVALID;
    if ((int64_t)q_pos0 + n_q > (int64_t)maxb * kBlk) return CSA2_ERR_INVALID;
    if (c->shared_key) return CSA2_ERR_UNSUPPORTED;  // the prefill kernels read per-head keys
    const WsPrefill L = ws_prefill(c, n_q, maxb);
    if (ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
    if (!pick_prefill(c->n_idx_heads, c->idx_dim, fn)) return CSA2_ERR_UNSUPPORTED;
    uint8_t *base = (uint8_t *)ws;
    *a = PrefillArgs{};
    a->q_codes = q_codes;
    a->q_scales = q_scales;
    a->w = w;
    a->q_pos0 = q_pos0;
    a->n_q = n_q;
    a->idx_cache = idx_cache;
    a->n_blocks = n_blocks;
    a->table = block_table;
    a->maxb = maxb;
    a->nb = (int32_t)(((int64_t)q_pos0 + n_q + kBlk - 1) / kBlk);
    a->kspan = base + L.kspan;
    a->pscore = (float *)(base + L.pscore);
    a->bscore = (float *)(base + L.bscore);
    a->gmax = (float *)(base + L.gmax);
    a->need = (uint32_t *)(base + L.need);
    a->qspan = base + L.qspan;
    a->arrive = L.nw ? (int32_t *)(base + L.arrive) : nullptr;
    a->ngmax = ngmax_of(maxb);
    a->n_pc = (a->nb + kPfChunkBlocks - 1) / kPfChunkBlocks;
    return CSA2_OK;
}

}  // namespace

extern "C" int csa2_index_prefill_scan(const csa2_config *c, const uint8_t *q_codes,
                                       const uint8_t *q_scales, const float *w, int32_t q_pos0,
                                       int32_t n_q, const uint8_t *idx_cache, int64_t n_blocks,
                                       const int32_t *block_table, int32_t maxb, void *ws,
                                       size_t ws_bytes, hipStream_t stream) {
    PrefillArgs a;
    PfFn fn;
    const int st = prefill_setup(c, q_codes, q_scales, w, q_pos0, n_q, idx_cache, n_blocks,
                                 block_table, maxb, ws, ws_bytes, &a, &fn);
    if (st) return st;
    if (n_q == 0) return CSA2_OK;
    fn(a, 0, stream);
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

extern "C" int csa2_index_prefill_finish(const csa2_config *c, const uint8_t *q_codes,
                                         const uint8_t *q_scales, const float *w,
                                         int32_t q_pos0, int32_t n_q, const uint8_t *idx_cache,
                                         int64_t n_blocks, const int32_t *block_table,
                                         int32_t maxb, int32_t *pool_blocks, int32_t *pool_len,
                                         int32_t *topk, int32_t *topk_len, void *ws,
                                         size_t ws_bytes, hipStream_t stream) {
    PrefillArgs a;
    PfFn fn;
    const int st = prefill_setup(c, q_codes, q_scales, w, q_pos0, n_q, idx_cache, n_blocks,
                                 block_table, maxb, ws, ws_bytes, &a, &fn);
    if (st) return st;
    if (!pool_blocks || !pool_len || !topk || !topk_len) return CSA2_ERR_INVALID;
    if (n_q == 0) return CSA2_OK;
    SelectArgs s{};
    s.ctx_len = nullptr;
    s.q_pos0 = q_pos0;
    s.maxb = maxb;
    s.B = n_q;
    s.K_blk = c->pool_blocks;
    s.k = c->topk;
    s.pscore = a.pscore;
    s.bscore = a.bscore;
    s.ps_b = kBlk;
    s.ps_j = (int64_t)n_q * kBlk;
    s.bs_b = kBlk;
    s.bs_g = (int64_t)n_q * kBlk;
    s.gmax = a.gmax;
    s.ngmax = a.ngmax;
    s.pool_blocks = pool_blocks;
    s.pool_len = pool_len;
    s.topk = topk;
    s.topk_len = topk_len;
    const WsPrefill L = ws_prefill(c, n_q, maxb);
    uint8_t *base = (uint8_t *)ws;
    if (n_q <= 16) {
        if (!L.nw) return launch_select(s, false, stream);
        // a long table: the two-phase selection per query (the scoring kernel cleared the
        // arrival counters)
        s.sel2.nw = L.nw;
        s.sel2.cand = (uint2 *)(base + L.cand);
        s.sel2.mu_sc = (float *)(base + L.mu_sc);
        s.sel2.mu_blk = (int32_t *)(base + L.mu_blk);
        s.sel2.cnt = (int32_t *)(base + L.cnt);
        s.sel2.arrive = (int32_t *)(base + L.arrive);
        return launch_select_full2(s, stream);
    }
    // more queries: the maxima pass left the position scores out; select the pools and flag
    // the blocks the top-k reads, rescore those, then select the top-k
    s.pf_need = a.need;
    s.pf_list = (int32_t *)(base + L.list);
    s.pf_meta = (uint4 *)(base + L.meta);
    int r = launch_select_prefill(s, 0, stream);
    if (r) return r;
    fn(a, 1, stream);
    if (hipGetLastError() != hipSuccess) return CSA2_ERR_HIP;
    return launch_select_prefill(s, 1, stream);
}

extern "C" int csa2_index_prefill(const csa2_config *c, const uint8_t *q_codes,
                                  const uint8_t *q_scales, const float *w, int32_t q_pos0,
                                  int32_t n_q, const uint8_t *idx_cache, int64_t n_blocks,
                                  const int32_t *block_table, int32_t maxb, int32_t *pool_blocks,
                                  int32_t *pool_len, int32_t *topk, int32_t *topk_len, void *ws,
                                  size_t ws_bytes, hipStream_t stream) {
    if (!pool_blocks || !pool_len || !topk || !topk_len) return CSA2_ERR_INVALID;
    const int st = csa2_index_prefill_scan(c, q_codes, q_scales, w, q_pos0, n_q, idx_cache,
                                           n_blocks, block_table, maxb, ws, ws_bytes, stream);
    if (st) return st;
    return csa2_index_prefill_finish(c, q_codes, q_scales, w, q_pos0, n_q, idx_cache, n_blocks,
                                     block_table, maxb, pool_blocks, pool_len, topk, topk_len,
                                     ws, ws_bytes, stream);
}
