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
// then [k, k+W) = window positions, in chunks of 64 rows.  A workgroup (split, sequence,
// head group of 16) runs NS chunk streams of 4 waves (16 rows each) over its cps chunks with
// an online softmax; NS = 2 for batches too small to fill the chip (the two streams take the
// chunks of each pair side by side and join through LDS at the end), NS = 1 otherwise.
//   1. The query rows are loaded while the row addresses resolve (top-k entry, then block
//      table), so those loads overlap that chain; NS = 2 also requests each lane's row
//      bytes before the chunk's first barriers.
//   2. Each lane converts one row's 128-dim quarter to bf16 with the gfx950 scaled
//      converters (exact: E2M1 / E4M3 values times a power of two fit bf16).  Those
//      registers are the B operand of S = Q K^T on MFMA 16x16x32 bf16 (fp32 accumulation);
//      the same values go to LDS row-major (V), read back with transpose reads.
//   3. Softmax statistics per head over the 64 rows (DPP row reductions + LDS).
//   4. O = P V on MFMA with P split into bf16 hi + lo parts (error ~2^-17 relative).
//   5. One split per sequence writes the outputs; with several, each writes its partial
//      (O, max, sum) to the workspace and the last split of (sequence, head group) to
//      arrive (an atomic counter) combines them.
// The appended window row of the fused append is staged in LDS by DMA at kernel start and
// quantised once by the stream whose chunk attends it.
#include <mutex>

#include "csa2_layer.h"
#include "csa2_quant.h"

namespace csa2 {

constexpr int kStreamThreads = 256;  // one chunk stream: 4 waves of 16 rows
constexpr int kD = kAttnDim;       // latent dim handled by these kernels
constexpr int kPStride = 64 + 4;   // padded row of the P tile (floats)
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 of the gfx9 family
constexpr int kSc1 = 16;                  // buffer access cache policy: agent scope (sc1)

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
    int32_t new_pos_off;  // the appended position is new_pos[b] + new_pos_off
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

// The V tile: the chunk's 64 rows in row order, kVStride elements apart (one 16-byte pad
// per row, so that the 8 lanes of a 16-byte store phase land on distinct banks).  The B
// operand of O = P V (8 consecutive rows of one dim per lane) comes from gfx950 transpose
// reads: in each 16-lane group, lane j = 4a + c receives element c of the 8-byte chunks
// addressed by lanes a, a + 4, a + 8 and a + 12, so when lane i addresses row r0 + i/4,
// dims d0 + 4 (i % 4) .. + 3, lane j receives rows r0 .. r0 + 3 of dim d0 + j.
constexpr int kVStride = kD + 8;
typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t v_rows8(const __bf16 *p) {  // rows r0 .. r0 + 7
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    typedef short i16x8_t __attribute__((ext_vector_type(8)));
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * kVStride));
    const i16x8_t w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, w);  // whole-vector cast (no per-element inserts)
}

struct AttnShared {
    __bf16 vt[64 * kVStride];              // V tile, row-major (65 KB)
    float ptile[16 * kPStride];
    float red_m[4][16], red_l[4][16];
    __align__(16) uint8_t fresh_row[kD + kD / 32];  // the appended window row (MXFP8)
    int last;
};

// Combine the splits of (b, head group hg), run by the last split to finish:
// out = sum_s 2^((m_s - M) c) O_s / sum_s 2^((m_s - M) c) l_s per head, accumulated with a
// running maximum over batches of splits.  With T = 16 NS threads per head, thread
// (head h = tid / T, q = tid % T) owns dims 4q + 4Ti of head h, so T threads read one
// partial row in 16T-byte runs; a batch's rows and (max, sum) pairs are all loaded before
// any is used (one memory round trip per batch).  The loads are agent-scope coherent (they
// bypass lines this XCD's caches may hold from earlier calls), so the merge needs no cache
// invalidation.  An empty split's row was never written: its values are discarded by a
// select, which keeps the loads unconditional.
template <int NS>
__device__ __forceinline__ void merge_splits(const AttnArgs &a, int b, int hg) {
    constexpr int T = 16 * NS, NV = kD / 4 / T, NB = NS == 2 ? 5 : 4;
    const int tid = threadIdx.x, h = tid / T, q = tid % T;
    // buffer resources over this (b, hg)'s partials (split 0 .. nsplit-1, 16 heads each);
    // the loads carry the agent scope bit (sc1)
    const int64_t sstride = (int64_t)a.Hq * kD;  // floats between splits
    const uint32_t o_bytes = (uint32_t)(sizeof(float) * ((a.nsplit - 1) * sstride + 16 * kD));
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        a.part_o + ((int64_t)b * a.nsplit * a.Hq + hg * 16) * kD, 0, o_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(
        a.part_ml + 2 * ((int64_t)b * a.nsplit * a.Hq + hg * 16), 0,
        (uint32_t)(sizeof(float) * 2 * ((a.nsplit - 1) * a.Hq + 16)), kBufferWord3);
    float4 acc[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) acc[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float M = -INFINITY, lw = 0.0f;
    for (int s0 = 0; s0 < a.nsplit; s0 += NB) {
        float2 st[NB];
        float4 v[NB][NV];
#pragma unroll
        for (int u = 0; u < NB; u++) {
            const int sp = min(s0 + u, a.nsplit - 1);
            st[u] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(
                rml, (int)(sizeof(float) * 2 * (sp * a.Hq + h)), 0, kSc1));
#pragma unroll
            for (int i = 0; i < NV; i++)
                v[u][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                    ro, (int)(sizeof(float) * (sp * sstride + h * kD + 4 * (q + T * i))), 0, kSc1));
        }
        float mu[NB], mb = M;
#pragma unroll
        for (int u = 0; u < NB; u++) {
            mu[u] = s0 + u < a.nsplit && st[u].y > 0.0f ? st[u].x : -INFINITY;
            mb = fmaxf(mb, mu[u]);
        }
        const float alpha = M == -INFINITY ? 0.0f : exp2f((M - mb) * a.scale_log2);
        lw *= alpha;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            acc[i].x *= alpha;
            acc[i].y *= alpha;
            acc[i].z *= alpha;
            acc[i].w *= alpha;
        }
#pragma unroll
        for (int u = 0; u < NB; u++) {
            const bool use = mu[u] != -INFINITY;
            const float e = use ? exp2f((mu[u] - mb) * a.scale_log2) : 0.0f;
            lw += use ? e * st[u].y : 0.0f;
#pragma unroll
            for (int i = 0; i < NV; i++) {
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
    for (int i = 0; i < NV; i++)
        dst[T * i] = make_float4(acc[i].x * inv, acc[i].y * inv, acc[i].z * inv, acc[i].w * inv);
    if (q == 0)
        a.lse[(int64_t)b * a.Hq + hg * 16 + h] = lw > 0.0f ? a.sm_scale * M + logf(lw) : -INFINITY;
}

// NS chunk streams of 4 waves per workgroup.  NS = 2 (batches too small to fill the chip):
// streams 0 and 1 take chunks c0 and c0 + 1 of each pair side by side, and the two states
// join through LDS at the end (each stream finishing half of the dims), which halves the
// splits the merge reads.  NS = 2 loads the 16 query rows once into LDS and every wave
// takes its slice into registers while the row addresses resolve; NS = 1 loads the slices
// straight into registers.
template <int NS>
__global__ __launch_bounds__(NS * kStreamThreads, 3 - NS) void k_attn(AttnArgs a) {
    __shared__ __align__(16) AttnShared shs[NS];
    __shared__ __align__(16) float4 fstage[kD / 4];  // the appended fp32 row, staged by DMA
    __shared__ __align__(16) uint4 qtile[NS == 2 ? 16 * (kD / 8 + 1) : 1];  // 16 query rows, padded

    // One split per pair (prefill, large batches): XCD x (dispatch places workgroup i on XCD
    // i % 8) takes a contiguous range of (sequence, head group) pairs in order, so the head
    // groups of one query, which read the same rows, and neighbouring queries, whose windows
    // overlap, share that XCD's L2.
    int pair = (int)blockIdx.y;
    if (a.nsplit == 1 && gridDim.y % 8 == 0) pair = (pair % 8) * (int)(gridDim.y / 8) + pair / 8;
    const int s = blockIdx.x, b = pair / a.HG, hg = pair % a.HG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int st = NS == 2 ? tid / kStreamThreads : 0, ts = tid % kStreamThreads, wave = ts >> 6;
    const int c16 = lane & 15, g4 = lane >> 4;
    AttnShared &sh = shs[st];

    // ---- every load that depends on nothing else is requested before any result is used:
    //      this lane's query slice (head c16, dims g4*128 ..; the A operand of S = Q K^T),
    //      the sequence's length, top-k length and append position, and the lane's top-k
    //      entries of the stream's first two chunks (read clamped into the row, masked once
    //      the length arrives).  NS = 2: the 16 query rows (16 KB) go to LDS, 32 bytes per
    //      thread, rows 65 16-byte chunks apart (8 lanes reading one chunk of 8 rows hit
    //      distinct banks), so that the workgroup fetches them once.
    bf16x8_t qa[16];
    uint4 qv[2];
    if (NS == 2) {
        const uint4 *qg = reinterpret_cast<const uint4 *>(a.q + ((int64_t)b * a.Hq + hg * 16) * kD);
#pragma unroll
        for (int j = 0; j < 2; j++) qv[j] = qg[tid + j * NS * kStreamThreads];  // 1024 pieces
    } else {
        const bf16x8_t *qh = reinterpret_cast<const bf16x8_t *>(
            a.q + ((int64_t)b * a.Hq + hg * 16 + c16) * kD + g4 * 128);
#pragma unroll
        for (int t = 0; t < 16; t++) qa[t] = qh[t];
    }
    // (absent pointers are replaced by topk_len, which is always valid, and the value ignored)
    const int32_t len_v = *(a.ctx_len ? a.ctx_len + b : a.topk_len + b);
    const int32_t tl_v = a.topk_len[b];
    const int32_t np_v = *(a.swa_new ? a.new_pos + b : a.topk_len + b);
    const int r_loc = 16 * wave + c16;
    const int nchunk = attn_splits(a.k, a.W);
    // split s takes every nsplit-th chunk from chunk s (so that the window's chunks, whose
    // rows are twice as long, go to different splits); stream st of the split takes the
    // split's chunks st, st + NS, ...: chunk s + nsplit (i NS + st) in its i-th step
    const int cstep = NS * a.nsplit;
    const int c_first = s + a.nsplit * st;
    auto topk_raw = [&](int c) -> int32_t {
        const int rg = c * kAttnRows + r_loc;
        return a.topk[(int64_t)b * a.k + min(rg, a.k - 1)];
    };
    const int32_t e_first = topk_raw(c_first), e_second = topk_raw(c_first + cstep);
    if (NS == 2) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int i = tid + j * NS * kStreamThreads;
            qtile[(i >> 6) * 65 + (i & 63)] = qv[j];
        }
    }

    const int L = clamp_ctx(a.ctx_len ? len_v : a.q_pos0 + b + 1, a.maxb);
    const int tl = max(0, min(tl_v, a.k));
    const int w0 = max(0, L - a.W), nwin = L - w0;
    const int np_b = a.swa_new ? np_v + a.new_pos_off : -1;

    // ---- the appended row, when one of this workgroup's chunks attends it: its 16 quantising
    //      threads (lanes 0..15 of the stream's first wave) stage the fp32 row in LDS by DMA
    //      now, so that the quantisation does not wait for it later
    const bool in_win = np_b >= w0 && np_b < L && np_b - w0 < a.W;
    const int fc = a.swa_new && np_b >= 0 && in_win ? (a.k + np_b - w0) / kAttnRows : -1;  // its chunk
    if (fc >= 0) {
        if (fc % a.nsplit == s && (fc / a.nsplit) % NS == st && ts < kD / 32) {
            const uint8_t *src = reinterpret_cast<const uint8_t *>(a.swa_new + (int64_t)b * kD) + 128 * ts;
#pragma unroll
            for (int j = 0; j < 8; j++)
                __builtin_amdgcn_global_load_lds(src + 16 * j,
                                                 (__attribute__((address_space(3))) void *)(fstage + 16 * j),
                                                 16, 0, 0);
        }
    }

    // ---- an appended row outside the attended window is still written (split 0, hg 0)
    if (a.swa_new && s == 0 && hg == 0 && np_b >= 0 && !in_win && tid < kD / 32) {
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

    // The top-k row chain, pipelined across the stream's chunks: while chunk c is computed,
    // the block-table entry of the stream's next chunk and the top-k entry of the one after
    // are in flight (entry -1 / block -1: no row).  Reads are clamped into their rows and
    // masked, so no load sits behind a branch.
    auto entry_of = [&](int c, int32_t raw) -> int {
        const int rg = c * kAttnRows + r_loc;
        return c < nchunk && rg < a.k && rg < tl ? raw : -1;
    };
    auto topk_at = [&](int c) -> int { return entry_of(c, topk_raw(c)); };
    auto block_of = [&](int p) -> int64_t {
        const bool in = p >= 0 && p < L;
        const int64_t ph = a.table[(int64_t)b * a.tstride + (in ? p : 0) / kBlk];
        return in && ph >= 0 && ph < a.n_blocks ? ph : -1;
    };
    int p_cur = entry_of(c_first, e_first), p_nxt = entry_of(c_first + cstep, e_second);
    // whether chunk c holds a row to attend (uniform: a function of the sequence's lengths)
    auto chunk_rows = [&](int c) -> bool {
        const int r0 = c * kAttnRows, r1 = r0 + kAttnRows, wend = a.k + min(nwin, a.W);
        return c < nchunk && (r0 < min(tl, a.k) || (r1 > a.k && r0 < wend));
    };
    int64_t ph_cur = block_of(p_cur);
    if (NS == 2) __syncthreads();  // the query tile is in LDS

    // the split's chunks in steps of NS: stream st takes chunk c0 + nsplit st
    for (int c0 = s; c0 < nchunk; c0 += cstep) {
        const int c = c0 + a.nsplit * st;
        const int rg = c * kAttnRows + r_loc;
        // ---- locate this lane's row (none when the stream's chunk is past the last)
        const uint8_t *rp = nullptr;
        bool fp8 = false, fresh = false;
        if (c >= nchunk) {
        } else if (rg < a.k) {
            if (ph_cur >= 0)
                rp = a.kv + ph_cur * (kBlk * (kD / 2 + kD / 32)) + (p_cur % kBlk) * (kD / 2 + kD / 32);
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
        {  // the chain of the next chunks (see above)
            const int64_t ph_nxt = block_of(p_nxt);
            const int p_nn = topk_at(c + 2 * cstep);
            p_cur = p_nxt;
            ph_cur = ph_nxt;
            p_nxt = p_nn;
        }
        // ---- this lane's row bytes: a main row's 64 code bytes and 4 scale bytes of dims
        //      g4*128 .., a window row's 128 and 4 (the appended row comes from LDS instead).
        //      They are requested before the barriers below, so that they overlap them.
        uint4 uu[8];
        uint32_t sc4 = 0u;
        auto load_row = [&] {
            if (valid && !fresh) {
                const uint4 *src = reinterpret_cast<const uint4 *>(rp + g4 * (fp8 ? 128 : 64));
                if (fp8) {
#pragma unroll
                    for (int i = 0; i < 8; i++) uu[i] = src[i];
                    sc4 = *reinterpret_cast<const uint32_t *>(rp + kD + 4 * g4);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) uu[i] = src[i];
                    sc4 = *reinterpret_cast<const uint32_t *>(rp + kD / 2 + 4 * g4);
                }
            }
        };
        // ---- the appended row, when this stream's chunk attends it: the stream's first wave
        //      quantises it from the staged fp32 row into LDS (and, for the first head group,
        //      into the ring), four lanes per 32-group (8 elements each, the group's amax by a
        //      quad max).  NS = 2 does it before the barriers below, which then order the
        //      writes before its lane reads them; NS = 1 after them, behind a barrier of its own.
        auto quant_fresh = [&] {
        if (c == fc && ts < kWave) {
            const int g = ts >> 2, qq = ts & 3;  // group, quarter of the group
            const float4 t0 = fstage[16 * (2 * qq) + g], t1 = fstage[16 * (2 * qq + 1) + g];
            const float v[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i++) am = fmaxf(am, fabsf(v[i]));
            am = fmaxf(am, dpp_f<0xB1>(am));  // quad [1,0,3,2]
            am = fmaxf(am, dpp_f<0x4E>(am));  // quad [2,3,0,1]
            const int e = group_exponent(am, 8);
            uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                w0 |= fp8_code(v[j], e) << (8 * j);
                w1 |= fp8_code(v[4 + j], e) << (8 * j);
            }
            const uint2 w01 = make_uint2(w0, w1);
            *reinterpret_cast<uint2 *>(sh.fresh_row + 32 * g + 8 * qq) = w01;
            if (qq == 0) sh.fresh_row[kD + g] = (uint8_t)(e + 127);
            if (hg == 0) {
                uint8_t *dst = a.swa_out + ((int64_t)b * a.rstride + np_b % a.C) * (kD + kD / 32);
                *reinterpret_cast<uint2 *>(dst + 32 * g + 8 * qq) = w01;
                if (qq == 0) dst[kD + g] = (uint8_t)(e + 127);
            }
        }
        };
        load_row();
        if (NS == 2) {
            quant_fresh();
            // this lane's query slice, while the row bytes are in flight (held only until S,
            // so that P V has the registers to read its V tiles ahead)
#pragma unroll
            for (int t = 0; t < 16; t++) {
                const uint4 u = qtile[c16 * 65 + g4 * 16 + t];
                qa[t] = *reinterpret_cast<const bf16x8_t *>(&u);
            }
        }
        if (!chunk_rows(c0) && !(NS == 2 && chunk_rows(c0 + a.nsplit))) continue;  // uniform
        __syncthreads();  // the previous chunks are done with V, P and the reductions
        if (NS == 1 && fc == c) {  // uniform: fc and c are the workgroup's
            quant_fresh();
            __syncthreads();
        }

        // ---- exact conversion to bf16, one piece kb = dims g4*128 + 8t .. +8 of the row at a
        //      time: stored to the V tile row-major and taken as the B operand of S = Q K^T
        //      for this wave's 16 rows and the 16 heads right away
        if (valid && fresh) {  // the appended row from LDS (bytewise scales: kept an LDS read)
            const uint4 *src = reinterpret_cast<const uint4 *>(sh.fresh_row + g4 * 128);
#pragma unroll
            for (int i = 0; i < 8; i++) uu[i] = src[i];
            const uint8_t *fs = sh.fresh_row + kD + 4 * g4;
            sc4 = fs[0] | (uint32_t)fs[1] << 8 | (uint32_t)fs[2] << 16 | (uint32_t)fs[3] << 24;
        }
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        auto kb_fp4 = [&](int t) {
            const uint32_t wd = word_of(uu[t >> 2], t & 3);
            const float sc = e8m0_to_f32((sc4 >> (8 * (t >> 2))) & 255u);
            return join4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 0),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 1),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 2),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 3));
        };
        auto kb_fp8 = [&](int t) {
            const uint32_t w0d = word_of(uu[t >> 1], 2 * (t & 1)), w1d = word_of(uu[t >> 1], 2 * (t & 1) + 1);
            const float sc = e8m0_to_f32((sc4 >> (8 * (t >> 2))) & 255u);
            return join4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0d, sc, false),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0d, sc, true),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1d, sc, false),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1d, sc, true));
        };
        auto put = [&](int t, bf16x8_t kb) {
            *reinterpret_cast<bf16x8_t *>(&sh.vt[r_loc * kVStride + g4 * 128 + 8 * t]) = kb;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], kb, acc, 0, 0, 0);
        };
        // wave-uniform fast paths (every row of the wave a main row, or every row a window
        // row) keep branches out of the 16 steps
        if (__all(valid && !fp8)) {
#pragma unroll
            for (int t = 0; t < 16; t++) put(t, kb_fp4(t));
        } else if (__all(valid && fp8)) {
#pragma unroll
            for (int t = 0; t < 16; t++) put(t, kb_fp8(t));
        } else {
#pragma unroll
            for (int t = 0; t < 16; t++) {
                bf16x8_t kb;
                if (valid && !fp8) kb = kb_fp4(t);
                else if (valid) kb = kb_fp8(t);
                else
#pragma unroll
                    for (int i = 0; i < 8; i++) kb[i] = (__bf16)0.0f;
                put(t, kb);
            }
        }
        // lane holds S[head 4*g4 + j][row c16 of this wave]
        float sv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            sv[j] = valid ? acc[j] : -INFINITY;
            const float m = row16_max(sv[j]);
            if (c16 == 0) sh.red_m[wave][4 * g4 + j] = m;
        }
        __syncthreads();  // V and the row maxima are in LDS
        // new running maxima, rescale factors, probabilities of this lane's row (a stream
        // whose chunk has no row keeps its state: mn = M, alpha = 1, p = 0)
        float alpha[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int h = 4 * g4 + j;
            const float mc = fmaxf(fmaxf(sh.red_m[0][h], sh.red_m[1][h]), fmaxf(sh.red_m[2][h], sh.red_m[3][h]));
            const float mn = fmaxf(M[j], mc);
            alpha[j] = M[j] == mn ? 1.0f : exp2f((M[j] - mn) * a.scale_log2);  // 0 for a first row
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
        // this lane's transpose-read address: rows 8 g4 + c16/4 (+ 32 ks), dims 4 (c16 % 4) (+ 16 nt)
        const __bf16 *vrow = &sh.vt[(8 * g4 + (c16 >> 2)) * kVStride + 4 * (c16 & 3)];
#pragma unroll
        for (int n = 0; n < 8; n++) {
            const int nt = 8 * wave + n;
#pragma unroll
            for (int j = 0; j < 4; j++) o[n][j] *= alpha[j];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const bf16x8_t vb = v_rows8(vrow + 32 * ks * kVStride + 16 * nt);
                o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[ks], vb, o[n], 0, 0, 0);
                o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[ks], vb, o[n], 0, 0, 0);
            }
        }
    }

    // ---- the two streams' states join through LDS: stream st finishes column tiles
    //      4 st .. 4 st + 3 of its waves (ok) and hands the other four (og) to the other
    //      stream through its own V tile (free now); both arrive at the same M and sum (the
    //      same two products added, in either order).  The halves are picked by selects, so
    //      that the LDS reads are issued together.
    f32x4_t ok[4];
    if (NS == 2) {
    __syncthreads();  // both streams are done with their V tiles
    float *xo_out = reinterpret_cast<float *>(shs[st].vt);
    const float *xo_in = reinterpret_cast<const float *>(shs[NS - 1 - st].vt);
#pragma unroll
    for (int n = 0; n < 4; n++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            ok[n][j] = st ? o[n + 4][j] : o[n][j];
            xo_out[(4 * n + j) * kStreamThreads + ts] = st ? o[n][j] : o[n + 4][j];
        }
    if (c16 == 0)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            shs[st].red_m[wave][4 * g4 + j] = M[j];
            shs[st].red_l[wave][4 * g4 + j] = lsum[j];
        }
    __syncthreads();
    float xi[4][4];
#pragma unroll
    for (int n = 0; n < 4; n++)
#pragma unroll
        for (int j = 0; j < 4; j++) xi[n][j] = xo_in[(4 * n + j) * kStreamThreads + ts];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float m1 = shs[NS - 1 - st].red_m[wave][4 * g4 + j], l1 = shs[NS - 1 - st].red_l[wave][4 * g4 + j];
        const float mn = fmaxf(M[j], m1);
        const float a0 = M[j] == mn ? 1.0f : exp2f((M[j] - mn) * a.scale_log2);
        const float a1 = m1 == mn ? 1.0f : exp2f((m1 - mn) * a.scale_log2);
        M[j] = mn;
        lsum[j] = lsum[j] * a0 + l1 * a1;
#pragma unroll
        for (int n = 0; n < 4; n++) ok[n][j] = ok[n][j] * a0 + xi[n][j] * a1;
    }
    }
    // the column tiles this thread writes: NS = 2 tiles 4 st + n of ok, NS = 1 all of o
    constexpr int NT = NS == 2 ? 4 : 8;
    auto tile_val = [&](int n) -> const f32x4_t & { return NS == 2 ? ok[n] : o[n]; };
    const int nt0 = NS == 2 ? 4 * st : 0;

    if (a.nsplit == 1) {
#pragma unroll
        for (int n = 0; n < NT; n++) {
            const int d = 16 * (8 * wave + nt0 + n) + c16;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int h = hg * 16 + 4 * g4 + j;
                a.out[((int64_t)b * a.Hq + h) * kD + d] = lsum[j] > 0.0f ? tile_val(n)[j] * (1.0f / lsum[j]) : 0.0f;
            }
        }
        if (st == 0) {
            if (wave == 0 && c16 == 0)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    a.lse[(int64_t)b * a.Hq + hg * 16 + 4 * g4 + j] =
                        lsum[j] > 0.0f ? a.sm_scale * M[j] + logf(lsum[j]) : -INFINITY;
        }
        return;
    }
    // The partial state goes out with agent-scope stores, which write through this XCD's L2
    // to memory.  The last split of (b, hg) to arrive combines them all: every wave waits for
    // its own partial stores to complete before the barrier, thread 0 then counts the split
    // in (a relaxed agent-scope atomic), and the last split reads the partials with
    // agent-scope loads.  Write-through stores and coherent loads replace a release fence and
    // an acquire, whose L2 write-back and invalidation many splits would otherwise run at once.
    auto put_coherent = [](float *p, float v) {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    {
        const int64_t pbase = ((int64_t)b * a.nsplit + s) * a.Hq + hg * 16;
        if (st == 0 && wave == 0 && c16 == 0)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int64_t i = pbase + 4 * g4 + j;
                put_coherent(a.part_ml + 2 * i, lsum[j] > 0.0f ? M[j] : -INFINITY);
                put_coherent(a.part_ml + 2 * i + 1, lsum[j]);
            }
        if (lsum[0] > 0.0f || lsum[1] > 0.0f || lsum[2] > 0.0f || lsum[3] > 0.0f) {
            float *po = a.part_o + pbase * kD;
#pragma unroll
            for (int n = 0; n < NT; n++) {
                const int d = 16 * (8 * wave + nt0 + n) + c16;
#pragma unroll
                for (int j = 0; j < 4; j++) put_coherent(po + (4 * g4 + j) * kD + d, tile_val(n)[j]);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int32_t *const cnt = a.count + (int64_t)b * a.HG + hg;
    if (tid == 0)
        shs[0].last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      a.nsplit - 1;
    __syncthreads();
    if (!shs[0].last) return;  // uniform
    merge_splits<NS>(a, b, hg);
    if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace csa2

using namespace csa2;

namespace {

// ------------------------------------------------------------------ static scratch
//
// csa2_sparse_attn_noalloc keeps the split partials and arrival counters of its calls in
// this file-scope device array instead of a caller workspace; each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, so its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address reaches kernels.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

__global__ void k_zero_words(int32_t *p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0;
}

// The scratch address of the current device; on the first call for a device its arrival
// counters are cleared (a fill kernel on `stream`), after which every call leaves them at
// zero again.
int scratch_of_current_device(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA2_ERR_HIP;
        k_zero_words<<<(kAttnCounters + 255) / 256, 256, 0, stream>>>((int32_t *)p, kAttnCounters);
        if (hipGetLastError() != hipSuccess) return CSA2_ERR_HIP;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return CSA2_OK;
}

int sparse_attn(const csa2_config *c, const float *swa_new, const int32_t *new_pos,
                int32_t new_pos_off, const uint16_t *q, const uint8_t *kv_cache, int64_t n_blocks,
                const int32_t *block_table, int32_t maxb, const uint8_t *swa_cache,
                uint8_t *swa_out, int32_t C, const int32_t *ctx_len, int32_t q_pos0,
                int32_t batch, const int32_t *topk, const int32_t *topk_len, float *out,
                float *lse, void *ws, size_t ws_bytes, hipStream_t stream,
                bool use_scratch = false, bool dry = false) {
    if (!c || !q || !kv_cache || n_blocks <= 0 || !block_table || maxb <= 0 ||
        batch < 0 || !topk || !topk_len || !out || !lse || (!ws && !use_scratch))
        return CSA2_ERR_INVALID;
    if (const int st = attn_cfg_status(c); st == CSA2_ERR_INVALID) return st;
    if (c->swa_window > 0 && (!swa_cache || C < c->swa_window)) return CSA2_ERR_INVALID;
    if (swa_new && (!new_pos || !swa_out || C <= 0)) return CSA2_ERR_INVALID;
    if (const int st = attn_cfg_status(c)) return st;
    const AttnPlan plan = attn_plan(batch, c->n_q_heads, c->topk, c->swa_window);
    const int nsplit = plan.nsplit;
    // (the plan splits only batches of fewer than kAttnCounters (sequence, head group) pairs)
    if (nsplit > 1 && (int64_t)batch * (c->n_q_heads / 16) > kAttnCounters) return CSA2_ERR_HIP;
    const WsAttn wl = ws_attn(batch, c->n_q_heads, c->kv_dim, nsplit);
    if (use_scratch) {
        if (wl.total > kScratchBytes) return CSA2_ERR_SCRATCH;
        if (batch == 0) return CSA2_OK;
        const int st = scratch_of_current_device(stream, &ws);
        if (st) return st;
        ws_bytes = kScratchBytes;
    }
    if (ws_bytes < wl.total) return CSA2_ERR_WORKSPACE;
    if (batch == 0 || dry) return CSA2_OK;
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
    a.new_pos_off = new_pos_off;
    a.swa_out = swa_out;
    if (plan.ns == 2) k_attn<2><<<dim3(nsplit, batch * a.HG), 2 * kStreamThreads, 0, stream>>>(a);
    else k_attn<1><<<dim3(nsplit, batch * a.HG), kStreamThreads, 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

}  // namespace

namespace csa2 {

// The window append of the token at position ctx_len[b] - 1 fused with attention (the layer
// calls): csa2_sparse_attn_append with pos = ctx_len - 1.
int sparse_attn_layer(const csa2_config *c, const float *swa_rows, const uint16_t *q,
                      const uint8_t *kv_cache, int64_t n_blocks, const int32_t *block_table,
                      int32_t maxb, uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                      int32_t batch, const int32_t *topk, const int32_t *topk_len, float *out,
                      float *lse, void *ws, size_t ws_bytes, hipStream_t stream, bool dry) {
    if (!swa_rows || !swa_cache || !ctx_len) return CSA2_ERR_INVALID;
    // (a dry run checks the host-side arguments; topk may not exist yet, any non-null stands in)
    const int32_t *tk = dry && !topk ? ctx_len : topk, *tl = dry && !topk_len ? ctx_len : topk_len;
    return sparse_attn(c, swa_rows, ctx_len, -1, q, kv_cache, n_blocks, block_table, maxb,
                       swa_cache, swa_cache, C, ctx_len, 0, batch, tk, tl, out, lse, ws,
                       ws_bytes, stream, false, dry);
}

}  // namespace csa2

extern "C" int csa2_sparse_attn(const csa2_config *c, const uint16_t *q, const uint8_t *kv_cache,
                                int64_t n_blocks, const int32_t *block_table, int32_t maxb,
                                const uint8_t *swa_cache, int32_t C, const int32_t *ctx_len,
                                int32_t batch, const int32_t *topk, const int32_t *topk_len,
                                float *out, float *lse, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
    if (!ctx_len) return CSA2_ERR_INVALID;
    return sparse_attn(c, nullptr, nullptr, 0, q, kv_cache, n_blocks, block_table, maxb, swa_cache,
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
    // the ring must still hold the oldest attended window row of the chunk's first query
    if (c && c->swa_window > 0 && n_q > 0 && (int64_t)C < (int64_t)n_q + c->swa_window - 1)
        return CSA2_ERR_INVALID;
    return sparse_attn(c, nullptr, nullptr, 0, q, kv_cache, n_blocks, block_table, maxb, swa_ring,
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
    return sparse_attn(c, swa_rows, pos, 0, q, kv_cache, n_blocks, block_table, maxb, swa_cache,
                       swa_cache, C, ctx_len, 0, batch, topk, topk_len, out, lse, ws, ws_bytes,
                       stream);
}

extern "C" int csa2_sparse_attn_noalloc(const csa2_config *c, const uint16_t *q,
                                        const uint8_t *kv_cache, int64_t n_blocks,
                                        const int32_t *block_table, int32_t maxb,
                                        const uint8_t *swa_cache, int32_t C,
                                        const int32_t *ctx_len, int32_t batch,
                                        const int32_t *topk, const int32_t *topk_len, float *out,
                                        float *lse, hipStream_t stream) {
    if (!ctx_len) return CSA2_ERR_INVALID;
    return sparse_attn(c, nullptr, nullptr, 0, q, kv_cache, n_blocks, block_table, maxb, swa_cache,
                       nullptr, C, ctx_len, 0, batch, topk, topk_len, out, lse, nullptr, 0, stream,
                       true);
}
