// csa2_select.hip -- the per-sequence selection of the hierarchical indexer: the pool of
// the K_blk best blocks and the k best positions inside it (Full), or the k best rescored
// pool positions (Reindex).
//
// What runs (dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心"; and
// prism.simon-ai.net/article/7901, "层级稀疏索引器：精准筛选关键信息"): the indexer keeps a
// pool of the best 8-position blocks and then the best positions inside the pool.
//
// Selection order: score descending, lower index first on equal scores; outputs ascending.
// Scores are compared through an order-preserving map to uint32 (s is never -0 or NaN).
//
// Pool selection without a full pass over the block maxima: with m_g the maximum of group
// g (8 consecutive blocks) and lambda the K_blk-th largest m_g, K_blk distinct blocks (the
// group maxima) score >= lambda, so the K_blk-th largest block score is >= lambda.  Every
// pool block therefore lies in a group with m_g >= lambda and scores >= lambda itself;
// only those blocks (about K_blk of them on unstructured data) enter the exact selection.
#include "csa2_block.h"
#include "csa2_select.h"

namespace csa2 {

// ------------------------------------------------------------------ exact block-wide select
//
// The K largest of a multiset of uint32 keys, lower index first among equal keys.  The
// digits adapt to the keys present: each pass histograms the current key range [lo, hi]
// into at most 2048 bins of width 2^s (LDS), keeps the bin that holds the K-th largest and
// narrows the range to it, so scores crowded into a few binades still spread over the
// bins.  Result: an item is selected iff key > thr, or key == thr and fewer than `need`
// such items precede it in index order.

constexpr int kSelThreads = 1024;
constexpr int kIPT = 16;                            // register items per thread
constexpr int kRegCap = kSelThreads * kIPT;         // 16384
constexpr int kHistBins = 2048;
constexpr uint32_t kAllTies = 0xFFFFFFFFu;

struct SelShared {
    __align__(16) uint32_t hist[kHistBins];  // reversed: hist[nbins - 1 - bin]; zero between passes
    __align__(16) uint32_t scan[kSelThreads / kWave];
    __align__(16) uint32_t red[3][kSelThreads / kWave];
    uint32_t res[4];
};

struct SelResult {
    uint32_t thr;
    uint32_t need;
};

// Block-wide min, max and sum of (lo, hi, n).
__device__ __forceinline__ void block_min_max_count(uint32_t &lo, uint32_t &hi, uint32_t &n,
                                                    SelShared &sm) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    lo = wave_reduce_to63(lo, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
    hi = wave_reduce_to63(hi, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
    n = wave_reduce_to63(n, [](uint32_t x, uint32_t y) { return x + y; });
    __syncthreads();
    if (lane == kWave - 1) {
        sm.red[0][wave] = lo;
        sm.red[1][wave] = hi;
        sm.red[2][wave] = n;
    }
    __syncthreads();
    lo = 0xFFFFFFFFu;
    hi = 0u;
    n = 0u;
#pragma unroll
    for (int i = 0; i < kSelThreads / kWave; i += 4) {
        const uint4 a4 = *reinterpret_cast<const uint4 *>(&sm.red[0][i]);
        const uint4 b4 = *reinterpret_cast<const uint4 *>(&sm.red[1][i]);
        const uint4 c4 = *reinterpret_cast<const uint4 *>(&sm.red[2][i]);
        lo = min(min(min(lo, a4.x), min(a4.y, a4.z)), a4.w);
        hi = max(max(max(hi, b4.x), max(b4.y, b4.z)), b4.w);
        n += c4.x + c4.y + c4.z + c4.w;
    }
}

// Exact K-th largest of a multiset of uint32 keys (items owned by the threads; Src::each(f)
// calls f(key) for each item, and may also call it with key 0, which stands for no item:
// real keys are >= 1 because no score is NaN), K >= 1 and <= the number of items.  Each
// pass histograms the current key range [lo, hi] into <= 2048 bins of width 2^s in LDS and
// narrows the range to the bin that holds the K-th largest.  All threads scan the bins
// (two per thread, highest bin first), so a pass costs three barriers and no serial
// section.  The lowest bin gets no atomics after the first pass: its count is the range's
// item count minus the other bins (a pile of equal minimal keys, such as scores that are
// exactly 0 after the ReLU, never serialises on one LDS address).
// Result: an item is selected iff key > thr, or key == thr and fewer than `need` such items
// precede it in index order (need == kAllTies: all of them).
// With `bounded`, every key lies in [lo0, hi0] (lo0 >= 1) and the caller's bounds replace
// the block-wide min / max / count: the first pass then counts the lowest bin with atomics
// too.  max_out (unbounded only) receives the largest key.
template <class Src>
__device__ __forceinline__ SelResult range_select(const Src &src, uint32_t K, SelShared &sm,
                                                  bool bounded = false, uint32_t lo0 = 0u,
                                                  uint32_t hi0 = 0u, uint32_t *max_out = nullptr) {
    const int tid = threadIdx.x, lane = lane_id(), wave = threadIdx.x / kWave;
    uint32_t lo = lo0, hi = hi0, n_in = 0u;
    bool imp0 = !bounded;  // the lowest bin counted implicitly (n_in known)
    if (!bounded) {
        lo = 0xFFFFFFFFu;
        hi = 0u;
        src.each([&](uint32_t key) {
            lo = min(lo, key ? key : 0xFFFFFFFFu);
            hi = max(hi, key);
            n_in += key != 0u;
        });
        block_min_max_count(lo, hi, n_in, sm);
        if (max_out) *max_out = hi;
    }
    uint32_t remaining = K;
#pragma unroll 1
    for (int pass = 0; pass < 6 && lo != hi; pass++) {
        const uint32_t w = hi - lo;
        const int s = max(0, 32 - __clz((int)w) - 11);  // (w >> s) < 2048
        const int nbins = (int)(w >> s) + 1;
        const int li0 = nbins - 1;                      // reversed index of the lowest bin
        // explicit bins: keys with lo + cut <= key <= hi (cut skips the implicit lowest bin)
        const uint32_t cut = imp0 ? (1u << s) : 0u;
        if (cut <= w) {
            const uint32_t wc = w - cut, base = lo + cut;
            src.each([&](uint32_t key) {
                const uint32_t off = key - base;  // wraps below the range (and for key 0)
                if (off <= wc) atomicAdd(&sm.hist[li0 - (int)((off + cut) >> s)], 1u);
            });
        }
        __syncthreads();
        // thread t: reversed bins 2t, 2t + 1 (read, then cleared for the next pass)
        const int r0 = 2 * tid;
        const int lim = imp0 ? li0 : li0 + 1;  // reversed bins below lim hold atomic counts
        uint2 hv = make_uint2(0u, 0u);
        if (r0 < lim) {
            hv = *reinterpret_cast<const uint2 *>(&sm.hist[r0]);
            *reinterpret_cast<uint2 *>(&sm.hist[r0]) = make_uint2(0u, 0u);
        }
        const uint32_t c0 = hv.x, c1 = r0 + 1 < lim ? hv.y : 0u, v = c0 + c1;
        const uint32_t incl = wave_incl_scan(v);
        if (lane == kWave - 1) sm.scan[wave] = incl;
        __syncthreads();
        uint32_t pw = 0u, total = 0u;
#pragma unroll
        for (int i = 0; i < kSelThreads / kWave; i += 4) {
            const uint4 q = *reinterpret_cast<const uint4 *>(&sm.scan[i]);
            const uint32_t x[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                pw += i + j < wave ? x[j] : 0u;
                total += x[j];
            }
        }
        const uint32_t before = pw + incl - v;
        if (remaining <= total) {
            if (before < remaining && remaining <= before + v) {
                const bool first = remaining <= before + c0;
                sm.res[0] = (uint32_t)(li0 - (first ? r0 : r0 + 1));
                sm.res[1] = first ? before : before + c0;
                sm.res[2] = first ? c0 : c1;
            }
        } else if (tid == 0) {  // the implicit lowest bin (imp0 only)
            sm.res[0] = 0u;
            sm.res[1] = total;
            sm.res[2] = n_in - total;
        }
        __syncthreads();
        const uint32_t d = sm.res[0], above = sm.res[1], cnt = sm.res[2];
        remaining -= above;
        n_in = cnt;
        imp0 = true;
        const uint32_t nlo = lo + (d << s);
        if (cnt == remaining) return {nlo, kAllTies};  // the whole bin is needed
        const uint64_t top = (uint64_t)nlo + ((1ull << s) - 1ull);
        hi = (uint32_t)min((uint64_t)hi, top);
        lo = nlo;
    }
    return {lo, remaining};
}

template <int N>
struct RegItems {
    uint32_t key[N];  // 0: no item
    template <class F>
    __device__ __forceinline__ void each(F f) const {
#pragma unroll
        for (int i = 0; i < N; i++) f(key[i]);
    }
    __device__ __forceinline__ uint32_t count() const {
        uint32_t n = 0;
#pragma unroll
        for (int i = 0; i < N; i++) n += key[i] != 0u;
        return n;
    }
};

// Ordered emission of the selected items of a register set whose items are in index order
// within the thread and threads in index order.  One packed scan gives, per thread, the
// items above the threshold and the ties before it; ties are taken lowest index first, so
// min(need, ties before) of them precede the thread's own.  `tie_base` / `out_base` carry
// the ties seen and items written by earlier chunks; both are advanced.  id(i) is written to
// out[position] for selected items (positions < out_cap).  Counts per chunk < 2^16.
template <int N, class IdF>
__device__ __forceinline__ void emit_selected(const RegItems<N> &it, IdF id, SelResult r,
                                              int32_t *out, uint32_t out_cap,
                                              uint32_t &tie_base, uint32_t &out_base,
                                              SelShared &sm) {
    uint32_t ngt = 0, neq = 0;  // thr >= 1, so absent items (key 0) count in neither
#pragma unroll
    for (int i = 0; i < N; i++) {
        ngt += it.key[i] > r.thr;
        neq += it.key[i] == r.thr;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kSelThreads>((ngt << 16) | neq, sm.scan, &tot);
    const uint32_t gt_before = ex >> 16, eq_before = ex & 0xFFFFu;
    uint32_t tr = tie_base + eq_before;  // ties before this thread's first item
    const uint32_t need = r.need;
    uint32_t o = out_base + gt_before + min(need, tr) - min(need, tie_base);
    const uint32_t all_gt = tot >> 16, all_eq = tot & 0xFFFFu;
    out_base += all_gt + (need == kAllTies ? all_eq : min(all_eq, need > tie_base ? need - tie_base : 0u));
    tie_base += all_eq;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const bool eq = it.key[i] == r.thr;
        const bool take = it.key[i] > r.thr || (eq && tr < need);
        tr += eq;
        if (take && o < out_cap) out[o] = id(i);
        o += take;
    }
}

// Select-all variant (fewer items than requested): every item in order.
template <int N, class IdF>
__device__ __forceinline__ void emit_all(const RegItems<N> &it, IdF id, int32_t *out,
                                         uint32_t out_cap, uint32_t &out_base, SelShared &sm) {
    uint32_t tot;
    uint32_t o = out_base + block_excl_scan<kSelThreads>(it.count(), sm.scan, &tot);
    out_base += tot;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const bool take = it.key[i] != 0u;
        if (take && o < out_cap) out[o] = id(i);
        o += take;
    }
}

// ------------------------------------------------------------------ k_select

// SelectArgs: csa2_select.h

struct SelectShared {
    SelShared sel;
    int32_t flag[2 * kSelThreads];         // flagged groups (ascending)
    int32_t pool[CSA2_MAX_POOL_BLOCKS];    // pool blocks (ascending)
};

// Exact top-K (K >= 1) of a register set (index order), emitted ascending into out.  The
// multiset must hold >= K items.
template <int N, class IdF>
__device__ __forceinline__ SelResult select_emit(const RegItems<N> &it, IdF id, uint32_t K,
                                                 int32_t *out, uint32_t out_cap, SelectShared &sm,
                                                 bool bounded = false, uint32_t lo0 = 0u,
                                                 uint32_t hi0 = 0u) {
    uint32_t tie_base = 0, out_base = 0;
    const SelResult r = range_select(it, K, sm.sel, bounded, lo0, hi0);
    emit_selected(it, id, r, out, out_cap, tie_base, out_base, sm.sel);
    return r;
}

// Block maxima of one sequence: block j at base[(j/8)*gstride + j%8] (groups of 8 blocks
// are contiguous).
struct BlockRow {
    const float *base;
    int64_t gstride;
    __device__ __forceinline__ float operator[](int j) const { return base[(j >> 3) * gstride + (j & 7)]; }
    __device__ __forceinline__ const float *group(int g) const { return base + g * gstride; }
};

// Items of the streaming path: all blocks j < nb whose maximum is >= lam, in chunks of kRegCap.
__device__ __forceinline__ void load_block_chunk(const BlockRow &bs, int nb, uint32_t lam, int c0,
                                                 RegItems<kIPT> &it) {
    const int j0 = c0 + (int)threadIdx.x * kIPT;
#pragma unroll
    for (int i = 0; i < kIPT; i++) {
        const int j = j0 + i;
        it.key[i] = 0u;
        if (j < nb) {
            const uint32_t key = order_key(bs[j]);
            it.key[i] = key >= lam ? key : 0u;
        }
    }
}

struct GlobalBlocks {
    BlockRow bs;
    int nb;
    uint32_t lam;
    template <class F>
    __device__ __forceinline__ void each(F f) const {
        for (int j = threadIdx.x; j < nb; j += kSelThreads) {
            const uint32_t key = order_key(bs[j]);
            if (key >= lam) f(key);
        }
    }
};

// Pool of the Full layer: the K_blk best blocks of sequence b, ascending, into sm.pool.
// Returns the pool length.
//   1. lambda = K_blk-th largest group maximum (exact select over <= 16384 group maxima
//      in registers), or no bound when there are at most K_blk groups;
//   2. the groups with maximum >= lambda, in ascending order (LDS), two per thread: their
//      blocks scoring >= lambda are the candidates;
//   3. exact select of K_blk among the candidates, ordered emission.
// More than 2048 such groups (heavy ties) or more than 16384 groups take a streaming path
// over all block maxima instead.
// *thr receives the pool's threshold key (every pool block's maximum is >= it; 0 when the
// pool holds every block).
__device__ __forceinline__ int select_pool(const SelectArgs &a, int b, int nb, SelectShared &sm,
                                           const float4 (&graw)[kIPT / 4], uint32_t *thr,
                                           uint32_t *kmax) {
    const int tid = threadIdx.x, K = a.K_blk;
    *thr = 0u;
    *kmax = 0u;  // largest block key when known (0: unknown)
    if (nb <= K) {
        for (int j = tid; j < nb; j += kSelThreads) sm.pool[j] = j;
        __syncthreads();
        return nb;
    }
    const BlockRow bs{a.bscore + (int64_t)b * a.bs_b, a.bs_g};
    const int ng = (nb + kItemBlocks - 1) / kItemBlocks;
    uint32_t lam = 0u;  // lower bound of the K-th largest block key
    bool fast = ng <= kRegCap;
    if (fast) {
        // group maxima (already loaded): thread t owns groups [t*16, t*16 + 16)
        RegItems<kIPT> g;
        const int g0 = tid * kIPT;
#pragma unroll
        for (int i = 0; i < kIPT; i += 4) {
            const float4 v = graw[i / 4];
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int t = 0; t < 4; t++) g.key[i + t] = g0 + i + t < ng ? order_key(f[t]) : 0u;
        }
        if (ng > K) lam = range_select(g, (uint32_t)K, sm.sel, false, 0u, 0u, kmax).thr;
        // ascending list of the groups whose maximum is >= lam
        uint32_t fl = 0;
#pragma unroll
        for (int i = 0; i < kIPT; i++)
            fl |= g.key[i] != 0u && g.key[i] >= lam ? 1u << i : 0u;
        uint32_t nfg;
        uint32_t o = block_excl_scan<kSelThreads>((uint32_t)__popc(fl), sm.sel.scan, &nfg);
        if (nfg <= 2u * kSelThreads) {
#pragma unroll
            for (int i = 0; i < kIPT; i++)
                if (fl & (1u << i)) sm.flag[o++] = g0 + i;
        }
        __syncthreads();
        if (nfg <= 2u * kSelThreads) {
            // candidates: blocks >= lam of flagged groups 2t and 2t+1.  Both groups' maxima
            // are requested before either is used (one memory round trip); an absent group
            // reads group 0 and blocks past nb (in the last group's row) are masked.
            RegItems<kIPT> c;
            int gid[2];
            float4 x[2][2];
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const int fi = 2 * tid + q;
                gid[q] = fi < (int)nfg ? sm.flag[fi] : -1;
                const float4 *src = reinterpret_cast<const float4 *>(bs.group(max(gid[q], 0)));
                x[q][0] = src[0];
                x[q][1] = src[1];
            }
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const float v[kItemBlocks] = {x[q][0].x, x[q][0].y, x[q][0].z, x[q][0].w,
                                              x[q][1].x, x[q][1].y, x[q][1].z, x[q][1].w};
#pragma unroll
                for (int t = 0; t < kItemBlocks; t++) {
                    const int i = q * kItemBlocks + t;
                    const uint32_t key = order_key(v[t]);
                    c.key[i] = gid[q] >= 0 && gid[q] * kItemBlocks + t < nb && key >= lam ? key : 0u;
                }
            }
            // every candidate key lies in [lam, largest group maximum]
            *thr = select_emit(c, [&](int i) { return gid[i / kItemBlocks] * kItemBlocks + i % kItemBlocks; },
                               (uint32_t)K, sm.pool, (uint32_t)K, sm, *kmax != 0u, lam, *kmax).thr;
        } else {
            fast = false;
        }
    }
    if (!fast) {
        // streaming path: every block maximum >= lam, in chunks of kRegCap
        uint32_t tie_base = 0, out_base = 0;
        GlobalBlocks src{bs, nb, lam};
        const SelResult r = range_select(src, (uint32_t)K, sm.sel);
        *thr = r.thr;
        for (int c0 = 0; c0 < nb; c0 += kRegCap) {
            RegItems<kIPT> c;
            load_block_chunk(bs, nb, lam, c0, c);
            emit_selected(c, [&](int i) { return c0 + tid * kIPT + i; }, r, sm.pool, (uint32_t)K,
                          tie_base, out_base, sm.sel);
        }
    }
    __syncthreads();
    return K;
}

// One histogram pass over the keys (0: no item) with two targets: lower edges of the bins
// holding the K1-th and the K2-th largest key (K1, K2 <= the number of keys); kmax (when
// given) receives the largest key.
template <class Src>
__device__ void two_bounds(const Src &src, uint32_t K1, uint32_t K2, SelShared &sm,
                           uint32_t *e1, uint32_t *e2, uint32_t *kmax = nullptr) {
    const int tid = threadIdx.x, lane = lane_id(), wave = threadIdx.x / kWave;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u, n = 0u;
    src.each([&](uint32_t key) {
        lo = min(lo, key ? key : 0xFFFFFFFFu);
        hi = max(hi, key);
        n += key != 0u;
    });
    block_min_max_count(lo, hi, n, sm);
    if (kmax) *kmax = n ? hi : 0u;
    if (n == 0u || lo >= hi) {  // no key, or all equal
        *e1 = *e2 = n ? lo : 0u;
        return;
    }
    const uint32_t w = hi - lo;
    const int s = max(0, 32 - __clz((int)w) - 11);  // (w >> s) < 2048
    const int nbins = (int)(w >> s) + 1, li0 = nbins - 1;
    src.each([&](uint32_t key) {
        const uint32_t off = key - lo;  // wraps for key 0
        if (key != 0u && off <= w) atomicAdd(&sm.hist[li0 - (int)(off >> s)], 1u);
    });
    __syncthreads();
    // thread t: reversed bins 2t, 2t + 1 (highest bin first), read and cleared
    const int r0 = 2 * tid;
    uint2 hv = make_uint2(0u, 0u);
    if (r0 < nbins) {
        hv = *reinterpret_cast<const uint2 *>(&sm.hist[r0]);
        *reinterpret_cast<uint2 *>(&sm.hist[r0]) = make_uint2(0u, 0u);
    }
    const uint32_t c0 = hv.x, c1 = r0 + 1 < nbins ? hv.y : 0u, v = c0 + c1;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == kWave - 1) sm.scan[wave] = incl;
    __syncthreads();
    uint32_t pw = 0u;
#pragma unroll
    for (int i = 0; i < kSelThreads / kWave; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(&sm.scan[i]);
        const uint32_t x[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; j++) pw += i + j < wave ? x[j] : 0u;
    }
    const uint32_t before = pw + incl - v;
    const uint32_t T[2] = {K1, K2};
#pragma unroll
    for (int i = 0; i < 2; i++)
        if (before < T[i] && T[i] <= before + v)
            sm.res[i] = (uint32_t)(li0 - (T[i] <= before + c0 ? r0 : r0 + 1));
    __syncthreads();
    *e1 = lo + (sm.res[0] << s);
    *e2 = lo + (sm.res[1] << s);
    __syncthreads();  // (res is written again by later selections)
}

// Top-k among the visible positions of the pool.  Thread t owns pool entries 2t and 2t+1.
// Only positions scoring >= a lower bound of the k-th largest position score are
// candidates.  Full: the pool threshold (each of the plen pool blocks has a position at
// its maximum, which is >= the threshold), valid when k <= plen.  Reindex: the k-th largest
// rescored block maximum among the pool entries (k distinct positions reach it); only
// entries whose maximum reaches it are read.  Scores come from the Full scan (pscore, by
// position) or from the Reindex rescoring (poolsc / poolbmax, by pool entry; -inf marks an
// invisible position).
template <bool REINDEX>
__device__ __forceinline__ void select_topk(const SelectArgs &a, int b, int L, const int32_t *pool,
                                            int plen, uint32_t pool_thr, uint32_t kmax,
                                            SelectShared &sm) {
    const int tid = threadIdx.x;
    // Everything read for the thread's pool entries e = 2t, 2t+1 is requested in one batch
    // (one memory round trip): Full, the position scores of the entries' blocks (the entry
    // itself comes from LDS); Reindex, the entry, its rescored maximum and its rescored
    // positions.  Reads of an absent entry are clamped into the row and masked below.
    int pj[2];
    float4 x[2][2];
    float bmax[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int e = 2 * tid + q;
        const int ec = min(e, a.K_blk - 1);
        const int pv = pool[ec];
        pj[q] = e < plen ? pv : -1;
        if (REINDEX) {
            bmax[q] = a.poolbmax[(int64_t)b * a.K_blk + ec];
            const float4 *src = reinterpret_cast<const float4 *>(a.poolsc + ((int64_t)b * a.K_blk + ec) * kBlk);
            x[q][0] = src[0];
            x[q][1] = src[1];
        }
    }
    // the maxima are only used under a condition: pinned here, so that their loads are not
    // sunk behind the entries' loads
    if (REINDEX) asm volatile("" : "+v"(bmax[0]), "+v"(bmax[1]));
    if (!REINDEX) {
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int pc = pj[q] >= 0 && pj[q] * kBlk < L ? pj[q] : 0;
            const float4 *src = reinterpret_cast<const float4 *>(a.pscore + (int64_t)b * a.ps_b + (int64_t)pc * a.ps_j);
            x[q][0] = src[0];
            x[q][1] = src[1];
        }
    }
    RegItems<2> bm;  // Reindex: block maxima of the thread's entries (0: no entry)
    uint32_t okm = 0, nvis = 0;  // okm bit q: entry q holds a visible block
#pragma unroll
    for (int q = 0; q < 2; q++) {  // branch-free, so that no load sinks behind another
        const bool ok = pj[q] >= 0 && pj[q] * kBlk < L;
        bm.key[q] = REINDEX && ok ? order_key(bmax[q]) : 0u;
        okm |= ok ? 1u << q : 0u;
        nvis += ok ? (uint32_t)min(kBlk, L - pj[q] * kBlk) : 0u;
    }
    uint32_t n_ent = __popc(okm);
    const uint32_t n_vis = block_sum<kSelThreads>((nvis << 16) | n_ent, sm.sel.scan);
    n_ent = n_vis & 0xFFFFu;
    const uint32_t need = min((uint32_t)a.k, n_vis >> 16);
    int32_t *out = a.topk + (int64_t)b * a.k;
    uint32_t lam = 0u;
    if (need > 0 && need < (n_vis >> 16) && need <= n_ent) {
        // Reindex: kmax receives the largest rescored block maximum, the upper end of every
        // candidate key
        // (a lower bound serves: one histogram pass gives the lower edge of the bin holding
        // the need-th largest rescored maximum, and the exact selection below is bounded by it)
        if (REINDEX && n_ent > need) {
            uint32_t e2;
            two_bounds(bm, need, need, sm.sel, &lam, &e2, &kmax);
        }
        else lam = pool_thr;
    }
    // candidate positions scoring >= lam (Reindex: of entries whose maximum reaches lam)
    RegItems<kIPT> it;
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const float sc[kBlk] = {x[q][0].x, x[q][0].y, x[q][0].z, x[q][0].w,
                                x[q][1].x, x[q][1].y, x[q][1].z, x[q][1].w};
        const bool live = (okm & (1u << q)) && (!REINDEX || bm.key[q] >= lam);
#pragma unroll
        for (int t = 0; t < kBlk; t++) {
            const int i = q * kBlk + t;
            const uint32_t key = order_key(sc[t]);
            it.key[i] = live && pj[q] * kBlk + t < L && (!REINDEX || sc[t] != -INFINITY) && key >= lam
                            ? key : 0u;
        }
    }
    if (need > 0) {
        auto pos = [&](int i) { return pj[i / kBlk] * kBlk + i % kBlk; };
        if (need == (n_vis >> 16) && lam == 0u) {
            uint32_t ob = 0;
            emit_all(it, pos, out, (uint32_t)a.k, ob, sm.sel);
        } else {
            // with a lower bound, every candidate key lies in [lam, largest key] (Full: the
            // largest group maximum; Reindex: the largest rescored block maximum)
            const bool bounded = lam != 0u && kmax != 0u;
            select_emit(it, pos, need, out, (uint32_t)a.k, sm, bounded, lam, kmax);
        }
    }
    for (int i = (int)need + tid; i < a.k; i += kSelThreads) out[i] = -1;
    if (tid == 0) a.topk_len[b] = (int32_t)need;
}

// Full mode in one workgroup: the pool from the group and block maxima, then the top-k inside
// it from the stored position scores, both written out.  graw: the thread's 16 group maxima.
__device__ __forceinline__ void full_select_one_wg(const SelectArgs &a, int b, int L, int nb,
                                                   SelectShared &sm, const float4 (&graw)[kIPT / 4]) {
    const int tid = threadIdx.x;
    uint32_t thr;
    uint32_t kmax;
    const int plen = select_pool(a, b, nb, sm, graw, &thr, &kmax);
    const int np = min(plen, nb);
    select_topk<false>(a, b, L, sm.pool, np, thr, kmax, sm);
    // the pool leaves last: stores complete in issue order with loads, so a store issued
    // before the top-k's score loads would have delayed their use by its write round trip
    int32_t *pool_out = a.pool_blocks + (int64_t)b * a.K_blk;
    for (int i = tid; i < a.K_blk; i += kSelThreads) pool_out[i] = i < np ? sm.pool[i] : -1;
    if (tid == 0) a.pool_len[b] = np;
}

template <bool REINDEX>
__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs a) {
    extern __shared__ __align__(16) uint8_t sh_raw[];
    SelectShared &sm = *reinterpret_cast<SelectShared *>(sh_raw);
    const int b = blockIdx.x, tid = threadIdx.x;
    // Full: the thread's 16 group maxima are requested before the sequence length arrives
    // (reads clamped into the allocated row of ngmax >= 4 floats; groups past the length are
    // masked, so a clamped read is never used)
    float4 graw[kIPT / 4];
    if (!REINDEX) {
        const float *gm = a.gmax + (int64_t)b * a.ngmax;
#pragma unroll
        for (int i = 0; i < kIPT / 4; i++) {
            const int gi = min(tid * kIPT + 4 * i, a.ngmax - 4);  // clamped into the row
            graw[i] = *reinterpret_cast<const float4 *>(gm + gi);
        }
    }
    const int L = clamp_len(a.ctx_len ? a.ctx_len[b] : a.q_pos0 + b + 1, a.maxb);
    if (!REINDEX) {  // pinned here, so that the loads are not sunk behind the length's branches
#pragma unroll
        for (int i = 0; i < kIPT / 4; i++)
            asm volatile("" : "+v"(graw[i].x), "+v"(graw[i].y), "+v"(graw[i].z), "+v"(graw[i].w));
    }
    const int nb = (L + kBlk - 1) / kBlk;
    for (int i = tid; i < kHistBins; i += kSelThreads) sm.sel.hist[i] = 0u;  // kept zero between passes
    __syncthreads();
    if (REINDEX) {
        const int plen = max(0, min(a.pool_len[b], a.K_blk));
        select_topk<true>(a, b, L, a.pool_blocks + (int64_t)b * a.K_blk, plen, 0u, 0u, sm);
        return;
    }
    full_select_one_wg(a, b, L, nb, sm, graw);
}

// ------------------------------------------------------------------ prefill in two passes
//
// The prefill scoring pass keeps block and group maxima only; the selection then runs in two
// phases around a second scoring pass that recomputes the position scores of the blocks the
// top-k can draw from.  With theta the k-th largest block maximum of the pool, the k pool
// blocks reaching it each hold a distinct position scoring >= theta, so the k-th best pool
// position scores >= theta and every top-k position lies in a pool block whose maximum is
// >= theta: those blocks (the flagged blocks) hold the whole candidate set.  When the pool
// has fewer than k blocks or at most k visible positions, every pool block is flagged.

// Query of workgroup `bid` of a grid of n: runs of 4 consecutive queries on one XCD (dispatch
// places workgroup i on XCD i % 8), whose block-maxima reads share cache lines (the layout
// puts 4 queries' 8 block maxima of a group in one 128-byte line).
__device__ __forceinline__ int pf_query_of(int bid, int n) {
    if (n % 32 != 0) return bid;
    const int x = bid % 8, slot = bid / 8;
    return 4 * (8 * (slot / 4) + x) + slot % 4;
}

// Phase 0, one workgroup per query: pool, theta, flagged blocks.  Built for 8 waves per SIMD
// (two workgroups per CU): thousands of these latency-bound selections run per chunk, and a
// second resident workgroup hides their barriers and round trips at the cost of a few spills.
__global__ __launch_bounds__(kSelThreads, 8) void k_select_pf_pool(SelectArgs a) {
    extern __shared__ __align__(16) uint8_t sh_raw[];
    SelectShared &sm = *reinterpret_cast<SelectShared *>(sh_raw);
    const int b = pf_query_of((int)blockIdx.x, (int)gridDim.x), tid = threadIdx.x;
    float4 graw[kIPT / 4];
    const float *gm = a.gmax + (int64_t)b * a.ngmax;
#pragma unroll
    for (int i = 0; i < kIPT / 4; i++) {
        const int gi = min(tid * kIPT + 4 * i, a.ngmax - 4);  // clamped into the row
        graw[i] = *reinterpret_cast<const float4 *>(gm + gi);
    }
    const int L = clamp_len(a.q_pos0 + b + 1, a.maxb);
    const int nb = (L + kBlk - 1) / kBlk;
    for (int i = tid; i < kHistBins; i += kSelThreads) sm.sel.hist[i] = 0u;
    __syncthreads();
    uint32_t thr, kmax;
    const int np = min(select_pool(a, b, nb, sm, graw, &thr, &kmax), nb);
    // block maxima and visible positions of the pool entries 2t, 2t+1
    const BlockRow bs{a.bscore + (int64_t)b * a.bs_b, a.bs_g};
    int pj[2];
    float v[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int e = 2 * tid + q;
        pj[q] = e < np ? sm.pool[e] : -1;
        v[q] = bs[max(pj[q], 0)];
    }
    RegItems<2> bm;
    uint32_t nvis = 0u;
#pragma unroll
    for (int q = 0; q < 2; q++) {
        bm.key[q] = pj[q] >= 0 ? order_key(v[q]) : 0u;
        nvis += pj[q] >= 0 ? (uint32_t)min(kBlk, L - pj[q] * kBlk) : 0u;
    }
    const uint32_t n_vis = block_sum<kSelThreads>(nvis, sm.sel.scan);
    uint32_t theta = 0u;
    if (np >= a.k && n_vis > (uint32_t)a.k) theta = range_select(bm, (uint32_t)a.k, sm.sel).thr;
    uint32_t fl = 0u;
#pragma unroll
    for (int q = 0; q < 2; q++) fl |= pj[q] >= 0 && bm.key[q] >= theta ? 1u << q : 0u;
    uint32_t cnt;
    uint32_t o = block_excl_scan<kSelThreads>((uint32_t)__popc(fl), sm.sel.scan, &cnt);
    int32_t *lst = a.pf_list + (int64_t)b * a.K_blk;
    // the query's flag words (word i: blocks 32i .. 32i + 31, i.e. word (i % 8) of chunk i / 8)
    // are built in LDS (the group list is free now) and stored once each, nonzero ones only;
    // a table too long for that sets them with global atomics
    const int nwords = (nb + 31) / 32;
    const bool lds_bits = nwords <= 2 * kSelThreads;  // uniform
    uint32_t *fb = reinterpret_cast<uint32_t *>(sm.flag);
    if (lds_bits) {
        for (int i = tid; i < nwords; i += kSelThreads) fb[i] = 0u;
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 2; q++) {
        if (fl & (1u << q)) {
            const int j = pj[q];
            lst[o++] = j;
            if (lds_bits) atomicOr(&fb[j >> 5], 1u << (j & 31));
            else atomicOr(&a.pf_need[(int64_t)(j >> 5) * a.B + b], 1u << (j & 31));
        }
    }
    if (lds_bits) {
        __syncthreads();
        for (int i = tid; i < nwords; i += kSelThreads)
            if (fb[i]) a.pf_need[(int64_t)i * a.B + b] = fb[i];
    }
    int32_t *pool_out = a.pool_blocks + (int64_t)b * a.K_blk;
    for (int i = tid; i < a.K_blk; i += kSelThreads) pool_out[i] = i < np ? sm.pool[i] : -1;
    if (tid == 0) {
        a.pool_len[b] = np;
        a.pf_meta[b] = make_uint4(theta, kmax, cnt, 0u);
    }
}

// Phase 1, one workgroup per query: the top-k among the positions of the flagged blocks that
// score >= theta (the position scores of exactly those blocks were recomputed).
__global__ __launch_bounds__(kSelThreads, 8) void k_select_pf_topk(SelectArgs a) {
    extern __shared__ __align__(16) uint8_t sh_raw[];
    SelectShared &sm = *reinterpret_cast<SelectShared *>(sh_raw);
    const int b = blockIdx.x, tid = threadIdx.x;
    const uint4 m = a.pf_meta[b];
    const int L = clamp_len(a.q_pos0 + b + 1, a.maxb);
    for (int i = tid; i < kHistBins; i += kSelThreads) sm.sel.hist[i] = 0u;
    __syncthreads();
    select_topk<false>(a, b, L, a.pf_list + (int64_t)b * a.K_blk, (int)m.z, m.x, m.y, sm);
}

// ------------------------------------------------------------------ two-phase Full selection
//
// One gather workgroup per 1024 groups of a sequence, the last of them to arrive finishing
// the selection.  Each gather workgroup reads every group maximum of its sequence and, in the
// same round trip, the block maxima of its own groups (read whether or not they will be
// needed), so that no single workgroup gathers the pool's scattered blocks (on one CU those
// reads had cost ~9 us).  Bounds from the group maxima in one histogram pass:
//   lam = the lower edge of the bin that holds the K_blk-th largest group maximum.  K_blk
//         distinct blocks (the groups' maximal blocks) reach the K_blk-th largest group
//         maximum, so every pool block scores >= lam and lies in a group whose maximum is
//         >= lam: the pool is the exact top-K_blk of these candidates.
//   mu  = the same edge for the k-th largest group maximum.  k distinct positions score
//         >= mu, so the k best positions all score >= mu and lie in blocks whose maximum is
//         >= mu.  With K_blk >= k those k positions are the k best of the pool (a block that
//         outranks a block holding one of them holds a position that outranks it), i.e. the
//         top-k of the definition.
// A gather workgroup writes its candidate blocks (order key, block) and the position scores of
// its blocks >= mu to its region; the last one reads the regions and selects both exactly.
// The last workgroup keeps the candidates in LDS (at most kSel2LdsCap) and one bound-reaching
// block per thread.  Sequences that fit the pool, and candidate sets beyond those limits
// (heavy ties), take the one-workgroup selection in the last workgroup instead.

// Prefix sums of the regions' candidate counts (pre) and bound-reaching block counts (mpre)
// of sequence b, and whether the two-phase selection holds: every region kept its
// bound-reaching blocks, the candidates fit LDS and the bound-reaching blocks one per thread.
// The two finishing workgroups take the same decision from the same counts.
__device__ __forceinline__ bool full2_counts(const Sel2Ws &q, int b, int32_t *pre, int32_t *mpre, int32_t *flag) {
    const int nw = q.nw, tid = threadIdx.x;
    if (tid < nw) {
        pre[tid + 1] = q.cnt[((int64_t)b * nw + tid) * 2];
        mpre[tid + 1] = q.cnt[((int64_t)b * nw + tid) * 2 + 1];
    }
    __syncthreads();
    if (tid == 0) {
        int okf = 1;
        pre[0] = mpre[0] = 0;
        for (int i = 1; i <= nw; i++) {
            okf &= mpre[i] >= 0;
            pre[i] += pre[i - 1];
            mpre[i] = mpre[i - 1] + max(mpre[i], 0);
        }
        flag[1] = okf && pre[nw] <= kSel2LdsCap && mpre[nw] <= kSelThreads;
    }
    __syncthreads();
    return flag[1] != 0;
}

// Iterations (of a short sleep) after which the top-k workgroup stops waiting for the gather
// workgroups of its sequence.  They were dispatched before it (lower workgroup index) and so
// are resident or done; the bound only guards against a broken launch.
constexpr uint32_t kSel2WaitLimit = 1u << 20;

// The top-k workgroup of the two-phase selection (index nw of its sequence), run beside the
// gather workgroups: mu from the group maxima (the same histogram pass, so the same value
// the gather workgroups use), then, once every gather workgroup has arrived, the exact top-k
// of the positions >= mu of the bound-reaching blocks, while the last gather workgroup selects
// the pool.  Off the fast path (or when the regions overflowed) the last gather workgroup
// selects both.  Resets the sequence's arrival counter for the next call.
__device__ __forceinline__ void full2_topk(const SelectArgs &a, int b, int L, bool fast,
                                        const float4 (&graw)[kIPT / 4], int ng, SelectShared &sm,
                                        int32_t *sh_mpre, int32_t *sh_flag) {
    const Sel2Ws &q = a.sel2;
    const int nw = q.nw, tid = threadIdx.x;
    __shared__ int32_t sh_pre2[kSel2MaxW + 1];
    uint32_t mu = 0u, ghi = 0u;
    if (fast) {
        RegItems<kIPT> g;
#pragma unroll
        for (int i = 0; i < kIPT; i += 4) {
            const float f[4] = {graw[i / 4].x, graw[i / 4].y, graw[i / 4].z, graw[i / 4].w};
#pragma unroll
            for (int t = 0; t < 4; t++) g.key[i + t] = tid * kIPT + i + t < ng ? order_key(f[t]) : 0u;
        }
        uint32_t lam;
        two_bounds(g, (uint32_t)min(a.K_blk, ng), (uint32_t)a.k, sm.sel, &lam, &mu, &ghi);
    }
    // wait for the gather workgroups: relaxed coherent polls (an acquire per poll would
    // invalidate this XCD's caches under the gather workgroups' reads), then one agent-scope
    // acquire, after which their regions are visible
    if (tid == 0) {
        uint32_t it = 0;
        while (__hip_atomic_load(q.arrive + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nw &&
               ++it < kSel2WaitLimit)
            __builtin_amdgcn_s_sleep(2);
        __hip_atomic_store(q.arrive + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    if (!fast || !full2_counts(q, b, sh_pre2, sh_mpre, sh_flag)) return;  // uniform
    const int n_m = sh_mpre[nw];
    // the bound-reaching block tid (blocks in order, one per thread) and its position scores
    const int e = tid;
    int mw = 0;
    if (e < n_m) {  // largest region r with mpre[r] <= e
        int lo = 0, hi = nw - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh_mpre[mid] <= e) lo = mid;
            else hi = mid - 1;
        }
        mw = lo;
    }
    const int64_t mslot = ((int64_t)b * nw + mw) * kSel2MuCap + (e < n_m ? e - sh_mpre[mw] : 0);
    const int32_t mb = e < n_m ? q.mu_blk[mslot] : -1;
    const float4 *msrc = reinterpret_cast<const float4 *>(q.mu_sc + mslot * kBlk);
    const float4 ms0 = msrc[0], ms1 = msrc[1];
    RegItems<kBlk> p;
    {
        const float sc[kBlk] = {ms0.x, ms0.y, ms0.z, ms0.w, ms1.x, ms1.y, ms1.z, ms1.w};
#pragma unroll
        for (int t = 0; t < kBlk; t++) {
            const uint32_t key = order_key(sc[t]);
            p.key[t] = mb >= 0 && mb * kBlk + t < L && key >= mu ? key : 0u;
        }
    }
    // top-k: the exact top-k of the positions >= mu of the blocks >= mu, ascending (every
    // such key lies in [mu, largest group maximum])
    select_emit(p, [&](int t) { return mb * kBlk + t; }, (uint32_t)a.k,
                a.topk + (int64_t)b * a.k, (uint32_t)a.k, sm, ghi != 0u, mu, ghi);
    if (tid == 0) a.topk_len[b] = a.k;
}

// XMAP (several sequences, nw a multiple of 8): a one-dimensional grid in which gather
// workgroup w of every sequence lands on XCD w % 8 (dispatch places workgroup i on XCD
// i % 8), so that the sequences' workgroups of one group range, which read the same lines of
// the interleaved block and position scores, share that XCD's L2.  Workgroup 8 k + x takes
// w = 8 (k / B) + x of sequence k % B (w > nw: none, it returns); every top-k workgroup
// (w = nw) still has a higher index than all gather workgroups.
template <bool XMAP>
__global__ __launch_bounds__(kSelThreads) void k_select_full2(SelectArgs a) {
    extern __shared__ __align__(16) uint8_t sh_raw[];
    SelectShared &sm = *reinterpret_cast<SelectShared *>(sh_raw);
    __shared__ int32_t sh_pre[kSel2MaxW + 1], sh_mpre[kSel2MaxW + 1];
    __shared__ int32_t sh_flag[2];
    const Sel2Ws &q = a.sel2;
    int w = blockIdx.x, b = blockIdx.y;
    if constexpr (XMAP) {
        const int id = (int)blockIdx.x, k = id >> 3;
        b = k % a.B;
        w = 8 * (k / a.B) + (id & 7);
        if (w > q.nw) return;  // (uniform, before any barrier)
    }
    const int nw = q.nw, tid = threadIdx.x;
    // requests: the thread's 16 group maxima (clamped into the row, masked once the length
    // is known), the length, and the 8 block maxima of this workgroup's group gi
    float4 graw[kIPT / 4];
    const float *gm = a.gmax + (int64_t)b * a.ngmax;
#pragma unroll
    for (int i = 0; i < kIPT / 4; i++) {
        const int gix = min(tid * kIPT + 4 * i, a.ngmax - 4);
        graw[i] = *reinterpret_cast<const float4 *>(gm + gix);
    }
    const int gi = w * kSel2GroupsPerW + tid;
    const float4 *bsrc = reinterpret_cast<const float4 *>(a.bscore + (int64_t)b * a.bs_b +
                                                         (int64_t)min(gi, a.ngmax - 1) * a.bs_g);
    float4 bm0 = bsrc[0], bm1 = bsrc[1];
    const int L = clamp_len(a.ctx_len ? a.ctx_len[b] : a.q_pos0 + b + 1, a.maxb);
#pragma unroll
    for (int i = 0; i < kIPT / 4; i++)
        asm volatile("" : "+v"(graw[i].x), "+v"(graw[i].y), "+v"(graw[i].z), "+v"(graw[i].w));
    asm volatile("" : "+v"(bm0.x), "+v"(bm0.y), "+v"(bm0.z), "+v"(bm0.w));
    asm volatile("" : "+v"(bm1.x), "+v"(bm1.y), "+v"(bm1.z), "+v"(bm1.w));
    const int nb = (L + kBlk - 1) / kBlk, ng = (nb + kItemBlocks - 1) / kItemBlocks;
    for (int i = tid; i < kHistBins; i += kSelThreads) sm.sel.hist[i] = 0u;  // kept zero between passes
    __syncthreads();
    const bool fast = nb > a.K_blk && a.K_blk >= a.k && ng > a.k;  // uniform per sequence
    uint32_t lam = 0u, mu = 0u, ghi = 0u;
    int cnt_c = 0, cnt_m = 0;
    const int64_t reg = (int64_t)b * nw + w;
    if (w == nw) {  // the top-k workgroup (uniform)
        full2_topk(a, b, L, fast, graw, ng, sm, sh_mpre, sh_flag);
        return;
    }
    if (fast) {
        RegItems<kIPT> g;
#pragma unroll
        for (int i = 0; i < kIPT; i += 4) {
            const float f[4] = {graw[i / 4].x, graw[i / 4].y, graw[i / 4].z, graw[i / 4].w};
#pragma unroll
            for (int t = 0; t < 4; t++) g.key[i + t] = tid * kIPT + i + t < ng ? order_key(f[t]) : 0u;
        }
        two_bounds(g, (uint32_t)min(a.K_blk, ng), (uint32_t)a.k, sm.sel, &lam, &mu, &ghi);
        if (ng <= a.K_blk) lam = 1u;  // every group holds pool candidates (real keys are >= 1)
        // this workgroup's candidates: the blocks >= lam of group gi (whose maximum is then
        // >= lam), and among them the blocks >= mu
        const float bv[kItemBlocks] = {bm0.x, bm0.y, bm0.z, bm0.w, bm1.x, bm1.y, bm1.z, bm1.w};
        uint32_t ck[kItemBlocks];
        uint32_t nc = 0u, nm = 0u;
#pragma unroll
        for (int i = 0; i < kItemBlocks; i++) {
            const int j = gi * kItemBlocks + i;
            const uint32_t key = order_key(bv[i]);
            ck[i] = gi < ng && j < nb && key >= lam ? key : 0u;
            nc += ck[i] != 0u;
            nm += ck[i] != 0u && ck[i] >= mu;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan<kSelThreads>(nc | (nm << 16), sm.sel.scan, &tot);
        const uint32_t tot_c = tot & 0xFFFFu, tot_m = tot >> 16;
        uint32_t oc = ex & 0xFFFFu, om = ex >> 16;
        uint2 *cand = q.cand + reg * (kSel2GroupsPerW * kItemBlocks);
        const bool mu_fits = tot_m <= (uint32_t)kSel2MuCap;
        // candidates to the region; the bound-reaching blocks to LDS, in block order
#pragma unroll
        for (int i = 0; i < kItemBlocks; i++) {
            const int j = gi * kItemBlocks + i;
            if (ck[i] != 0u) cand[oc++] = make_uint2(ck[i], (uint32_t)j);
            if (mu_fits && ck[i] != 0u && ck[i] >= mu) sm.pool[om++] = j;
        }
        __syncthreads();
        // their position scores, one block per thread
        if (mu_fits && tid < (int)tot_m) {
            const int j = sm.pool[tid];
            const float4 *src = reinterpret_cast<const float4 *>(a.pscore + (int64_t)b * a.ps_b + (int64_t)j * a.ps_j);
            const float4 x0 = src[0], x1 = src[1];
            float4 *dst = reinterpret_cast<float4 *>(q.mu_sc + (reg * kSel2MuCap + tid) * kBlk);
            dst[0] = x0;
            dst[1] = x1;
            q.mu_blk[reg * kSel2MuCap + tid] = j;
        }
        cnt_c = (int)tot_c;
        cnt_m = mu_fits ? (int)tot_m : -1;
    }
    if (tid == 0) {
        q.cnt[reg * 2] = cnt_c;
        q.cnt[reg * 2 + 1] = cnt_m;
    }
    // the last workgroup of the sequence to arrive finishes (every wave's stores are ordered
    // before the barrier; thread 0's agent-scope release publishes them, the last one's acquire
    // covers the other workgroups' regions)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0)
        sh_flag[0] = __hip_atomic_fetch_add(q.arrive + b, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                     nw - 1;
    __syncthreads();
    if (!sh_flag[0]) return;  // uniform
    const bool ok = fast && full2_counts(a.sel2, b, sh_pre, sh_mpre, sh_flag);
    if (!ok) {  // the one-workgroup selection (its group maxima read again: a rare path)
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kIPT / 4; i++) {
            const int gix = min(tid * kIPT + 4 * i, a.ngmax - 4);
            graw[i] = *reinterpret_cast<const float4 *>(gm + gix);
        }
        full_select_one_wg(a, b, L, nb, sm, graw);
        return;
    }
    const int n_c = sh_pre[nw], n_m = sh_mpre[nw];
    uint2 *lds_c = reinterpret_cast<uint2 *>(sh_raw + sizeof(SelectShared));  // [kSel2LdsCap]
    auto region_of = [&](const int32_t *pre, int i) {  // largest r with pre[r] <= i
        int lo = 0, hi = nw - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    // candidates i = tid + 1024 r (strided, so that every wave shares the histogram atomics)
    // into registers for the threshold and into LDS in index order for the emission
    RegItems<kSel2LdsCap / kSelThreads> c;
#pragma unroll
    for (int r = 0; r < kSel2LdsCap / kSelThreads; r++) {
        const int i = tid + kSelThreads * r;
        const bool in = i < n_c;
        const int rw = in ? region_of(sh_pre, i) : 0;
        const uint2 v = q.cand[((int64_t)b * nw + rw) * (kSel2GroupsPerW * kItemBlocks) + (in ? i - sh_pre[rw] : 0)];
        c.key[r] = in ? v.x : 0u;
        if (in) lds_c[i] = v;
    }
    (void)n_m;
    __syncthreads();
    // pool: the exact top-K_blk of the candidates, emitted ascending from LDS (thread t owns
    // candidates [8t, 8t + 8))
    {
        // every candidate key lies in [lam, largest group maximum]
        const SelResult r = range_select(c, (uint32_t)a.K_blk, sm.sel, ghi != 0u, lam, ghi);
        constexpr int PT = kSel2LdsCap / kSelThreads;
        RegItems<PT> o;
        int32_t oid[PT];
#pragma unroll
        for (int j = 0; j < PT; j++) {
            const int i = tid * PT + j;
            const uint2 v = i < n_c ? lds_c[i] : make_uint2(0u, 0u);
            o.key[j] = v.x;
            oid[j] = (int32_t)v.y;
        }
        uint32_t tie_base = 0, out_base = 0;
        emit_selected(o, [&](int j) { return oid[j]; }, r, a.pool_blocks + (int64_t)b * a.K_blk,
                      (uint32_t)a.K_blk, tie_base, out_base, sm.sel);
    }
    if (tid == 0) a.pool_len[b] = a.K_blk;
}

constexpr size_t kSelectShared = sizeof(SelectShared);

int launch_select_full2(const SelectArgs &a, hipStream_t stream) {
    if (a.B <= 0) return CSA2_OK;
    // nw gather workgroups per sequence, then its top-k workgroup (the highest index, so that
    // its gather workgroups are dispatched before it)
    const size_t shm = kSelectShared + sizeof(uint2) * kSel2LdsCap;
    if (a.B > 1 && a.sel2.nw % 8 == 0)
        k_select_full2<true><<<8 * a.B * ((a.sel2.nw + 1 + 7) / 8), kSelThreads, shm, stream>>>(a);
    else
        k_select_full2<false><<<dim3(a.sel2.nw + 1, a.B), kSelThreads, shm, stream>>>(a);
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_select_prefill(const SelectArgs &a, int phase, hipStream_t stream) {
    if (a.B <= 0) return CSA2_OK;
    if (phase == 0) k_select_pf_pool<<<a.B, kSelThreads, kSelectShared, stream>>>(a);
    else k_select_pf_topk<<<a.B, kSelThreads, kSelectShared, stream>>>(a);
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_select(const SelectArgs &a, bool reindex, hipStream_t stream) {
    if (a.B <= 0) return CSA2_OK;
    if (reindex) k_select<true><<<a.B, kSelThreads, kSelectShared, stream>>>(a);
    else k_select<false><<<a.B, kSelThreads, kSelectShared, stream>>>(a);
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

}  // namespace csa2
