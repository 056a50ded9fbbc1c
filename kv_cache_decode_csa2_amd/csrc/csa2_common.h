// csa2_common.h -- device helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

constexpr int kBlk = CSA2_BLOCK;
constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// fp32 value of an E8M0 scale code (2^(c-127)); code 0 is the subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
    return c ? __uint_as_float(c << 23) : __uint_as_float(0x00400000u);
}

// Order-preserving map of an fp32 score to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_up(v, o, kWave);
        if (l >= o) v += t;
    }
    return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Coherent (L1-bypassing) load of a value other workgroups update with atomics.
__device__ __forceinline__ uint32_t load_coherent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace csa2

namespace csa2 {

// Radix digit of the block-score histogram built during the scan (top 12 bits of the
// order-preserving key).
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;

// Per-sequence state kept in the workspace between the kernels of one Full call.  The
// counters are zero on entry and are zero again when the call has finished (the last
// scan workgroup of a sequence resets `done`, k_pool_final resets n_sel / n_cand).
struct SeqState {
    int32_t thr;     // threshold digit of the pool (-1: every block qualifies)
    int32_t above;   // blocks with a digit above thr
    int32_t n_sel;   // blocks appended to the selected list
    int32_t n_cand;  // blocks appended to the candidate list (digit == thr)
    int32_t done;    // scan chunks finished
    int32_t pad[3];
};

constexpr int kMaxBatch = 4096;  // sequences per call (the scan keeps a work list in LDS)

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the index calls.  Offsets in bytes from the workspace base.  The state and
// histogram regions must be zero before the first call that uses the workspace.
struct WsIndex {
    size_t st, hist, bscore, sel, cand, pscore, total;
};

__host__ __device__ inline WsIndex ws_index(int B, int maxb, int K_blk) {
    WsIndex w;
    size_t o = 0;
    w.st = o;           o = align256(o + sizeof(SeqState) * (size_t)B);
    w.hist = o;         o = align256(o + sizeof(uint32_t) * (size_t)B * kHistBins);
    w.bscore = o;       o = align256(o + sizeof(float) * (size_t)B * maxb);
    w.sel = o;          o = align256(o + sizeof(int32_t) * (size_t)B * K_blk);
    w.cand = o;         o = align256(o + sizeof(uint32_t) * 2 * (size_t)B * maxb);
    w.pscore = o;       o = align256(o + sizeof(float) * (size_t)B * K_blk * kBlk);
    w.total = o;
    return w;
}

// Workspace of the attention call: per split partial numerators and (max, sum) pairs.
constexpr int kAttnRows = 64;  // rows per attention workgroup
struct WsAttn {
    size_t part_o, part_ml, total;
};
__host__ __device__ inline int attn_splits(int k, int W) { return (k + W + kAttnRows - 1) / kAttnRows; }
__host__ __device__ inline WsAttn ws_attn(int B, int Hq, int D, int nsplit) {
    WsAttn w;
    size_t o = 0;
    w.part_o = o;  o = align256(o + sizeof(float) * (size_t)B * nsplit * Hq * D);
    w.part_ml = o; o = align256(o + sizeof(float) * 2 * (size_t)B * nsplit * Hq);
    w.total = o;
    return w;
}

}  // namespace csa2
