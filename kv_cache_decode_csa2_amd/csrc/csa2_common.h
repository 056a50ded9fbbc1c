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

// Indexer keys stored per position: one per head, or one shared by all query heads.
inline int key_heads(const csa2_config *c) { return c->shared_key ? 1 : c->n_idx_heads; }

// Inclusive scan over the 64 lanes of a wave: DPP row shifts within rows of 16 lanes,
// then row broadcasts of lanes 15 and 31 into the rows above.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return (uint32_t)x;
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

// Global append (MXFP4 latent row and indexer key) of n_new tokens per sequence at positions
// pos0[b] + pos_off + t; arguments as csa2_append_global, already validated.
int launch_append_global(const csa2_config *cfg, const float *latent, const float *idx_k,
                         const int32_t *block_table, int32_t maxb, int64_t n_blocks,
                         const int32_t *pos0, int32_t pos_off, int32_t batch, int32_t n_new,
                         uint8_t *kv_cache, uint8_t *idx_cache, hipStream_t stream);

constexpr int kMaxBatch = 4096;  // sequences per index call (the scan keeps a prefix in LDS)

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the attention call: per split partial numerators and (max, sum) pairs, and
// one arrival counter per (sequence, head group), which every call leaves at zero.
constexpr int kAttnRows = 64;  // rows per attention workgroup
struct WsAttn {
    size_t part_o, part_ml, count, total;
};
__host__ __device__ inline int attn_splits(int k, int W) { return (k + W + kAttnRows - 1) / kAttnRows; }

constexpr int kAttnDim = 512;        // latent dim of the attention kernels
constexpr int kAttnMaxSplits = 512;  // 64-row chunks a merge handles (k + W <= 32768)

// Status of cfg's attention shape: CSA2_ERR_INVALID for values out of range,
// CSA2_ERR_UNSUPPORTED for a shape without a kernel (the attention calls and the attention
// workspace query both apply it).
inline int attn_cfg_status(const csa2_config *c) {
    if (!c || c->topk <= 0 || c->swa_window < 0 || c->n_q_heads <= 0 || c->kv_dim <= 0)
        return CSA2_ERR_INVALID;
    if (c->kv_dim != kAttnDim || c->n_q_heads % 16 || c->n_q_heads > 128) return CSA2_ERR_UNSUPPORTED;
    if (attn_splits(c->topk, c->swa_window) > kAttnMaxSplits) return CSA2_ERR_UNSUPPORTED;
    return CSA2_OK;
}

// Row chunks of 64 per workgroup stream.  A batch of at least 512 (sequence, head group)
// pairs fills the chip with one-stream workgroups (splits up to about 1024 workgroups);
// smaller batches take two-stream workgroups, each owning up to cps chunks (cps even).  A
// two-stream workgroup holds nearly all of a CU's LDS, so the splits aim at one wave of them
// on the 256 CUs: more would run as a second wave, which costs more than the extra chunks
// each workgroup takes instead.
struct AttnPlan {
    int nsplit, cps, ns;  // splits, chunks per split, chunk streams per workgroup
};
__host__ __device__ inline AttnPlan attn_plan(int B, int Hq, int k, int W) {
    const int nchunk = attn_splits(k, W);
    const int groups = (B > 0 ? B : 1) * (Hq / 16 > 0 ? Hq / 16 : 1);
    const int ns = groups >= 512 ? 1 : 2;
    const int units = (nchunk + ns - 1) / ns;  // chunks, or chunk pairs
    int sp = ns == 1 ? (1024 + groups - 1) / groups : 256 / groups;
    sp = sp < 1 ? 1 : (sp > units ? units : sp);
    const int ups = (units + sp - 1) / sp;  // units per split
    return AttnPlan{(units + ups - 1) / ups, ns * ups, ns};
}

// The arrival counters sit in a fixed region at the start of every attention workspace, so
// one zero-once workspace can serve calls of any batch, query count or split plan: splits
// (nsplit > 1) only happen for fewer than kAttnCounters (sequence, head group) pairs, and
// pair i always counts at word i.  Partials follow the counters.
constexpr int kAttnCounters = 1024;
__host__ __device__ inline WsAttn ws_attn(int B, int Hq, int D, int nsplit) {
    WsAttn w;
    size_t o = 0;
    w.count = o;   o = align256(o + sizeof(int32_t) * (size_t)kAttnCounters);
    if (nsplit <= 1) {  // one split: the kernel writes the outputs, no partials
        w.part_o = w.part_ml = o;
        w.total = o;
        return w;
    }
    w.part_o = o;  o = align256(o + sizeof(float) * (size_t)B * nsplit * Hq * D);
    w.part_ml = o; o = align256(o + sizeof(float) * 2 * (size_t)B * nsplit * Hq);
    w.total = o;
    return w;
}

}  // namespace csa2
