// csa2_block.h -- wave- and block-level reductions and scans shared by the indexer kernels
// (gfx950, wave64).
#pragma once
#include "csa2_common.h"

namespace csa2 {

constexpr int kItemBlocks = 8;  // blocks per scan item = blocks per group maximum

// Wave reductions through DPP: quad swaps, half-row and row mirrors, then row broadcasts of
// lanes 15 and 31; the result is complete in lane 63.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_to63(uint32_t v, Op op) {
    int x = (int)v;
    x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false));   // quad [1,0,3,2]
    x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false));   // quad [2,3,0,1]
    x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false));  // row_half_mirror
    x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false));  // row_mirror
    x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return (uint32_t)x;
}

// Block-wide sum (every thread gets the total).  sh: NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    v = wave_reduce_to63(v, [](uint32_t x, uint32_t y) { return x + y; });
    __syncthreads();
    if (lane == kWave - 1) sh[wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(sh + i);
        t += q.x + q.y + q.z + q.w;
    }
    return t;
}

// Exclusive scan over the threads of the block (thread order), returns total via *tot.
// sh: NT/64 words, 16-byte aligned.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh, uint32_t *tot) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == kWave - 1) sh[wave] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(sh + i);
        const uint32_t x[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4 && i + j < NT / kWave; j++) {
            before += (i + j < wave) ? x[j] : 0u;
            all += x[j];
        }
    }
    *tot = all;
    return before + incl - v;
}

__device__ __forceinline__ int clamp_len(int32_t L, int maxb) {
    const int64_t cap = (int64_t)maxb * kBlk;
    return L < 0 ? 0 : (int)(L > cap ? cap : L);
}

}  // namespace csa2
