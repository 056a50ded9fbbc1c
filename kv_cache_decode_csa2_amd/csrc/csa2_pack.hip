// csa2_pack.hip -- MXFP4 / MXFP8 quantisation, dequantisation and cache appends.
//
// Formats and rounding: csa2_quant.h (OCP MX E2M1 / E4M3FN with per-32 E8M0 scales).
//
// One thread quantises one 32-element group: 128 contiguous input bytes, 16 (FP4) or 32
// (FP8) contiguous output bytes.  These kernels run once per new token and are not on
// the bandwidth-critical path.
#include "csa2_quant.h"

namespace csa2 {

__global__ void k_quant_fp4(const float *x, int64_t n_groups, uint8_t *codes, uint8_t *scales) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < n_groups) quant_fp4(x + g * 32, codes + g * 16, scales + g);
}

__global__ void k_quant_fp8(const float *x, int64_t n_groups, uint8_t *codes, uint8_t *scales) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < n_groups) quant_fp8(x + g * 32, codes + g * 32, scales + g);
}

// Dequantisation through the gfx950 scaled converters: bit-exact (value * 2^(s-127)).
__global__ void k_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_groups,
                              float *out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n_groups) return;
    const float sc = e8m0_to_f32(scales[g]);
    const uint4 c = *reinterpret_cast<const uint4 *>(codes + g * 16);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float2 *o = reinterpret_cast<float2 *>(out + g * 32);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], sc, 0);
        auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], sc, 1);
        auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], sc, 2);
        auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], sc, 3);
        o[4 * i + 0] = make_float2(p0[0], p0[1]);
        o[4 * i + 1] = make_float2(p1[0], p1[1]);
        o[4 * i + 2] = make_float2(p2[0], p2[1]);
        o[4 * i + 3] = make_float2(p3[0], p3[1]);
    }
}

__global__ void k_dequant_fp8(const uint8_t *codes, const uint8_t *scales, int64_t n_groups,
                              float *out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n_groups) return;
    const float sc = e8m0_to_f32(scales[g]);
    const uint4 *c4 = reinterpret_cast<const uint4 *>(codes + g * 32);
    const uint4 a = c4[0], b = c4[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float2 *o = reinterpret_cast<float2 *>(out + g * 32);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], sc, false);
        auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], sc, true);
        o[2 * i] = make_float2(lo[0], lo[1]);
        o[2 * i + 1] = make_float2(hi[0], hi[1]);
    }
}

// Full-layer append: one thread per 32-group of a new row; groups 0 .. D/32-1 are the main
// latent, the rest the indexer key (head-major).
__global__ void k_append_global(const float *latent, const float *idx_k,
                                const int32_t *block_table, int32_t maxb, int64_t n_blocks,
                                const int32_t *pos0, int32_t pos_off, int32_t n_new,
                                uint8_t *kv_cache, uint8_t *idx_cache, int32_t D, int32_t H,
                                int32_t dI, int64_t n_rows) {
    const int gl = D / 32, gi = H * (dI / 32), gpr = gl + gi;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_rows * gpr) return;
    const int64_t row = t / gpr;
    const int grp = (int)(t % gpr);
    const bool is_main = grp < gl;
    if (!(is_main ? latent : idx_k)) return;
    const int G = dI / 32, hg = grp - gl, h = hg / G, g = hg % G;
    // the group's 32 values are requested first: they do not depend on the slot lookup
    float v[32];
    load_group(is_main ? latent + row * D + grp * 32 : idx_k + row * (H * dI) + hg * 32, v);
    const int b = (int)(row / n_new);
    const int64_t p = (int64_t)pos0[b] + pos_off + (row % n_new);
    if (p < 0 || p / kBlk >= maxb) return;
    const int64_t phys = block_table[(int64_t)b * maxb + p / kBlk];
    if (phys < 0 || phys >= n_blocks) return;
    const int s = (int)(p % kBlk);
    uint32_t w[4];
    const uint32_t sc = quant_fp4_regs(v, w);
    uint8_t *codes, *scale;
    if (is_main) {
        const int64_t rb = D / 2 + D / 32;
        uint8_t *dst = kv_cache + phys * (kBlk * rb) + s * rb;
        codes = dst + grp * 16;
        scale = dst + D / 2 + grp;
    } else {
        const int64_t codes_bytes = (int64_t)kBlk * H * dI / 2;
        uint8_t *blk = idx_cache + phys * (codes_bytes + (int64_t)kBlk * H * G);
        codes = blk + ((g * kBlk + s) * H + h) * 16;
        scale = blk + codes_bytes + (s * H + h) * G + g;
    }
    *reinterpret_cast<uint4 *>(codes) = make_uint4(w[0], w[1], w[2], w[3]);
    *scale = (uint8_t)sc;
}

__global__ void k_append_swa(const float *rows, const int32_t *pos0, int32_t n_new,
                             uint8_t *swa, int32_t C, int32_t D, int64_t n_rows) {
    const int gpr = D / 32;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_rows * gpr) return;
    const int64_t row = t / gpr;
    const int grp = (int)(t % gpr);
    const int b = (int)(row / n_new);
    const int64_t p = (int64_t)pos0[b] + (row % n_new);
    if (p < 0) return;
    uint8_t *dst = swa + ((int64_t)b * C + p % C) * (D + D / 32);
    quant_fp8(rows + row * D + grp * 32, dst + grp * 32, dst + D + grp);
}

// Block transfer: row r of `rows` <-> physical block blocks[r] of a block cache, in 16-byte
// chunks (one per thread, grid-stride).  Gather writes zeros for an entry outside
// [0, n_blocks); scatter skips it.
template <bool GATHER>
__global__ void k_blocks_copy(const uint8_t *src, uint8_t *dst, const int32_t *blocks,
                              int64_t n_chunks, int32_t cpb, int64_t n_blocks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_chunks; i += stride) {
        const int64_t r = i / cpb;
        const int c = (int)(i - r * cpb);
        const int64_t blk = blocks[r];
        const bool ok = blk >= 0 && blk < n_blocks;
        const int64_t cache_chunk = blk * cpb + c;
        if (GATHER) {
            const uint4 v = ok ? reinterpret_cast<const uint4 *>(src)[cache_chunk] : make_uint4(0u, 0u, 0u, 0u);
            reinterpret_cast<uint4 *>(dst)[i] = v;
        } else if (ok) {
            reinterpret_cast<uint4 *>(dst)[cache_chunk] = reinterpret_cast<const uint4 *>(src)[i];
        }
    }
}

}  // namespace csa2

using namespace csa2;

namespace {
int grid_for(int64_t n, int bs) { return (int)((n + bs - 1) / bs); }
int launched() { return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }
bool cfg_dims_ok(const csa2_config *c) {
    return c && c->kv_dim > 0 && c->kv_dim % 32 == 0 && c->n_idx_heads > 0 &&
           c->idx_dim > 0 && c->idx_dim % 32 == 0 && (c->shared_key == 0 || c->shared_key == 1);
}
}  // namespace

extern "C" int csa2_quantize_mxfp4(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                                   uint8_t *scales, hipStream_t stream) {
    if (!x || !codes || !scales || n_rows < 0 || dim <= 0 || dim % 32) return CSA2_ERR_INVALID;
    const int64_t ng = n_rows * (dim / 32);
    if (ng == 0) return CSA2_OK;
    k_quant_fp4<<<grid_for(ng, 256), 256, 0, stream>>>(x, ng, codes, scales);
    return launched();
}

extern "C" int csa2_quantize_mxfp8(const float *x, int64_t n_rows, int32_t dim, uint8_t *codes,
                                   uint8_t *scales, hipStream_t stream) {
    if (!x || !codes || !scales || n_rows < 0 || dim <= 0 || dim % 32) return CSA2_ERR_INVALID;
    const int64_t ng = n_rows * (dim / 32);
    if (ng == 0) return CSA2_OK;
    k_quant_fp8<<<grid_for(ng, 256), 256, 0, stream>>>(x, ng, codes, scales);
    return launched();
}

extern "C" int csa2_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                                  int32_t dim, float *out, hipStream_t stream) {
    if (!codes || !scales || !out || n_rows < 0 || dim <= 0 || dim % 32) return CSA2_ERR_INVALID;
    const int64_t ng = n_rows * (dim / 32);
    if (ng == 0) return CSA2_OK;
    k_dequant_fp4<<<grid_for(ng, 256), 256, 0, stream>>>(codes, scales, ng, out);
    return launched();
}

extern "C" int csa2_dequant_mxfp8(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                                  int32_t dim, float *out, hipStream_t stream) {
    if (!codes || !scales || !out || n_rows < 0 || dim <= 0 || dim % 32) return CSA2_ERR_INVALID;
    const int64_t ng = n_rows * (dim / 32);
    if (ng == 0) return CSA2_OK;
    k_dequant_fp8<<<grid_for(ng, 256), 256, 0, stream>>>(codes, scales, ng, out);
    return launched();
}

int csa2::launch_append_global(const csa2_config *cfg, const float *latent,
                               const float *idx_k, const int32_t *block_table, int32_t maxb,
                               int64_t n_blocks, const int32_t *pos0, int32_t pos_off,
                               int32_t batch, int32_t n_new, uint8_t *kv_cache,
                               uint8_t *idx_cache, hipStream_t stream) {
    const int64_t rows = (int64_t)batch * n_new;
    if (rows == 0) return CSA2_OK;
    const int kh = key_heads(cfg);
    const int gpr = cfg->kv_dim / 32 + kh * (cfg->idx_dim / 32);
    const int64_t n = rows * gpr;
    k_append_global<<<grid_for(n, 256), 256, 0, stream>>>(
        latent, idx_k, block_table, maxb, n_blocks, pos0, pos_off, n_new, kv_cache, idx_cache,
        cfg->kv_dim, kh, cfg->idx_dim, rows);
    return launched();
}

extern "C" int csa2_append_global(const csa2_config *cfg, const float *latent,
                                  const float *idx_k, const int32_t *block_table, int32_t maxb,
                                  int64_t n_blocks, const int32_t *pos0, int32_t batch,
                                  int32_t n_new, uint8_t *kv_cache, uint8_t *idx_cache,
                                  hipStream_t stream) {
    if (!cfg_dims_ok(cfg) || !block_table || !pos0 || maxb <= 0 || n_blocks <= 0 ||
        batch < 0 || n_new < 0)
        return CSA2_ERR_INVALID;
    if ((latent && !kv_cache) || (idx_k && !idx_cache) || (!latent && !idx_k))
        return CSA2_ERR_INVALID;
    return csa2::launch_append_global(cfg, latent, idx_k, block_table, maxb, n_blocks, pos0, 0,
                                      batch, n_new, kv_cache, idx_cache, stream);
}

extern "C" int csa2_append_swa(const csa2_config *cfg, const float *rows, const int32_t *pos0,
                               int32_t batch, int32_t n_new, uint8_t *swa_cache, int32_t C,
                               hipStream_t stream) {
    if (!cfg_dims_ok(cfg) || !rows || !pos0 || !swa_cache || C <= 0 || batch < 0 || n_new < 0)
        return CSA2_ERR_INVALID;
    const int64_t nrows = (int64_t)batch * n_new;
    if (nrows == 0) return CSA2_OK;
    const int64_t n = nrows * (cfg->kv_dim / 32);
    k_append_swa<<<grid_for(n, 256), 256, 0, stream>>>(rows, pos0, n_new, swa_cache, C,
                                                        cfg->kv_dim, nrows);
    return launched();
}

namespace {
int blocks_copy_args_ok(const void *a, const void *b, const int32_t *blocks, int32_t n,
                        int64_t n_blocks, int64_t block_bytes) {
    return n >= 0 && n_blocks > 0 && block_bytes > 0 && block_bytes % 16 == 0 &&
           (n == 0 || (a && b && blocks));
}
int blocks_grid(int64_t n_chunks) {
    const int64_t g = (n_chunks + 255) / 256;
    return (int)(g < 8192 ? (g > 0 ? g : 1) : 8192);
}
}  // namespace

extern "C" int csa2_blocks_gather(const uint8_t *cache, int64_t n_blocks, int64_t block_bytes,
                                  const int32_t *blocks, int32_t n, uint8_t *rows,
                                  hipStream_t stream) {
    if (!blocks_copy_args_ok(cache, rows, blocks, n, n_blocks, block_bytes)) return CSA2_ERR_INVALID;
    if (n == 0) return CSA2_OK;
    const int32_t cpb = (int32_t)(block_bytes / 16);
    const int64_t chunks = (int64_t)n * cpb;
    k_blocks_copy<true><<<blocks_grid(chunks), 256, 0, stream>>>(cache, rows, blocks, chunks, cpb, n_blocks);
    return launched();
}

extern "C" int csa2_blocks_scatter(const uint8_t *rows, const int32_t *blocks, int32_t n,
                                   uint8_t *cache, int64_t n_blocks, int64_t block_bytes,
                                   hipStream_t stream) {
    if (!blocks_copy_args_ok(rows, cache, blocks, n, n_blocks, block_bytes)) return CSA2_ERR_INVALID;
    if (n == 0) return CSA2_OK;
    const int32_t cpb = (int32_t)(block_bytes / 16);
    const int64_t chunks = (int64_t)n * cpb;
    k_blocks_copy<false><<<blocks_grid(chunks), 256, 0, stream>>>(rows, cache, blocks, chunks, cpb, n_blocks);
    return launched();
}
