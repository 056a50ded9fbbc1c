// csa2_pack.hip -- MXFP4 / MXFP8 quantisation, dequantisation and cache appends.
//
// Formats (the pages say only "FP4" for indexer Q/K and main KV and "FP8" for the window
// KV -- dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心"): OCP MX E2M1 and
// E4M3FN elements with one E8M0 scale per 32 elements.  Scale exponent
// e = floor(log2(amax)) - emax (emax 2 for E2M1, 8 for E4M3FN), clamped to >= -127.
// Elements round to nearest, ties to the even code, and saturate; the sign bit is kept.
//
// One thread quantises one 32-element group: 128 contiguous input bytes, 16 (FP4) or 32
// (FP8) contiguous output bytes.  These kernels run once per new token and are not on
// the bandwidth-critical path.
#include "csa2_common.h"

namespace csa2 {

__device__ __forceinline__ int group_exponent(float amax, int emax) {
    const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    if (ex == 0) return -127;  // zero or subnormal amax: floor(log2) <= -127
    const int e = ex - 127 - emax;
    return e < -127 ? -127 : e;
}

// E2M1 code of x at scale 2^e.  |x| * 2^-e < 8 by construction of e; the thresholds are
// the midpoints of the E2M1 grid, "<" or "<=" chosen so that ties go to the even code.
__device__ __forceinline__ uint32_t fp4_code(float x, int e) {
    const float a = fabsf(ldexpf(x, -e));
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                 (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(x) >> 28) & 8u);
}

// E4M3FN code of x at scale 2^e; |x| * 2^-e < 512.
__device__ __forceinline__ uint32_t fp8_code(float x, int e) {
    const float a = fabsf(ldexpf(x, -e));
    uint32_t code;
    if (a < 0.015625f) {  // below the smallest normal 2^-6: grid step 2^-9
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        const int ex = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6 .. 8
        const uint32_t q = (uint32_t)rintf(ldexpf(a, 3 - ex));           // 8 .. 16
        code = (uint32_t)((ex + 7) << 3) + (q - 8u);
    }
    if (code > 0x7Eu) code = 0x7Eu;  // saturate at 448 (0x7F is NaN)
    return code | ((__float_as_uint(x) >> 24) & 0x80u);
}

__device__ __forceinline__ void load_group(const float *src, float v[32]) {
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float4 t = s4[i];
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
}

__device__ __forceinline__ float group_amax(const float v[32]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) m = fmaxf(m, fabsf(v[i]));
    return m;
}

// Quantise one group to 16 code bytes + 1 scale byte.
__device__ __forceinline__ void quant_fp4(const float *src, uint8_t *codes, uint8_t *scale) {
    float v[32];
    load_group(src, v);
    const int e = group_exponent(group_amax(v), 2);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) acc |= fp4_code(v[8 * i + j], e) << (4 * j);
        w[i] = acc;
    }
    *reinterpret_cast<uint4 *>(codes) = make_uint4(w[0], w[1], w[2], w[3]);
    *scale = (uint8_t)(e + 127);
}

__device__ __forceinline__ void quant_fp8(const float *src, uint8_t *codes, uint8_t *scale) {
    float v[32];
    load_group(src, v);
    const int e = group_exponent(group_amax(v), 8);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) acc |= fp8_code(v[4 * i + j], e) << (8 * j);
        w[i] = acc;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(codes);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    *scale = (uint8_t)(e + 127);
}

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
                                const int32_t *pos0, int32_t n_new, uint8_t *kv_cache,
                                uint8_t *idx_cache, int32_t D, int32_t H, int32_t dI,
                                int64_t n_rows) {
    const int gl = D / 32, gi = H * (dI / 32), gpr = gl + gi;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_rows * gpr) return;
    const int64_t row = t / gpr;
    const int grp = (int)(t % gpr);
    const int b = (int)(row / n_new);
    const int64_t p = (int64_t)pos0[b] + (row % n_new);
    if (p < 0 || p / kBlk >= maxb) return;
    const int64_t phys = block_table[(int64_t)b * maxb + p / kBlk];
    if (phys < 0 || phys >= n_blocks) return;
    const int s = (int)(p % kBlk);
    if (grp < gl) {
        if (!latent) return;
        const int64_t rb = D / 2 + D / 32;
        uint8_t *dst = kv_cache + phys * (kBlk * rb) + s * rb;
        quant_fp4(latent + row * D + grp * 32, dst + grp * 16, dst + D / 2 + grp);
    } else {
        if (!idx_k) return;
        const int G = dI / 32, hg = grp - gl, h = hg / G, g = hg % G;
        const int64_t codes_bytes = (int64_t)kBlk * H * dI / 2;
        uint8_t *blk = idx_cache + phys * (codes_bytes + (int64_t)kBlk * H * G);
        quant_fp4(idx_k + row * (H * dI) + hg * 32, blk + ((g * kBlk + s) * H + h) * 16,
                  blk + codes_bytes + (s * H + h) * G + g);
    }
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

}  // namespace csa2

using namespace csa2;

namespace {
int grid_for(int64_t n, int bs) { return (int)((n + bs - 1) / bs); }
int launched() { return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }
bool cfg_dims_ok(const csa2_config *c) {
    return c && c->kv_dim > 0 && c->kv_dim % 32 == 0 && c->n_idx_heads > 0 &&
           c->idx_dim > 0 && c->idx_dim % 32 == 0;
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
    const int64_t rows = (int64_t)batch * n_new;
    if (rows == 0) return CSA2_OK;
    const int gpr = cfg->kv_dim / 32 + cfg->n_idx_heads * (cfg->idx_dim / 32);
    const int64_t n = rows * gpr;
    k_append_global<<<grid_for(n, 256), 256, 0, stream>>>(
        latent, idx_k, block_table, maxb, n_blocks, pos0, n_new, kv_cache, idx_cache,
        cfg->kv_dim, cfg->n_idx_heads, cfg->idx_dim, rows);
    return launched();
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
