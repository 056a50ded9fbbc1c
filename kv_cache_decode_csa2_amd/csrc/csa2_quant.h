// csa2_quant.h -- MXFP4 / MXFP8 quantisation of one 32-element group (device code shared
// by the append kernels and the fused window append of the attention kernel).
//
// Formats (the pages say only "FP4" for indexer Q/K and main KV and "FP8" for the window
// KV -- dbyun.net/article/10794, "KV Cache 成为这一代架构改造的核心"): OCP MX E2M1 and
// E4M3FN elements with one E8M0 scale per 32 elements.  Scale exponent
// e = floor(log2(amax)) - emax (emax 2 for E2M1, 8 for E4M3FN), clamped to >= -127.
// Elements round to nearest, ties to the even code, and saturate; the sign bit is kept.
#pragma once
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

// One FP4 group quantised into registers: w[0..3] hold the 32 codes (8 per word, element
// 8i+j in bits 4j..4j+3 of w[i]); returns the E8M0 scale code.
__device__ __forceinline__ uint32_t quant_fp4_regs(const float v[32], uint32_t w[4]) {
    const int e = group_exponent(group_amax(v), 2);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) acc |= fp4_code(v[8 * i + j], e) << (4 * j);
        w[i] = acc;
    }
    return (uint32_t)(e + 127);
}

// Quantise one group to 16 code bytes + 1 scale byte.
__device__ __forceinline__ void quant_fp4(const float *src, uint8_t *codes, uint8_t *scale) {
    float v[32];
    load_group(src, v);
    uint32_t w[4];
    const uint32_t sc = quant_fp4_regs(v, w);
    *reinterpret_cast<uint4 *>(codes) = make_uint4(w[0], w[1], w[2], w[3]);
    *scale = (uint8_t)sc;
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

// One FP8 group quantised into registers: w[0..7] hold the 32 codes (4 per word, element
// 4i+j in byte j of w[i]); returns the E8M0 scale code.
__device__ __forceinline__ uint32_t quant_fp8_regs(const float v[32], uint32_t w[8]) {
    const int e = group_exponent(group_amax(v), 8);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) acc |= fp8_code(v[4 * i + j], e) << (8 * j);
        w[i] = acc;
    }
    return (uint32_t)(e + 127);
}

}  // namespace csa2
