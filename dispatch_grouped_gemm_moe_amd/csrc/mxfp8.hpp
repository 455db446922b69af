// MXFP8 element helpers shared by the quantising kernels: OCP Microscaling
// v1.0 E4M3 elements with one E8M0 scale per 32 elements.
#pragma once

#include "common.hpp"

namespace moe {

// smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 for amax = 0
__device__ __forceinline__ int mx_scale_exp(float amax) {
    if (!(amax > 0.0f)) return 0;
    int p;
    const float m = frexpf(amax, &p);  // amax = m * 2^p, m in [0.5, 1)
    int e = p - 9 + (m > 0.875f ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// four values -> four E4M3 codes (round to nearest even, saturating at 448)
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// 16 consecutive values of one thread -> 16 codes scaled by 2^-e
__device__ __forceinline__ intx4 fp8x16(const float* v, int e) {
    intx4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = (int)fp8x4(ldexpf(v[4 * q], -e), ldexpf(v[4 * q + 1], -e), ldexpf(v[4 * q + 2], -e),
                          ldexpf(v[4 * q + 3], -e));
    return o;
}

// One 32-element block of a bf16 row (src, 16-byte aligned) -> 32 E4M3 codes
// at dst (16-byte aligned); returns the E8M0 scale byte (e + 127).
__device__ __forceinline__ uint8_t mx_quant_block32(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst) {
    const intx4* s = (const intx4*)src;
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const intx4 raw = s[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[8 * q + 2 * e] = __builtin_bit_cast(float, (uint32_t)raw[e] << 16);
            v[8 * q + 2 * e + 1] = __builtin_bit_cast(float, (uint32_t)raw[e] & 0xffff0000u);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(v[c]));
    const int e = mx_scale_exp(amax);
    intx4* d = (intx4*)dst;
    d[0] = fp8x16(v, e);
    d[1] = fp8x16(v + 16, e);
    return (uint8_t)(e + 127);
}

// Scale byte of block b of a row with nb blocks into the GEMM operand scale
// layout [mx_groups(cols)][rows][4]; the row's last block also zeroes the
// bytes of its group past the row's end.
__device__ __forceinline__ void mx_store_scale_byte(uint8_t* scales, int64_t rows, int64_t row, int b, int nb,
                                                    uint8_t sc) {
    uint8_t* d = scales + ((int64_t)(b >> 2) * rows + row) * 4;
    d[b & 3] = sc;
    if (b + 1 == nb)
        for (int z = (b & 3) + 1; z < 4; ++z) d[z] = 0;
}

// The two scales (pair = block 2j | block 2j+1 << 8) of 64-element block j of
// a row in the GEMM operand scale layout (scales [groups][rows][4]): half j % 2
// of the row's dword of group j / 2.  The last block of a row with an odd
// number of them writes the whole dword, its upper half zero.
__device__ __forceinline__ void mx_store_scale_pair(uint8_t* scales, int64_t rows, int64_t row, int j, int nj,
                                                    uint32_t pair) {
    uint8_t* d = scales + ((int64_t)(j >> 1) * rows + row) * 4;
    if ((j & 1) == 0 && j + 1 == nj)
        *(uint32_t*)d = pair;
    else
        *(uint16_t*)(d + 2 * (j & 1)) = (uint16_t)pair;
}

// A row's 64 values held as 16 per thread by four consecutive lanes (lane % 4 =
// 16-column group): quantise along the row, write the 64 codes at `codes` (this
// lane's 16 at codes + 16 * (lane % 4)) and the two block scales as 64-element
// block j of nj of row `row` in the operand scale layout `scales` [.][rows][4].
__device__ __forceinline__ void mx_quant_row64(const float* v, int lane4, uint8_t* codes, uint8_t* scales,
                                               int64_t rows, int64_t row, int j, int nj) {
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) m = fmaxf(m, fabsf(v[c]));
    m = fmaxf(m, __shfl_xor(m, 1, kWave));  // lanes 0,1: block 0; lanes 2,3: block 1
    const int e = mx_scale_exp(m);
    *(intx4*)(codes + 16 * lane4) = fp8x16(v, e);
    const int e_hi = __shfl_xor(e, 2, kWave);
    if (lane4 == 0) mx_store_scale_pair(scales, rows, row, j, nj, (uint32_t)(e + 127) | ((uint32_t)(e_hi + 127) << 8));
}

}  // namespace moe
