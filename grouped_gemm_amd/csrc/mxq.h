// MXQ: the MX-fp8 quantization rule shared by the quantizer kernel and the
// GEMM1 epilogues that requantize act.
//
// e4m3 codes with one e8m0 scale (value 2^(byte-127)) per 32 contiguous
// elements ("Prime Flash MoE", section 7). Scale rule ("Porting Block-Scaled
// GEMM Kernels from Blackwell to Rubin", section 6.2, read as: the scale
// byte is amax/448 rounded up to a power of two): s = the smallest integer
// with amax <= 448 * 2^s, clamped to [-127, 127]; codes = e4m3(v * 2^-s),
// round to nearest even, saturating at 448. s is read off amax's exponent
// and mantissa bits, so no division is made.
#pragma once

#include "common.h"

namespace moe {

// MXQ scale exponent from the block's amax (finite, >= 0).
__device__ __forceinline__ int mx_scale_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int ef = static_cast<int>(u >> 23);
    if (ef == 0) return -127;  // zero or below 2^-126: the clamp decides
    int s = ef - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// 2^e as a float for e in [-127, 127] (2^-127 is subnormal, still exact).
__device__ __forceinline__ float pow2f(int e) {
    return e >= -126 ? __uint_as_float(static_cast<uint32_t>(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// e4m3fn code of v (already divided by the block scale), nearest even,
// saturating; the sign comes from `sign_src` so a value that underflows
// keeps the sign of the input.
__device__ __forceinline__ uint32_t e4m3_encode(float v, float sign_src) {
    const uint32_t sign = (__float_as_uint(sign_src) >> 24) & 0x80u;
    const float x = fabsf(v);
    uint32_t code;
    if (x >= 448.0f) {
        code = 0x7e;
    } else if (x < 0.015625f) {                   // below 2^-6: multiples of 2^-9
        code = static_cast<uint32_t>(rintf(x * 512.0f));
    } else {
        const uint32_t u = __float_as_uint(x);
        const uint32_t r = (u + 0x7ffffu + ((u >> 20) & 1u)) >> 20;  // exponent|3 mantissa bits, RNE
        code = r - (120u << 3);
        if (code > 0x7eu) code = 0x7e;
    }
    return sign | code;
}

// MXFP4 weights ("GC-MoE on SM120", scale formats: 4-bit E2M1 codes in
// blocks of 32 along K, one UE8M0 power-of-two scale per block). e2m1: 1 sign bit, 2
// exponent bits (bias 1), 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3,
// 4, 6. Scale rule MXQ4, the MX-fp8 rule with 6 in place of 448: s = the
// smallest integer with amax <= 6 * 2^s, clamped to [-127, 127]; codes
// e2m1(v * 2^-s), nearest with ties to the even code, saturating at 6.

// MXQ4 scale exponent from the block's amax (finite, >= 0): amax = 1.m * 2^E
// needs s = E - 2 while 1.m <= 1.5, else E - 1.
__device__ __forceinline__ int mx4_scale_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int ef = static_cast<int>(u >> 23);
    if (ef == 0) return -127;  // zero or below 2^-126: the clamp decides
    int s = ef - 129 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// e2m1 code of v (already divided by the block scale). On [0, 2] the values
// are the multiples of 0.5 (code = 2x), on [2, 4] of 1 (code = x + 2), on
// [4, 6] of 2 (code = x/2 + 4); rintf rounds ties to even, and on each
// piece an even integer is an even code. The sign comes from `sign_src`.
__device__ __forceinline__ uint32_t e2m1_encode(float v, float sign_src) {
    const uint32_t sign = (__float_as_uint(sign_src) >> 28) & 0x8u;
    const float x = fabsf(v);
    uint32_t code;
    if (x < 2.0f) code = static_cast<uint32_t>(rintf(x * 2.0f));
    else if (x < 4.0f) code = static_cast<uint32_t>(rintf(x)) + 2u;
    else if (x < 6.0f) code = static_cast<uint32_t>(rintf(x * 0.5f)) + 4u;
    else code = 7u;
    return sign | code;
}

}  // namespace moe
