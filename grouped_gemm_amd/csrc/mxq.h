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

}  // namespace moe
