// Symmetric per-row int8 quantisation of one element: code = rint(x / s),
// round half to even, clamped to [-127, 127], with s = amax / 127 of the row
// ("Qwen3.6-35B-A3B-w8a8 config.json and recipe.yaml" walkthrough,
// quantization_config group_0 "input_activations" / "weights").  Shared by
// the quantisation kernels and by the router, which quantises the tokens it
// has already staged.
//
// x / s is the IEEE quotient: with y = 1/s correctly rounded (one IEEE divide
// per row), q0 = x*y, r = x - s*q0 (exact, by fma) and q = q0 + r*y (one fma)
// give the correctly rounded x/s whenever no intermediate is subnormal
// (Markstein's theorem).  That holds when s >= 2^-100: a subnormal x then has
// |x/s| < 2^-26 and code 0 either way.  Rows with a smaller scale use the
// divide itself.
#pragma once
#include "device_common.h"

namespace w8a8 {

// clamp(rint(q), -127, 127) as a byte.  The bounds are integers, so clamping
// first and rounding after gives the same integer (NaN clamps to -127 either
// way); adding 1.5 * 2^23 rounds the clamped value half-to-even into the low
// mantissa bits, whose low byte is then the two's-complement code.
// (the byte is the low byte of the returned word; the other bits are junk)
__device__ __forceinline__ uint32_t clamp_code(float q)
{
    const float c = fminf(fmaxf(q, -127.0f), 127.0f);
    return __float_as_uint(c + 12582912.0f);
}

__device__ __forceinline__ uint32_t quant_code(float v, float s) { return clamp_code(v / s); }

// fl(v / s) from the correctly rounded reciprocal y (see above)
__device__ __forceinline__ uint32_t quant_code_fma(float v, float s, float y)
{
    const float q0 = v * y;
    const float r = fmaf(-s, q0, v);
    return clamp_code(fmaf(r, y, q0));
}

// the low bytes of four words, in order, as one word (three byte permutes)
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3)
{
    const uint32_t p01 = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);   // [c0.b0, c1.b0, 0, 0]
    const uint32_t p23 = __builtin_amdgcn_perm(c3, c2, 0x0c0c0400u);   // [c2.b0, c3.b0, 0, 0]
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);              // [c0, c1, c2, c3]
}

__device__ __forceinline__ uint2 pack8(const float v[8], float s, float y, bool fast)
{
    uint32_t c[8];
    if (fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = quant_code_fma(v[i], s, y);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = quant_code(v[i], s);
    }
    return make_uint2(pack_low_bytes(c[0], c[1], c[2], c[3]), pack_low_bytes(c[4], c[5], c[6], c[7]));
}

constexpr float QUANT_FAST_MIN_SCALE = 0x1p-100f;

}  // namespace w8a8
