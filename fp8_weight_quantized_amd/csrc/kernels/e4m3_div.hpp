// E4M3 codes of x / s for many x and one scale s, equal bit for bit to the
// codes of the IEEE fp32 quotient that the deployment guide's conversion
// ("FP8量化与长上下文实测：Llama 3 70B部署优化指南", §3.1) rounds:
// E4M3_RNE_SAT(fl32(x / s)).
//
// A correctly rounded fp32 division costs about ten vector instructions and a
// branch per value, which made the per-tensor activation cast, and above all
// the decode GEMM that casts the activations it stages, bound by the ALU.
// Instead, with r = fl32(1 / s) computed once per kernel (an IEEE division),
// every quotient is formed by a product and Markstein's FMA correction
// (Markstein, "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990; the correction step of IA-64
// division):
//   q0 = fl32(x * r),   q1 = fma(fma(-q0, s, x), r, q0),
// and for scales the caller does not guarantee to be dynamic ones, a second
// step q2 = fma(fma(-q1, s, x), r, q1).  Markstein's theorem: if r is within
// half an ulp of 1 / s and q within one ulp of x / s, then fma(-q, s, x) is
// exact and fma(that, r, q) is the correctly rounded x / s.  q1 is within one
// ulp, so the second step is correctly rounded for any normal scale.  One
// step was checked exhaustively against IEEE division on the CPU for every
// finite bf16 x and every dynamic scale max(fl32(amax / 448), 1e-12) of a
// finite bf16 amax (1.2e9 pairs, no difference), plus 8000 other scales in
// [2^-40, 2^40]; the dynamic per-tensor activation cast and the weight
// quantizers (per row and per group, whose scales have the same form) use it.
//
// Quotients of magnitude 512 and more saturate to +-448 either way, so there
// (and for infinities) q0 is used as it is; below 2^-10 every value rounds to
// a signed zero, and the sign of a zero quotient is the sign of x, so the
// result takes x's sign.  Scales whose reciprocal is not a normal number with
// margin (held scales beyond 2^125, or non-finite ones) take the IEEE
// division throughout.
#pragma once

#include "device_common.hpp"

namespace fp8q {
namespace dev {

struct E4M3Div {
    float s;          // the scale
    float r;          // fl32(1 / s)
    bool fast;        // r and s normal with margin: the product path is valid
    bool two_steps;   // the scale is not known to be a dynamic one

    // dynamic: s = max(fl32(amax / 448), 1e-12f) for a bf16 amax, where one
    // correction step is exhaustively verified.
    __device__ __forceinline__ explicit E4M3Div(float scale, bool dynamic = false)
        : s(scale), two_steps(!dynamic)
    {
        r = 1.0f / scale;
        fast = scale >= 0x1p-125f && scale <= 0x1p125f && r >= 0x1p-125f && r <= 0x1p125f;
    }

    // fl32(x / s) where |x / s| < 512; q0 (already saturating) beyond.
    __device__ __forceinline__ float quot(float x) const
    {
        const float q0 = __fmul_rn(x, r);
        float q = __fmaf_rn(__fmaf_rn(-q0, s, x), r, q0);
        if (two_steps)
            q = __fmaf_rn(__fmaf_rn(-q, s, x), r, q);
        return __builtin_fabsf(q0) < 512.0f ? __builtin_copysignf(q, x) : q0;
    }

    // Eight bf16 values (a uint4) divided by s, cast to eight E4M3 codes.
    __device__ __forceinline__ uint2 codes8(uint4 v) const
    {
        if (!fast)
            return quantize8(v, s);
        uint2 c;
        c.x = e4m3x4(quot(bf16_lo(v.x)), quot(bf16_hi(v.x)), quot(bf16_lo(v.y)), quot(bf16_hi(v.y)));
        c.y = e4m3x4(quot(bf16_lo(v.z)), quot(bf16_hi(v.z)), quot(bf16_lo(v.w)), quot(bf16_hi(v.w)));
        return c;
    }
};

}  // namespace dev
}  // namespace fp8q
