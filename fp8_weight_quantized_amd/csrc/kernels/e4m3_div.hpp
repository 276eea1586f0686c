// E4M3 codes of x / s for many x and one scale s, equal bit for bit to the
// codes of the IEEE fp32 quotient that the deployment guide's conversion
// ("FP8量化与长上下文实测：Llama 3 70B部署优化指南", §3.1) rounds:
// E4M3_RNE_SAT(fl32(x / s)).
//
// A correctly rounded fp32 division costs about ten vector instructions, and
// in the per-tensor activation cast that work, not the memory traffic, set
// the time.  With r = fl32(1 / s) computed once, t = fl32(x * r) is within
// 1.5 * 2^-23 * |x / s| of x / s, so within 2^-22 * |t| of fl32(x / s) (both
// normal).  E4M3 rounding (with the saturating clamp) is a monotone step
// function of its input, so if t * (1 - 2^-20) and t * (1 + 2^-20) -- an
// interval that contains fl32(x / s) with a 4x margin -- round to the same
// code, that is the code of fl32(x / s).  Otherwise (t lies near a midpoint
// between two E4M3 values, about 1 element in 10^5) the exact quotient is
// computed.  Zeros keep their sign through the product; every value below
// 2^-10 rounds to a signed zero either way.  Scales whose reciprocal is not a
// normal number with margin (held scales beyond 2^125, or non-finite ones)
// take the exact division throughout.
#pragma once

#include "device_common.hpp"

namespace fp8q {
namespace dev {

struct E4M3Div {
    float s;     // the scale
    float r;     // fl32(1 / s)
    bool fast;   // r and s normal with margin: the product path is valid

    __device__ __forceinline__ explicit E4M3Div(float scale) : s(scale)
    {
        r = 1.0f / scale;
        fast = scale >= 0x1p-125f && scale <= 0x1p125f && r >= 0x1p-125f && r <= 0x1p125f;
    }

    // Eight bf16 values (a uint4) divided by s, cast to eight E4M3 codes.
    __device__ __forceinline__ uint2 codes8(uint4 v) const
    {
        if (!fast)
            return quantize8(v, s);
        constexpr float dn = 1.0f - 0x1p-20f;
        constexpr float up = 1.0f + 0x1p-20f;
        const float t0 = bf16_lo(v.x) * r, t1 = bf16_hi(v.x) * r;
        const float t2 = bf16_lo(v.y) * r, t3 = bf16_hi(v.y) * r;
        const float t4 = bf16_lo(v.z) * r, t5 = bf16_hi(v.z) * r;
        const float t6 = bf16_lo(v.w) * r, t7 = bf16_hi(v.w) * r;
        uint2 a, b;
        a.x = e4m3x4(t0 * dn, t1 * dn, t2 * dn, t3 * dn);
        a.y = e4m3x4(t4 * dn, t5 * dn, t6 * dn, t7 * dn);
        b.x = e4m3x4(t0 * up, t1 * up, t2 * up, t3 * up);
        b.y = e4m3x4(t4 * up, t5 * up, t6 * up, t7 * up);
        if (a.x == b.x && a.y == b.y)
            return a;
        return quantize8(v, s);
    }
};

}  // namespace dev
}  // namespace fp8q
