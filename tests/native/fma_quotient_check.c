/*
 * The decode and activation-cast kernels form x / s as
 *   q0 = fl32(x * r), r = fl32(1 / s);  q1 = fma(fma(-q0, s, x), r, q0)
 * (one Markstein correction step, used for dynamic per-tensor scales) and,
 * for other scales, a second step q2 = fma(fma(-q1, s, x), r, q1).  This
 * program checks, with the host's correctly rounded fmaf and IEEE division,
 * that the corrected quotient equals fl32(x / s) for every finite bf16 x and
 *   - every dynamic scale s = max(fl32(amax / 448), 1e-12f) of a finite bf16
 *     amax (one step), and
 *   - pseudo-random fp32 scales in [2^-40, 2^40] and the powers of two there
 *     (one and two steps),
 * wherever |x / s| < 512 (beyond, both saturate to +-448 in E4M3: the
 * kernels then use q0, which is checked to be at least 512 * (1 - 2^-22)).
 * Values below 2^-11 all round to a signed zero in E4M3 and are only
 * required to agree in that.  Exit status 0 iff no difference.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static long long checked, bad;

static void check_scale(float s, int steps)
{
    volatile float one = 1.0f, vs = s;
    const float r = one / vs;
    if (!(s >= 0x1p-125f && s <= 0x1p125f && r >= 0x1p-125f && r <= 0x1p125f))
        return;  /* the kernels divide directly for such scales */
    for (uint32_t h = 0; h < 65536; ++h) {
        const float x = f_of(h << 16);
        if (!isfinite(x))
            continue;
        volatile float vx = x;
        const float ref = vx / vs;
        const float q0 = x * r;
        if (fabsf(q0) >= 512.0f) {
            if (!(fabsf(ref) > 464.0f)) {
                if (bad < 10)
                    printf("saturation: s=%a x=%a ref=%a q0=%a\n", s, x, ref, q0);
                ++bad;
            }
            continue;
        }
        float q = fmaf(fmaf(-q0, s, x), r, q0);
        if (steps > 1)
            q = fmaf(fmaf(-q, s, x), r, q);
        q = copysignf(q, x);
        ++checked;
        if (u_of(q) != u_of(ref) && !(fabsf(ref) < 0x1p-11f && fabsf(q) < 0x1p-11f &&
                                      signbit(ref) == signbit(q))) {
            if (bad < 10)
                printf("difference: steps=%d s=%a x=%a ref=%a q=%a\n", steps, s, x, ref, q);
            ++bad;
        }
    }
}

int main(int argc, char **argv)
{
    const int nrand = argc > 1 ? atoi(argv[1]) : 1000;
    for (uint32_t h = 1; h < 0x7F80u; ++h) {
        volatile float amax = f_of(h << 16), d = 448.0f;
        float s = amax / d;
        if (s < 1e-12f)
            s = 1e-12f;
        check_scale(s, 1);
    }
    uint64_t st = 88172645463325252ull;
    for (int i = 0; i < nrand; ++i) {
        st ^= st << 13;
        st ^= st >> 7;
        st ^= st << 17;
        const int e = (int)(st % 81) - 40;
        const float m = 1.0f + (float)((st >> 20) & 0x7FFFFF) / 8388608.0f;
        for (int steps = 1; steps <= 2; ++steps) {
            check_scale(ldexpf(m, e), steps);
            check_scale(ldexpf(1.0f, e), steps);
        }
    }
    printf("checked %lld quotients, %lld differences\n", checked, bad);
    return bad != 0;
}
