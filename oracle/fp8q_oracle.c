/*
 * fp8q oracle -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A deliberately plain, slow CPU implementation of what the FP8
 * weight-quantized linear path computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library; the
 * product (the HIP library and its Python binding) never calls it and shares
 * no code with it.
 *
 * Build flags matter for bit-exactness: -O2 -fno-fast-math -ffp-contract=off,
 * so that every fp32 division is an IEEE-754 correctly rounded division and
 * no multiply-add is fused.  OpenMP is used only across independent outputs
 * (rows, or output elements whose own k-order is fixed), so the number of
 * threads never changes a result.
 *
 * Sources (web pages on FP8 quantization of Llama 3):
 *   [P2] "FP8量化与长上下文实测：Llama 3 70B部署优化指南"
 *        §1.1 -- E4M3: 4 exponent bits, 3 mantissa bits, largest value about
 *                448, smallest non-zero about 2^-9.
 *        §1.2 -- weights scaled per channel, activations per tensor.
 *        §3.1 -- conversion: per-channel absmax / 448, scale clamped below at
 *                1e-12, weight divided by the scale and cast to
 *                float8_e4m3fn; scale kept beside the weight.
 *   [P1] "Llama 3 精读" FP8 + 128K deployment write-up
 *        §2.1 -- E4M3 range is symmetric, [-448, 448].
 *        §3.1 step 2 -- the activation scale is an exponential moving
 *                average with decay 0.9999.
 *        §3.1 step 3 -- the FP8 MatMul modes fp8_w_bf16_a (FP8 weight, BF16
 *                activation), fp8_w_fp16_a and fp8_w_fp8_a (FP8 weight and
 *                activation).
 *        §5.3 tip 2 -- a temperature term (1 + 0.1 T) on the new EMA term.
 *   [P2] §4.3 -- per-group granularity, the step beyond per-channel.
 *   [P2] §3.2 -- the FP8 KV cache: a running maximum per attention layer,
 *                raised by prefill batches, read as it stands by decode.
 *   [P3] "Some Technical Notes About Llama 3" commentary, §3.2 -- the KV
 *                cache layout [layers, kv_heads, seq_len, head_dim].
 *
 * Readings where the pages are silent or contradict each other (each one is
 * listed, with its reason, in the design notes of the repository):
 *   - scale arithmetic is fp32 (the scale is stored as a float),
 *   - the quotient is an IEEE fp32 division, then a separate RNE cast to E4M3
 *     (two roundings, in that order),
 *   - values at or beyond 448 in magnitude saturate to +-448,
 *   - the sign of zero is kept (negatives that round to zero give code 0x80),
 *   - the activation scale uses the same formula as the weight scale, taken
 *     over the whole tensor,
 *   - an EMA-scaled call casts with the state held before the call and then
 *     updates the state (the scale lags by one call); the first call is seeded
 *     with the dynamic scale; the update is fp32, unfused, floored at 1e-12.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define ORACLE_ABI 2

int oracle_abi_version(void) { return ORACLE_ABI; }

/* ------------------------------------------------------------------------ */
/* E4M3 (OCP "e4m3fn") decode, from the bit fields.                          */
/* [P2 §1.1] 4 exponent bits and 3 mantissa bits; max about 448, smallest    */
/* non-zero about 2^-9.  With 4+3 bits, a maximum of 448 = 1.75 * 2^8 forces  */
/* exponent bias 7 and an all-ones exponent that is still finite (only the    */
/* mantissa 111 pattern of it is NaN); 2^-9 = 2^(1-7) * 2^-3 is then the      */
/* smallest subnormal.  There are no infinities.                              */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u;
    unsigned e = (code >> 3) & 15u;
    unsigned m = code & 7u;
    double mag;
    if (e == 15u && m == 7u)
        return NAN;
    if (e == 0u)
        mag = ldexp((double)m, -9);                 /* m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

void oracle_e4m3_table(double *out256)
{
    for (unsigned c = 0; c < 256u; ++c)
        out256[c] = oracle_e4m3_value(c);
}

/* The 127 non-negative finite magnitudes, codes 0x00..0x7E, in code order. */
static double g_mag[127];
static int g_mag_ready = 0;

static void mag_init(void)
{
    if (g_mag_ready)
        return;
    for (unsigned c = 0; c < 127u; ++c)
        g_mag[c] = oracle_e4m3_value(c);
    g_mag_ready = 1;
}

__attribute__((constructor)) static void oracle_init(void) { mag_init(); }

/* ------------------------------------------------------------------------ */
/* Cast fp32 -> E4M3 code, round to nearest, ties to even, saturating.       */
/* [P2 §3.1] cast to float8_e4m3fn (round to nearest even);                  */
/* [P1 §2.1] representable range is [-448, 448]: anything beyond saturates.  */
/* Method: search the table of representable magnitudes for the nearest one; */
/* on an exact tie pick the code whose mantissa LSB is 0 (an even code).     */
/* The sign is attached afterwards, so -0 and negative values that round to  */
/* zero give 0x80.                                                           */
/* ------------------------------------------------------------------------ */
static unsigned pick_nearest(double a, unsigned lo_code)
{
    /* g_mag[lo_code] <= a < g_mag[lo_code + 1] */
    double dlo = a - g_mag[lo_code];
    double dhi = g_mag[lo_code + 1] - a;
    if (dlo < dhi)
        return lo_code;
    if (dhi < dlo)
        return lo_code + 1;
    return (lo_code & 1u) ? lo_code + 1 : lo_code;   /* tie: even code */
}

unsigned oracle_cast_e4m3(float t)
{
    if (isnan(t))
        return 0x7Fu;                    /* out of domain; canonical NaN */
    unsigned sign = signbit(t) ? 0x80u : 0u;
    double a = fabs((double)t);
    if (a >= 448.0)
        return sign | 0x7Eu;             /* saturate */
    /* binary search for the largest code with g_mag[code] <= a */
    unsigned lo = 0, hi = 126;           /* g_mag[0] = 0 <= a < g_mag[126] = 448 */
    while (hi - lo > 1u) {
        unsigned mid = (lo + hi) / 2u;
        if (g_mag[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    return sign | pick_nearest(a, lo);
}

/* The same cast found by a different route: a linear scan for the arg-min  */
/* distance over all 127 magnitudes.  Used only to cross-check the search.  */
unsigned oracle_cast_e4m3_scan(float t)
{
    if (isnan(t))
        return 0x7Fu;
    unsigned sign = signbit(t) ? 0x80u : 0u;
    double a = fabs((double)t);
    if (a >= 448.0)
        return sign | 0x7Eu;
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c < 127u; ++c) {
        double d = fabs(g_mag[c] - a);
        if (d < bestd || (d == bestd && (c & 1u) == 0u)) {
            best = c;
            bestd = d;
        }
    }
    return sign | best;
}

void oracle_cast_e4m3_array(const float *t, int64_t count, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = (uint8_t)oracle_cast_e4m3(t[i]);
}

/* Cast every fp32 bit pattern in [first, first + count) and store the codes. */
void oracle_cast_e4m3_bits(uint32_t first, int64_t count, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        uint32_t b = first + (uint32_t)i;
        float t;
        memcpy(&t, &b, 4);
        out[i] = (uint8_t)oracle_cast_e4m3(t);
    }
}

/* ------------------------------------------------------------------------ */
/* BF16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.   */
/* ------------------------------------------------------------------------ */
static float bf16_value(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Scale from an absolute maximum.                                           */
/* [P2 §3.1] scale = absmax / 448, then clamped below at 1e-12.              */
/* fp32 IEEE division; the clamp constant is the fp32 value nearest 1e-12.   */
/* ------------------------------------------------------------------------ */
float oracle_scale_from_amax(float amax)
{
    float s = amax / 448.0f;
    const float floor_ = 1e-12f;
    if (s < floor_)
        s = floor_;
    return s;
}

/* One quantized element: fp32 quotient first, then the E4M3 cast. */
static uint8_t quantize_one(float w, float s)
{
    float t = w / s;                     /* IEEE fp32 division */
    return (uint8_t)oracle_cast_e4m3(t);
}

/* ------------------------------------------------------------------------ */
/* Per-output-channel weight quantization.                                   */
/* [P2 §3.1] for each row n of the [out, in] weight: absmax over the row,    */
/* scale = absmax/448 clamped at 1e-12, codes = cast(w / scale).             */
/* [P2 §1.2] weights use per-channel scales.                                 */
/* Returns 1 if any input was NaN or infinite (such input is out of domain), */
/* else 0.                                                                   */
/* ------------------------------------------------------------------------ */
int oracle_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                           uint8_t *q, int64_t ld_q, float *scale)
{
    int nonfinite = 0;
#pragma omp parallel for schedule(static) reduction(| : nonfinite)
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t *row = w + r * ld_w;
        float amax = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            float a = fabsf(bf16_value(row[c]));
            if (!isfinite(a))
                nonfinite = 1;
            if (a > amax)
                amax = a;
        }
        float s = oracle_scale_from_amax(amax);
        scale[r] = s;
        for (int64_t c = 0; c < k; ++c)
            q[r * ld_q + c] = quantize_one(bf16_value(row[c]), s);
    }
    return nonfinite;
}

/* ------------------------------------------------------------------------ */
/* Per-group weight quantization.                                            */
/* [P2 §4.3] names per-group granularity as the step beyond per-channel      */
/* scales.  Reading: each output row is cut along the input dimension into   */
/* groups of `group` consecutive values (the last one may be shorter), and   */
/* each group gets the scale of [P2 §3.1] over its own values.               */
/* scale is [n, ceil(k / group)], row-major.  group == k is per-channel.     */
/* ------------------------------------------------------------------------ */
int oracle_quantize_weight_grouped(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                                   int64_t group, uint8_t *q, int64_t ld_q, float *scale)
{
    const int64_t ngroups = (k + group - 1) / group;
    int nonfinite = 0;
#pragma omp parallel for schedule(static) reduction(| : nonfinite)
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t *row = w + r * ld_w;
        for (int64_t g = 0; g < ngroups; ++g) {
            const int64_t c0 = g * group;
            const int64_t c1 = c0 + group < k ? c0 + group : k;
            float amax = 0.0f;
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(bf16_value(row[c]));
                if (!isfinite(a))
                    nonfinite = 1;
                if (a > amax)
                    amax = a;
            }
            float s = oracle_scale_from_amax(amax);
            scale[r * ngroups + g] = s;
            for (int64_t c = c0; c < c1; ++c)
                q[r * ld_q + c] = quantize_one(bf16_value(row[c]), s);
        }
    }
    return nonfinite;
}

/* ------------------------------------------------------------------------ */
/* Dynamic per-tensor activation quantization.                               */
/* [P2 §1.2] activations use a single per-tensor scale; the scale formula is */
/* the one of [P2 §3.1] taken over all elements of the tensor, recomputed    */
/* on every call.                                                            */
/* ------------------------------------------------------------------------ */
/* Largest |x| over a bf16 tensor; *nonfinite is set if any element is NaN or
 * infinite (a NaN never becomes the maximum). */
static float act_amax(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x, int *nonfinite)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t c = 0; c < k; ++c) {
            float a = fabsf(bf16_value(x[r * ld_x + c]));
            if (!isfinite(a))
                *nonfinite = 1;
            if (a > amax)
                amax = a;
        }
    return amax;
}

int oracle_quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                        uint8_t *q, int64_t ld_q, float *scale_out)
{
    int nonfinite = 0;
    float amax = act_amax(x, m, k, ld_x, &nonfinite);
    float s = oracle_scale_from_amax(amax);
    *scale_out = s;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r)
        for (int64_t c = 0; c < k; ++c)
            q[r * ld_q + c] = quantize_one(bf16_value(x[r * ld_x + c]), s);
    return nonfinite;
}

/* ------------------------------------------------------------------------ */
/* Static per-tensor activation quantization.                                */
/* [P2 §1.2] one scale for the whole tensor; here the scale is given rather  */
/* than recomputed from X (the static form of the activation scale, [P1 §3.1 */
/* step 2]), so values beyond 448 * s occur and saturate to +-448.           */
/* codes = cast(fl32(X / s)), the same element step as the weights.          */
/* ------------------------------------------------------------------------ */
int oracle_quantize_act_static(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                               float s, uint8_t *q, int64_t ld_q)
{
    int nonfinite = 0;
    (void)act_amax(x, m, k, ld_x, &nonfinite);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r)
        for (int64_t c = 0; c < k; ++c)
            q[r * ld_q + c] = quantize_one(bf16_value(x[r * ld_x + c]), s);
    return nonfinite;
}

/* ------------------------------------------------------------------------ */
/* EMA update of the activation scale.                                       */
/* [P1 §3.1 step 2] the per-tensor activation scale is an exponential moving */
/* average with decay d (0.9999 there): s = d * s_old + (1 - d) * s_new,     */
/* where s_new is the dynamic scale of the tensor just seen.                 */
/* [P1 §5.3, tip 2] the temperature variant multiplies the new term by       */
/* (1 + 0.1 * T); T = 0 gives the plain average.                             */
/* Arithmetic is fp32 (the scale is a float), evaluated left to right as     */
/* written, with no fused multiply-add; 1 - d is formed in fp32 (exact for    */
/* d in [0.5, 1]).  The result is a scale, so it keeps the 1e-12 floor of     */
/* [P2 §3.1].                                                                */
/* ------------------------------------------------------------------------ */
float oracle_ema_scale(float s_old, float s_new, float decay, float temperature)
{
    float keep = decay * s_old;
    float weight = 1.0f - decay;
    float fresh = weight * s_new;
    float tenth = 0.1f;
    float heat = 1.0f + tenth * temperature;
    fresh = fresh * heat;
    float s = keep + fresh;
    const float floor_ = 1e-12f;
    if (s < floor_)
        s = floor_;
    return s;
}

/* ------------------------------------------------------------------------ */
/* One call of EMA-scaled activation quantization.                           */
/* seed != 0: dynamic quantization of X (its own absmax scale); the state    */
/*            and *scale_used both become that scale.                        */
/* seed == 0: X is cast with the state as it stood before the call (the      */
/*            scale is delayed by one call), then the state takes one EMA    */
/*            step towards the dynamic scale of X; *scale_used receives the  */
/*            scale the codes were made with.                                */
/* Returns the non-finite flag of X.                                         */
/* ------------------------------------------------------------------------ */
int oracle_quantize_act_ema(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                            uint8_t *q, int64_t ld_q, float *state, float decay,
                            float temperature, int seed, float *scale_used)
{
    if (seed) {
        int nf = oracle_quantize_act(x, m, k, ld_x, q, ld_q, scale_used);
        *state = *scale_used;
        return nf;
    }
    float s_old = *state;
    int nf = oracle_quantize_act_static(x, m, k, ld_x, s_old, q, ld_q);
    int unused = 0;
    float s_new = oracle_scale_from_amax(act_amax(x, m, k, ld_x, &unused));
    *scale_used = s_old;
    *state = oracle_ema_scale(s_old, s_new, decay, temperature);
    return nf;
}

/* ------------------------------------------------------------------------ */
/* FP8 KV-cache write with an online running-max scale.                      */
/* [P2 §3.2] KV values appear only at inference time, so each attention      */
/* layer keeps a running maximum: every prefill batch raises it and the      */
/* scale is computed from it; decode quantizes the new K/V with the latest   */
/* scale as it stands.  [P2 §3.1] gives the scale formula and the cast.      */
/* Readings: K and V keep a running maximum each; the layer cache is         */
/* [heads, slots, head_dim] per tensor ([P3 §3.2]'s first layout, one layer); */
/* a calibrating call raises the maximum before it casts its own batch.      */
/*   k, v       [t_count, ld] bf16; row t holds heads * head_dim values,      */
/*              head h at columns h*head_dim .. (h+1)*head_dim - 1            */
/*   slot[t]    cache row of token t; rows outside [0, slots) are skipped     */
/*   running[2] running max of |K| and |V| (in/out)                           */
/*   scale_out[2]  the scales the codes of this call were made with           */
/* Returns a bit set: 1 = a non-finite input, 2 = a slot out of range.        */
/* ------------------------------------------------------------------------ */
int oracle_kv_cache_write(const uint16_t *k, const uint16_t *v, int64_t t_count, int64_t heads,
                          int64_t head_dim, int64_t ld, const int64_t *slot,
                          uint8_t *k_cache, uint8_t *v_cache, int64_t slots,
                          float *running, float *scale_out, int calibrate)
{
    const uint16_t *src[2] = {k, v};
    uint8_t *dst[2] = {k_cache, v_cache};
    const int64_t width = heads * head_dim;
    int flags = 0;
    for (int which = 0; which < 2; ++which) {
        int nonfinite = 0;
        float amax = act_amax(src[which], t_count, width, ld, &nonfinite);
        if (nonfinite)
            flags |= 1;
        if (calibrate && amax > running[which])
            running[which] = amax;
        const float s = oracle_scale_from_amax(running[which]);
        scale_out[which] = s;
        for (int64_t t = 0; t < t_count; ++t) {
            const int64_t row = slot[t];
            if (row < 0 || row >= slots) {
                flags |= 2;
                continue;
            }
            for (int64_t h = 0; h < heads; ++h)
                for (int64_t d = 0; d < head_dim; ++d) {
                    const uint16_t x = src[which][t * ld + h * head_dim + d];
                    dst[which][(h * slots + row) * head_dim + d] = quantize_one(bf16_value(x), s);
                }
        }
    }
    return flags;
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 (fp16) decode, from the bit fields: 1 sign bit, 5      */
/* exponent bits with bias 15, 10 mantissa bits; exponent 0 is subnormal    */
/* (m * 2^-24), exponent 31 is infinity (m = 0) or NaN.                      */
/* ------------------------------------------------------------------------ */
double oracle_f16_value(unsigned bits)
{
    unsigned s = (bits >> 15) & 1u;
    unsigned e = (bits >> 10) & 31u;
    unsigned m = bits & 1023u;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp(1.0 + (double)m / 1024.0, (int)e - 15);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* The scaled linear layer, in fp64.                                         */
/* [P1 §3.1 step 3] the three FP8 MatMul modes:                              */
/*   mode 0, fp8_w_bf16_a:  Y[m,n] = s_w[n] * sum_k X[m,k] * dec(Wq[n,k]),   */
/*                          X bf16                                            */
/*   mode 1, fp8_w_fp8_a:   Y[m,n] = s_x * s_w[n] * sum_k dec(Xq[m,k]) *      */
/*                                   dec(Wq[n,k])                            */
/*   mode 2, fp8_w_fp16_a:  mode 0 with X in fp16                            */
/* The weight follows the [out, in] layout of a linear layer, so Y = X W^T.   */
/* Every term is widened to double and summed in increasing k.  For mode 1    */
/* every product is a multiple of 2^-18 below 2^17, so the double sum is      */
/* exact for any K below 2^18.                                               */
/* `rows` selects which rows of X to evaluate (NULL means all m rows); the    */
/* result has shape [nrows, n] in y.                                         */
/* ------------------------------------------------------------------------ */
void oracle_linear(int mode, const void *x, int64_t m, int64_t k, int64_t ld_x,
                   float x_scale, const uint8_t *wq, int64_t n, int64_t ld_w,
                   const float *w_scale, const int64_t *rows, int64_t nrows,
                   double *y)
{
    double tab[256];
    oracle_e4m3_table(tab);
    if (rows == NULL)
        nrows = m;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t i = 0; i < nrows; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int64_t r = rows ? rows[i] : i;
            const uint8_t *wrow = wq + j * ld_w;
            double acc = 0.0;
            if (mode == 0) {
                const uint16_t *xrow = (const uint16_t *)x + r * ld_x;
                for (int64_t c = 0; c < k; ++c)
                    acc += (double)bf16_value(xrow[c]) * tab[wrow[c]];
                y[i * n + j] = acc * (double)w_scale[j];
            } else if (mode == 2) {
                const uint16_t *xrow = (const uint16_t *)x + r * ld_x;
                for (int64_t c = 0; c < k; ++c)
                    acc += oracle_f16_value(xrow[c]) * tab[wrow[c]];
                y[i * n + j] = acc * (double)w_scale[j];
            } else {
                const uint8_t *xrow = (const uint8_t *)x + r * ld_x;
                for (int64_t c = 0; c < k; ++c)
                    acc += tab[xrow[c]] * tab[wrow[c]];
                y[i * n + j] = acc * ((double)x_scale * (double)w_scale[j]);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* The linear layer with per-group weight scales, in fp64.                   */
/* Each group's products are summed, then scaled by that group's scale:      */
/*   Y[m,n] = s_x * sum_g s_w[n,g] * sum_{k in g} a(X[m,k]) * dec(Wq[n,k])   */
/* with a() the activation value of the mode (as in oracle_linear) and       */
/* s_x = 1 in the 16-bit modes.  Groups and scales as in                     */
/* oracle_quantize_weight_grouped.                                           */
/* ------------------------------------------------------------------------ */
void oracle_linear_grouped(int mode, const void *x, int64_t m, int64_t k, int64_t ld_x,
                           float x_scale, const uint8_t *wq, int64_t n, int64_t ld_w,
                           const float *w_scale, int64_t group, const int64_t *rows,
                           int64_t nrows, double *y)
{
    double tab[256];
    oracle_e4m3_table(tab);
    const int64_t ngroups = (k + group - 1) / group;
    if (rows == NULL)
        nrows = m;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t i = 0; i < nrows; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int64_t r = rows ? rows[i] : i;
            const uint8_t *wrow = wq + j * ld_w;
            double total = 0.0;
            for (int64_t g = 0; g < ngroups; ++g) {
                const int64_t c0 = g * group;
                const int64_t c1 = c0 + group < k ? c0 + group : k;
                double acc = 0.0;
                for (int64_t c = c0; c < c1; ++c) {
                    double a;
                    if (mode == 0)
                        a = (double)bf16_value(((const uint16_t *)x)[r * ld_x + c]);
                    else if (mode == 2)
                        a = oracle_f16_value(((const uint16_t *)x)[r * ld_x + c]);
                    else
                        a = tab[((const uint8_t *)x)[r * ld_x + c]];
                    acc += a * tab[wrow[c]];
                }
                total += acc * (double)w_scale[j * ngroups + g];
            }
            y[i * n + j] = mode == 1 ? total * (double)x_scale : total;
        }
    }
}
