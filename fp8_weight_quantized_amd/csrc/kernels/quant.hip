// Quantization kernels: per-output-channel weight quantization, per-tensor
// activation quantization -- dynamic (two passes), with a held static scale
// (one pass) or with an EMA scale (one pass plus a one-workgroup update) --
// and the bare fp32 -> E4M3 cast.  The method is the conversion of the
// deployment guide ("FP8量化与长上下文实测：Llama 3 70B部署优化指南", §3.1):
// absmax / 448 with the scale clamped at 1e-12, an fp32 division, and an RNE
// cast to E4M3 that saturates at +-448; weights get one scale per output row,
// activations one scale per tensor (§1.2).  The EMA scale is the one of the
// "Llama 3 精读" write-up (§3.1 step 2, §5.3 tip 2).
//
// All of them are HBM-bound streaming kernels: bf16 in (2 B/element), codes out
// (1 B/element).  Loads are 16 B per lane, stores 8 B per lane, fully
// coalesced; the reductions use wave shuffles and a few words of LDS.
#include "device_common.hpp"
#include "e4m3_div.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Weights: one workgroup per output row.  CH > 0: the row is held in
// registers (at most CH 16-byte chunks per thread) between the absmax and the
// cast, so every weight byte is read from HBM once.  CH == 0: rows longer
// than 16 * 256 * 8 elements are streamed twice (the second pass mostly hits
// in L2 / Infinity Cache).
// ---------------------------------------------------------------------------
template <int CH>
__global__ __launch_bounds__(kThreads) void k_quant_weight(
    const uint16_t *__restrict__ w, int64_t k, int64_t ld_w,
    uint8_t *__restrict__ q, int64_t ld_q, float *__restrict__ scale,
    int32_t *__restrict__ flag)
{
    __shared__ uint32_t red[kThreads / kWave];
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * ld_w;
    uint8_t *qr = q + row * ld_q;
    const int64_t nfull = k >> 3;          // full 8-element (16-byte) chunks
    const int tail = (int)(k & 7);
    const int tid = threadIdx.x;

    uint32_t key = 0;
    uint4 buf[CH > 0 ? CH : 1];
    if constexpr (CH > 0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t idx = tid + (int64_t)c * kThreads;
            if (idx < nfull) {
                buf[c] = ld_nt16(wr + idx * 8);
                uint32_t m01 = max(abs_key_max2(buf[c].x), abs_key_max2(buf[c].y));
                uint32_t m23 = max(abs_key_max2(buf[c].z), abs_key_max2(buf[c].w));
                key = max(key, max(m01, m23));
            }
        }
    } else {
        for (int64_t idx = tid; idx < nfull; idx += kThreads) {
            // (a default load: the second pass re-reads the row from cache)
            uint4 v = *reinterpret_cast<const uint4 *>(wr + idx * 8);
            key = max(key, max(max(abs_key_max2(v.x), abs_key_max2(v.y)),
                               max(abs_key_max2(v.z), abs_key_max2(v.w))));
        }
    }
    if (tid < tail)
        key = max(key, (uint32_t)(wr[nfull * 8 + tid] & 0x7FFFu));

    key = block_max_u32(key, red);
    const float s = scale_from_key(key);
    if (tid == 0) {
        scale[row] = s;
        if (flag != nullptr && key >= 0x7F80u)
            *flag = 1;
    }

    // s = max(fl32(amax / 448), 1e-12) of a bf16 amax: the quotients by the
    // product and one FMA correction equal the IEEE divisions
    const E4M3Div div(s, true);
    if constexpr (CH > 0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t idx = tid + (int64_t)c * kThreads;
            if (idx < nfull)
                st_nt8(qr + idx * 8, div.codes8(buf[c]));
        }
    } else {
        for (int64_t idx = tid; idx < nfull; idx += kThreads) {
            uint4 v = ld_nt16(wr + idx * 8);
            st_nt8(qr + idx * 8, div.codes8(v));
        }
    }
    if (tid < tail) {
        const float t = __uint_as_float((uint32_t)wr[nfull * 8 + tid] << 16) / s;
        qr[nfull * 8 + tid] = (uint8_t)(e4m3x4(t, 0.f, 0.f, 0.f) & 0xFFu);
    }
}

// Rows that are not 16-byte aligned (a leading dimension that is not a
// multiple of 8, or an offset pointer): the same computation element by
// element, reading the row twice.
__global__ __launch_bounds__(kThreads) void k_quant_weight_scalar(
    const uint16_t *__restrict__ w, int64_t k, int64_t ld_w,
    uint8_t *__restrict__ q, int64_t ld_q, float *__restrict__ scale,
    int32_t *__restrict__ flag)
{
    __shared__ uint32_t red[kThreads / kWave];
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * ld_w;
    uint8_t *qr = q + row * ld_q;
    uint32_t key = 0;
    for (int64_t e = threadIdx.x; e < k; e += kThreads)
        key = max(key, (uint32_t)(wr[e] & 0x7FFFu));
    key = block_max_u32(key, red);
    const float s = scale_from_key(key);
    if (threadIdx.x == 0) {
        scale[row] = s;
        if (flag != nullptr && key >= 0x7F80u)
            *flag = 1;
    }
    for (int64_t e = threadIdx.x; e < k; e += kThreads) {
        const float t = __uint_as_float((uint32_t)wr[e] << 16) / s;
        qr[e] = (uint8_t)(e4m3x4(t, 0.f, 0.f, 0.f) & 0xFFu);
    }
}

// ---------------------------------------------------------------------------
// Weights, per-group scales (the deployment guide §4.3 names per-group
// granularity as the step beyond per-channel): one workgroup per output row.
// A group of 8 * LPG values is the 16-byte chunks of LPG consecutive lanes
// (256 threads hold 256 consecutive chunks per round, and LPG divides 64, so
// a group never straddles a wave); its maximum is a shuffle reduction over
// those lanes.  Every weight byte is read once.  The row's last chunk may be
// partial: its missing values count as 0 (which cannot raise a maximum) and
// are not stored.
// ---------------------------------------------------------------------------
// One 16-byte chunk of a row; a partial chunk is filled with zeros.
__device__ __forceinline__ uint4 load_chunk(const uint16_t *wr, int64_t e0, int valid)
{
    if (valid == 8)
        return ld_nt16(wr + e0);
    uint4 v = {0u, 0u, 0u, 0u};
    if (valid > 0) {
        uint32_t h[8];
        for (int i = 0; i < 8; ++i)
            h[i] = i < valid ? wr[e0 + i] : 0u;
        v = uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
    return v;
}

// Group maximum, scale, codes and (first lane of the group) the scale store
// for one 16-byte chunk c of the row.
template <int LPG>
__device__ __forceinline__ void quant_chunk(uint4 v, int64_t c, int valid, uint8_t *qr, float *sr,
                                            int32_t *flag)
{
    const uint32_t key = group_max_u32<LPG>(key_max8(v));
    const float s = scale_from_key(key);
    const int64_t e0 = c * 8;
    // one reciprocal per chunk; the product and one FMA correction equal the
    // IEEE quotients for this form of scale
    const E4M3Div div(s, true);
    if (valid == 8) {
        st_nt8(qr + e0, div.codes8(v));
    } else if (valid > 0) {
        const uint2 codes = div.codes8(v);
        for (int i = 0; i < valid; ++i)
            qr[e0 + i] = (uint8_t)(((i < 4 ? codes.x : codes.y) >> (8 * (i & 3))) & 0xFFu);
    }
    if (valid > 0 && (threadIdx.x & (LPG - 1)) == 0) {
        sr[c / LPG] = s;
        if (flag != nullptr && key >= 0x7F80u)
            *flag = 1;
    }
}

// CH > 0: the row has at most CH * 256 chunks, all loaded into registers
// before any is reduced, so every lane has CH loads in flight; CH == 0:
// longer rows, one round of 256 chunks at a time.
template <int LPG, int CH>
__global__ __launch_bounds__(kThreads) void k_quant_weight_grouped(
    const uint16_t *__restrict__ w, int64_t k, int64_t ld_w,
    uint8_t *__restrict__ q, int64_t ld_q, float *__restrict__ scale, int64_t ngroups,
    int32_t *__restrict__ flag)
{
    static_assert(LPG >= 1 && LPG <= kWave && (LPG & (LPG - 1)) == 0, "lanes per group");
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * ld_w;
    uint8_t *qr = q + row * ld_q;
    float *sr = scale + row * ngroups;
    auto valid_of = [&](int64_t c) {
        const int64_t e0 = c * 8;
        return e0 >= k ? 0 : (int)min<int64_t>(8, k - e0);
    };
    if constexpr (CH > 0) {
        uint4 buf[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t c = threadIdx.x + (int64_t)i * kThreads;
            buf[i] = load_chunk(wr, c * 8, valid_of(c));
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t c = threadIdx.x + (int64_t)i * kThreads;
            quant_chunk<LPG>(buf[i], c, valid_of(c), qr, sr, flag);
        }
    } else {
        const int64_t nch = (k + 7) >> 3;
        for (int64_t base = 0; base < nch; base += kThreads) {
            const int64_t c = base + threadIdx.x;
            quant_chunk<LPG>(load_chunk(wr, c * 8, valid_of(c)), c, valid_of(c), qr, sr, flag);
        }
    }
}

// Rows that are not 16-byte aligned: one thread per group, element by element.
__global__ __launch_bounds__(kThreads) void k_quant_weight_grouped_scalar(
    const uint16_t *__restrict__ w, int64_t k, int64_t ld_w, int64_t group,
    uint8_t *__restrict__ q, int64_t ld_q, float *__restrict__ scale, int64_t ngroups,
    int32_t *__restrict__ flag)
{
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * ld_w;
    uint8_t *qr = q + row * ld_q;
    for (int64_t gi = threadIdx.x; gi < ngroups; gi += kThreads) {
        const int64_t c0 = gi * group;
        const int64_t c1 = min(k, c0 + group);
        uint32_t key = 0;
        for (int64_t c = c0; c < c1; ++c)
            key = max(key, (uint32_t)(wr[c] & 0x7FFFu));
        const float s = scale_from_key(key);
        scale[row * ngroups + gi] = s;
        if (flag != nullptr && key >= 0x7F80u)
            *flag = 1;
        for (int64_t c = c0; c < c1; ++c) {
            const float t = __uint_as_float((uint32_t)wr[c] << 16) / s;
            qr[c] = (uint8_t)(e4m3x4(t, 0.f, 0.f, 0.f) & 0xFFu);
        }
    }
}

// ---------------------------------------------------------------------------
// Activations, pass 1: each workgroup writes the |x| key maximum of its share
// of the tensor to partial[blockIdx.x].  No atomics, no initialisation.
// ---------------------------------------------------------------------------

// Layouts of an activation tensor, from fastest to most general.
enum ActLayout : int {
    kFlat = 0,      // ld == k, k % 8 == 0, 16-byte aligned: one stream of 16-byte chunks
    kRows = 1,      // rows 16-byte aligned: 16-byte chunks per row, element tail
    kScalar = 2     // anything else: element by element
};

__global__ __launch_bounds__(kThreads) void k_act_amax(
    const uint16_t *__restrict__ x, int64_t m, int64_t k, int64_t ld_x,
    uint32_t *__restrict__ partial, int layout)
{
    __shared__ uint32_t red[kThreads / kWave];
    uint32_t key = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (layout == kScalar) {
        const int64_t total = m * k;
        for (; i < total; i += stride) {
            const int64_t row = i / k;
            key = max(key, (uint32_t)(x[row * ld_x + (i - row * k)] & 0x7FFFu));
        }
    } else if (layout == kFlat) {
        // contiguous tensor: a flat stream of 16-byte chunks, 4 in flight per thread
        const uint4 *p = reinterpret_cast<const uint4 *>(x);
        const int64_t total = m * (k >> 3);
        for (; i + 3 * stride < total; i += 4 * stride) {
            uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
            key = max(key, max(max(key_max8(a), key_max8(b)), max(key_max8(c), key_max8(d))));
        }
        for (; i < total; i += stride)
            key = max(key, key_max8(p[i]));
    } else {
        const int64_t cpr = (k + 7) >> 3;          // chunks per row, last one may be partial
        const int64_t total = m * cpr;
        for (; i < total; i += stride) {
            const int64_t row = i / cpr;
            const int64_t j = (i - row * cpr) * 8;
            const uint16_t *p = x + row * ld_x + j;
            if (j + 8 <= k) {
                key = max(key, key_max8(*reinterpret_cast<const uint4 *>(p)));
            } else {
                for (int64_t e = 0; e < k - j; ++e)
                    key = max(key, (uint32_t)(p[e] & 0x7FFFu));
            }
        }
    }
    key = block_max_u32(key, red);
    if (threadIdx.x == 0)
        partial[blockIdx.x] = key;
}

// ---------------------------------------------------------------------------
// Activations, the cast.  Where its scale comes from:
//   kFromPartials  dynamic quantization, pass 2: every workgroup folds the
//                  pass-1 maxima (a few KB, L2-resident) into the tensor's
//                  scale; workgroup 0 publishes it (to x_scale, and to
//                  seed_out when that is given) with the non-finite flag.
//   kHeld          a scale held in device memory (*held), read once per
//                  workgroup; the tensor is read once.  The |x| maximum is
//                  reduced only to raise the non-finite flag.
//   kHeldTrack     as kHeld, and each workgroup also writes the |x| maximum of
//                  its share to partial_out[blockIdx.x], from the same loads,
//                  for the EMA update that follows.
// ---------------------------------------------------------------------------
enum ScaleSource : int { kFromPartials = 0, kHeld = 1, kHeldTrack = 2 };

template <int SRC>
__global__ __launch_bounds__(kThreads) void k_act_cast(
    const uint16_t *__restrict__ x, int64_t m, int64_t k, int64_t ld_x,
    uint8_t *__restrict__ q, int64_t ld_q,
    const uint32_t *__restrict__ partial, int npart,
    float *__restrict__ x_scale, float *__restrict__ seed_out,
    const float *__restrict__ held, uint32_t *__restrict__ partial_out,
    int32_t *__restrict__ flag, int layout)
{
    constexpr bool kTrack = SRC != kFromPartials;
    __shared__ uint32_t red[kThreads / kWave];
    uint32_t key = 0;
    float s;
    if constexpr (SRC == kFromPartials) {
        for (int j = threadIdx.x; j < npart; j += kThreads)
            key = max(key, partial[j]);
        key = block_max_u32(key, red);
        s = scale_from_key(key);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            *x_scale = s;
            if (seed_out != nullptr)
                *seed_out = s;
            if (flag != nullptr && key >= 0x7F80u)
                *flag = 1;
        }
        key = 0;
    } else {
        s = *held;
    }

    const E4M3Div div(s, SRC == kFromPartials);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (layout == kScalar) {
        const int64_t total = m * k;
        for (; i < total; i += stride) {
            const int64_t row = i / k;
            const int64_t c = i - row * k;
            const uint16_t h = x[row * ld_x + c];
            if constexpr (kTrack)
                key = max(key, (uint32_t)(h & 0x7FFFu));
            const float t = __uint_as_float((uint32_t)h << 16) / s;
            q[row * ld_q + c] = (uint8_t)(e4m3x4(t, 0.f, 0.f, 0.f) & 0xFFu);
        }
    } else if (layout == kFlat) {
        // the tensor's last read and the codes' only write: non-temporal
        const uint4 *p = reinterpret_cast<const uint4 *>(x);
        uint2 *o = reinterpret_cast<uint2 *>(q);
        const int64_t total = m * (k >> 3);
        for (; i + 3 * stride < total; i += 4 * stride) {
            const uint4 a = ld_nt16(p + i), b = ld_nt16(p + i + stride);
            const uint4 c = ld_nt16(p + i + 2 * stride), d = ld_nt16(p + i + 3 * stride);
            if constexpr (kTrack)
                key = max(key, max(max(key_max8(a), key_max8(b)), max(key_max8(c), key_max8(d))));
            st_nt8(o + i, div.codes8(a));
            st_nt8(o + i + stride, div.codes8(b));
            st_nt8(o + i + 2 * stride, div.codes8(c));
            st_nt8(o + i + 3 * stride, div.codes8(d));
        }
        for (; i < total; i += stride) {
            const uint4 a = ld_nt16(p + i);
            if constexpr (kTrack)
                key = max(key, key_max8(a));
            st_nt8(o + i, div.codes8(a));
        }
    } else {
        const int64_t cpr = (k + 7) >> 3;
        const int64_t total = m * cpr;
        for (; i < total; i += stride) {
            const int64_t row = i / cpr;
            const int64_t j = (i - row * cpr) * 8;
            const uint16_t *p = x + row * ld_x + j;
            uint8_t *o = q + row * ld_q + j;
            if (j + 8 <= k) {
                const uint4 a = *reinterpret_cast<const uint4 *>(p);
                if constexpr (kTrack)
                    key = max(key, key_max8(a));
                *reinterpret_cast<uint2 *>(o) = div.codes8(a);
            } else {
                for (int64_t e = 0; e < k - j; ++e) {
                    if constexpr (kTrack)
                        key = max(key, (uint32_t)(p[e] & 0x7FFFu));
                    const float t = __uint_as_float((uint32_t)p[e] << 16) / s;
                    o[e] = (uint8_t)(e4m3x4(t, 0.f, 0.f, 0.f) & 0xFFu);
                }
            }
        }
    }

    if constexpr (SRC == kHeldTrack) {
        key = block_max_u32(key, red);
        if (threadIdx.x == 0)
            partial_out[blockIdx.x] = key;
    } else if constexpr (SRC == kHeld) {
        if (flag != nullptr) {
            key = block_max_u32(key, red);
            if (threadIdx.x == 0 && key >= 0x7F80u)
                *flag = 1;
        }
    }
}

// ---------------------------------------------------------------------------
// EMA step of the per-tensor activation scale ("Llama 3 精读" write-up §3.1
// step 2: a moving average with decay d; §5.3 tip 2: the new term times
// (1 + 0.1 T)).  fp32, evaluated in the written order with every product and
// sum rounded on its own (no fused multiply-add), then the 1e-12 floor that
// every scale of the method keeps.
// ---------------------------------------------------------------------------
__device__ __noinline__ float ema_step(float s_old, float s_new, float decay, float temperature)
{
#pragma clang fp contract(off)
    const float keep = decay * s_old;
    const float weight = 1.0f - decay;
    float fresh = weight * s_new;
    const float heat = 1.0f + 0.1f * temperature;
    fresh = fresh * heat;
    const float s = keep + fresh;
    return s < kScaleFloor ? kScaleFloor : s;
}

// One workgroup: fold the per-workgroup maxima of the tracked cast into the
// tensor's dynamic scale, hand out the scale the cast used, step the state.
__global__ __launch_bounds__(kThreads) void k_act_ema_update(
    const uint32_t *__restrict__ partial, int npart, float *__restrict__ state,
    float *__restrict__ x_scale, float decay, float temperature, int32_t *__restrict__ flag)
{
    __shared__ uint32_t red[kThreads / kWave];
    uint32_t key = 0;
    for (int j = threadIdx.x; j < npart; j += kThreads)
        key = max(key, partial[j]);
    key = block_max_u32(key, red);
    if (threadIdx.x == 0) {
        const float s_old = *state;
        *x_scale = s_old;
        *state = ema_step(s_old, scale_from_key(key), decay, temperature);
        if (flag != nullptr && key >= 0x7F80u)
            *flag = 1;
    }
}

// ---------------------------------------------------------------------------
// Bare cast: fp32 -> E4M3 codes, four per lane per step.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_cast_f32(
    const float *__restrict__ x, int64_t count, uint8_t *__restrict__ out)
{
    const int64_t n4 = count >> 2;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const float4 *p = reinterpret_cast<const float4 *>(x);
    uint32_t *o = reinterpret_cast<uint32_t *>(out);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
        float4 v = p[i];
        o[i] = e4m3x4(v.x, v.y, v.z, v.w);
    }
    if (blockIdx.x == 0 && threadIdx.x < (count & 3)) {
        const int64_t e = n4 * 4 + threadIdx.x;
        out[e] = (uint8_t)(e4m3x4(x[e], 0.f, 0.f, 0.f) & 0xFFu);
    }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (host).
// ---------------------------------------------------------------------------
namespace launch {

static bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipError_t quantize_weight(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                           uint8_t *q, int64_t ld_q, float *scale, int32_t *flag,
                           hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const int64_t per_thread = div_up(k >> 3, kThreads);
    const dim3 grid((unsigned)n), block(kThreads);
    const bool vec = aligned(w, 16) && ld_w % 8 == 0 && aligned(q, 8) && ld_q % 8 == 0;
    if (!vec)
        hipLaunchKernelGGL(k_quant_weight_scalar, grid, block, 0, stream, w, k, ld_w, q, ld_q, scale, flag);
    else if (per_thread <= 1)
        hipLaunchKernelGGL(k_quant_weight<1>, grid, block, 0, stream, w, k, ld_w, q, ld_q, scale, flag);
    else if (per_thread <= 2)
        hipLaunchKernelGGL(k_quant_weight<2>, grid, block, 0, stream, w, k, ld_w, q, ld_q, scale, flag);
    else if (per_thread <= 4)
        hipLaunchKernelGGL(k_quant_weight<4>, grid, block, 0, stream, w, k, ld_w, q, ld_q, scale, flag);
    else if (per_thread <= 8)
        hipLaunchKernelGGL(k_quant_weight<8>, grid, block, 0, stream, w, k, ld_w, q, ld_q, scale, flag);
    else if (per_thread <= 16)
        hipLaunchKernelGGL(k_quant_weight<16>, grid, block, 0, stream, w, k, ld_w, q, ld_q, scale, flag);
    else
        hipLaunchKernelGGL(k_quant_weight<0>, grid, block, 0, stream, w, k, ld_w, q, ld_q, scale, flag);
    return hipGetLastError();
}

hipError_t quantize_weight_grouped(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                                   int64_t group, uint8_t *q, int64_t ld_q, float *scale,
                                   int32_t *flag, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const int64_t ngroups = div_up(k, group);
    const dim3 grid((unsigned)n), block(kThreads);
    const bool vec = aligned(w, 16) && ld_w % 8 == 0 && aligned(q, 8) && ld_q % 8 == 0;
    if (!vec) {
        hipLaunchKernelGGL(k_quant_weight_grouped_scalar, grid, block, 0, stream, w, k, ld_w, group,
                           q, ld_q, scale, ngroups, flag);
        return hipGetLastError();
    }
    const int64_t rounds = div_up(div_up(k, 8), kThreads);     // chunks per thread
#define FP8Q_GQ(LPG)                                                                          \
    do {                                                                                      \
        if (rounds <= 1)                                                                      \
            hipLaunchKernelGGL((k_quant_weight_grouped<LPG, 1>), grid, block, 0, stream, w, k,   \
                               ld_w, q, ld_q, scale, ngroups, flag);                          \
        else if (rounds <= 2)                                                                 \
            hipLaunchKernelGGL((k_quant_weight_grouped<LPG, 2>), grid, block, 0, stream, w, k,   \
                               ld_w, q, ld_q, scale, ngroups, flag);                          \
        else if (rounds <= 4)                                                                 \
            hipLaunchKernelGGL((k_quant_weight_grouped<LPG, 4>), grid, block, 0, stream, w, k,   \
                               ld_w, q, ld_q, scale, ngroups, flag);                          \
        else if (rounds <= 8)                                                                 \
            hipLaunchKernelGGL((k_quant_weight_grouped<LPG, 8>), grid, block, 0, stream, w, k,   \
                               ld_w, q, ld_q, scale, ngroups, flag);                          \
        else                                                                                  \
            hipLaunchKernelGGL((k_quant_weight_grouped<LPG, 0>), grid, block, 0, stream, w, k,   \
                               ld_w, q, ld_q, scale, ngroups, flag);                          \
    } while (0)
    switch (group) {
    case 64: FP8Q_GQ(8); break;
    case 128: FP8Q_GQ(16); break;
    case 256: FP8Q_GQ(32); break;
    case 512: FP8Q_GQ(64); break;
    default: return hipErrorInvalidValue;
    }
#undef FP8Q_GQ
    return hipGetLastError();
}

// Blocks of the activation passes: about two 16-byte chunks per thread up to
// kActMaxBlocks blocks (a decode-sized tensor then spreads over tens of CUs
// instead of one or two), more per thread beyond.
int act_blocks(int64_t m, int64_t k)
{
    const int64_t chunks = m * div_up(k, 8);
    int64_t g = div_up(chunks, (int64_t)kThreads * 2);
    if (g < 1)
        g = 1;
    if (g > kActMaxBlocks)
        g = kActMaxBlocks;
    return (int)g;
}

static int act_layout(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x, const uint8_t *q,
                      int64_t ld_q)
{
    (void)m;
    const bool rows_ok = aligned(x, 16) && ld_x % 8 == 0 && aligned(q, 8) && ld_q % 8 == 0;
    return !rows_ok ? kScalar : (ld_x == k && ld_q == k && k % 8 == 0) ? kFlat : kRows;
}

hipError_t act_amax(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x, uint32_t *partial,
                    hipStream_t stream)
{
    const int g = act_blocks(m, k);
    const bool rows_ok = aligned(x, 16) && ld_x % 8 == 0;
    const int layout = !rows_ok ? kScalar : (ld_x == k && k % 8 == 0) ? kFlat : kRows;
    hipLaunchKernelGGL(k_act_amax, dim3(g), dim3(kThreads), 0, stream, x, m, k, ld_x, partial,
                       layout);
    return hipGetLastError();
}

// Dynamic per-tensor quantization: the absmax pass, then the cast that folds
// its partial maxima.  seed_out (optional) receives a copy of the scale.
static hipError_t quantize_act_dynamic(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                                       uint8_t *q, int64_t ld_q, float *x_scale, float *seed_out,
                                       uint32_t *partial, int32_t *flag, hipStream_t stream)
{
    const int g = act_blocks(m, k);
    const int layout = act_layout(x, m, k, ld_x, q, ld_q);
    hipLaunchKernelGGL(k_act_amax, dim3(g), dim3(kThreads), 0, stream, x, m, k, ld_x, partial,
                       layout);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_act_cast<kFromPartials>, dim3(g), dim3(kThreads), 0, stream, x, m, k,
                       ld_x, q, ld_q, (const uint32_t *)partial, g, x_scale, seed_out,
                       (const float *)nullptr, (uint32_t *)nullptr, flag, layout);
    return hipGetLastError();
}

hipError_t quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                        uint8_t *q, int64_t ld_q, float *x_scale, uint32_t *partial,
                        int32_t *flag, hipStream_t stream)
{
    return quantize_act_dynamic(x, m, k, ld_x, q, ld_q, x_scale, nullptr, partial, flag, stream);
}

hipError_t quantize_act_static(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                               const float *scale, uint8_t *q, int64_t ld_q, int32_t *flag,
                               hipStream_t stream)
{
    const int g = act_blocks(m, k);
    const int layout = act_layout(x, m, k, ld_x, q, ld_q);
    hipLaunchKernelGGL(k_act_cast<kHeld>, dim3(g), dim3(kThreads), 0, stream, x, m, k, ld_x, q,
                       ld_q, (const uint32_t *)nullptr, 0, (float *)nullptr, (float *)nullptr,
                       scale, (uint32_t *)nullptr, flag, layout);
    return hipGetLastError();
}

hipError_t quantize_act_ema(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                            uint8_t *q, int64_t ld_q, float *x_scale, float *state,
                            float decay, float temperature, bool seed, uint32_t *partial,
                            int32_t *flag, hipStream_t stream)
{
    if (seed)
        return quantize_act_dynamic(x, m, k, ld_x, q, ld_q, x_scale, state, partial, flag, stream);
    const int g = act_blocks(m, k);
    const int layout = act_layout(x, m, k, ld_x, q, ld_q);
    hipLaunchKernelGGL(k_act_cast<kHeldTrack>, dim3(g), dim3(kThreads), 0, stream, x, m, k, ld_x,
                       q, ld_q, (const uint32_t *)nullptr, 0, (float *)nullptr, (float *)nullptr,
                       (const float *)state, partial, (int32_t *)nullptr, layout);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_act_ema_update, dim3(1), dim3(kThreads), 0, stream,
                       (const uint32_t *)partial, g, state, x_scale, decay, temperature, flag);
    return hipGetLastError();
}

hipError_t cast_f32(const float *x, int64_t count, uint8_t *out, hipStream_t stream)
{
    if (count == 0)
        return hipSuccess;
    int64_t g = div_up(div_up(count, 4), (int64_t)kThreads * 4);
    if (g < 1)
        g = 1;
    if (g > 4096)
        g = 4096;
    hipLaunchKernelGGL(k_cast_f32, dim3((unsigned)g), dim3(kThreads), 0, stream, x, count, out);
    return hipGetLastError();
}

}  // namespace launch
}  // namespace fp8q
