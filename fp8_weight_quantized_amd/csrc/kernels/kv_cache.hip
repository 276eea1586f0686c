// FP8 KV-cache write with an online running-max scale.
//
// The deployment guide ("FP8量化与长上下文实测：Llama 3 70B部署优化指南", §3.2)
// quantizes the KV cache with scales that cannot be computed ahead of time:
// each attention layer keeps a running maximum, every prefill batch raises
// it, and decode casts new K/V with the scale as it stands.  The scale and
// the cast are those of §3.1.  Here K and V keep one running maximum each.
//
// New tokens arrive token-major, as the k/v projections produce them
// ([tokens, heads * head_dim] bf16); the cache of one layer is head-major,
// [heads, slots, head_dim] E4M3 codes (the contiguous layout of the "Some
// Technical Notes About Llama 3" commentary, §3.2).  Token t goes to cache
// row slot[t]; rows outside the cache are skipped and flagged, never written.
//
// Both kernels stream 16-byte chunks (8 values of one head) with a flat,
// grid-strided index; blockIdx.y selects K (0) or V (1).  HBM-bound: 2 B in
// and 1 B out per value, plus a second read of the batch when calibrating.
#include "device_common.hpp"
#include "e4m3_div.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

constexpr int kThreads = 256;

// Flag bits reported to the caller.
constexpr int32_t kFlagNonFinite = 1;
constexpr int32_t kFlagBadSlot = 2;

struct KvArgs {
    const uint16_t *src[2];      // K, V: [tokens, ld] bf16
    uint8_t *cache[2];           // K, V caches: [heads, slots, head_dim]
    const int64_t *slot;         // [tokens]
    float *running;              // [2] running max of |K|, |V|
    float *scale_out;            // [2] the scales the codes were made with
    uint32_t *partial;           // [2][gridDim.x] per-block |x| key maxima (calibrating)
    int32_t *flags;              // optional
    int64_t ld;
    int64_t slots;
    uint32_t chunks;             // tokens * heads * head_dim / 8
    uint32_t per_token;          // heads * head_dim / 8
    uint32_t per_head;           // head_dim / 8
    uint32_t head_dim;
};

// Calibrating calls, pass 1: |x| maximum of each block's share of K or V.
__global__ __launch_bounds__(kThreads) void k_kv_amax(KvArgs a)
{
    __shared__ uint32_t red[kThreads / kWave];
    const int which = blockIdx.y;
    const uint16_t *x = which ? a.src[1] : a.src[0];
    uint32_t key = 0;
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < a.chunks; i += stride) {
        const uint32_t t = i / a.per_token;
        const uint32_t c = i - t * a.per_token;
        key = max(key, key_max8(*reinterpret_cast<const uint4 *>(x + t * a.ld + (int64_t)c * 8)));
    }
    key = block_max_u32(key, red);
    if (threadIdx.x == 0)
        a.partial[which * gridDim.x + blockIdx.x] = key;
}

// The cast.  CAL: fold pass 1's maxima, raise the running maximum (every
// block computes the same value; block 0 stores it), then cast with the
// raised scale.  !CAL: cast with the scale of the running maximum as it is.
// RCP (a prefill chunk, several chunks per thread): the quotients by one
// reciprocal and two FMA correction steps (the running maximum may have been
// set by the caller, so the scale need not have the dynamic form; two steps
// are exact for any normal scale, and other scales take the IEEE division),
// the same codes as the division per value that !RCP (a decode step's few
// tokens) does.
template <bool CAL, bool RCP>
__global__ __launch_bounds__(kThreads) void k_kv_cast(KvArgs a)
{
    __shared__ uint32_t red[kThreads / kWave];
    __shared__ int32_t bad;
    const int which = blockIdx.y;
    if (threadIdx.x == 0)
        bad = 0;
    float r = which ? a.running[1] : a.running[0];
    if constexpr (CAL) {
        uint32_t key = 0;
        for (uint32_t j = threadIdx.x; j < gridDim.x; j += kThreads)
            key = max(key, a.partial[which * gridDim.x + j]);
        key = block_max_u32(key, red);
        const float amax = __uint_as_float(key << 16);
        // a NaN maximum leaves r as it was (the flag reports the input)
        r = amax > r ? amax : r;
    } else {
        __syncthreads();
    }
    float s = r / kE4M3Max;
    s = s < kScaleFloor ? kScaleFloor : s;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if constexpr (CAL)
            a.running[which] = r;
        a.scale_out[which] = s;
    }
    const uint16_t *x = which ? a.src[1] : a.src[0];
    uint8_t *cache = which ? a.cache[1] : a.cache[0];
    int32_t local = 0;
    const uint32_t stride = gridDim.x * kThreads;
    [[maybe_unused]] const E4M3Div div(RCP ? s : 1.0f);
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < a.chunks; i += stride) {
        const uint32_t t = i / a.per_token;
        const uint32_t c = i - t * a.per_token;
        const uint32_t h = c / a.per_head;
        const uint32_t j = c - h * a.per_head;
        const uint4 v = *reinterpret_cast<const uint4 *>(x + t * a.ld + (int64_t)c * 8);
        if (key_max8(v) >= 0x7F80u)
            local |= kFlagNonFinite;
        const int64_t row = a.slot[t];
        if (row < 0 || row >= a.slots) {
            local |= kFlagBadSlot;
            continue;
        }
        *reinterpret_cast<uint2 *>(cache + ((int64_t)h * a.slots + row) * a.head_dim + j * 8) =
            RCP ? div.codes8(v) : quantize8(v, s);
    }
    if (a.flags != nullptr) {
        if (local != 0)
            atomicOr(&bad, local);
        __syncthreads();
        if (threadIdx.x == 0 && bad != 0)
            atomicOr(a.flags, bad);
    }
}

}  // namespace

namespace launch {

int kv_blocks(int64_t tokens, int64_t heads, int64_t head_dim)
{
    const int64_t chunks = tokens * heads * head_dim / 8;
    int64_t g = (chunks + 2 * kThreads - 1) / (2 * kThreads);
    if (g < 1)
        g = 1;
    if (g > kActMaxBlocks)
        g = kActMaxBlocks;
    return (int)g;
}

hipError_t kv_cache_write(const uint16_t *k, const uint16_t *v, int64_t tokens, int64_t heads,
                          int64_t head_dim, int64_t ld, const int64_t *slot, uint8_t *k_cache,
                          uint8_t *v_cache, int64_t slots, float *running, float *scale_out,
                          bool calibrate, uint32_t *partial, int32_t *flags, hipStream_t stream)
{
    KvArgs a;
    a.src[0] = k;
    a.src[1] = v;
    a.cache[0] = k_cache;
    a.cache[1] = v_cache;
    a.slot = slot;
    a.running = running;
    a.scale_out = scale_out;
    a.partial = partial;
    a.flags = flags;
    a.ld = ld;
    a.slots = slots;
    a.chunks = (uint32_t)(tokens * heads * head_dim / 8);
    a.per_token = (uint32_t)(heads * head_dim / 8);
    a.per_head = (uint32_t)(head_dim / 8);
    a.head_dim = (uint32_t)head_dim;
    const dim3 grid((unsigned)kv_blocks(tokens, heads, head_dim), 2), block(kThreads);
    // at least 4 chunks per thread: the reciprocal's setup pays off
    const bool rcp = (int64_t)a.chunks >= 4 * (int64_t)grid.x * kThreads;
    if (calibrate) {
        hipLaunchKernelGGL(k_kv_amax, grid, block, 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if (rcp)
            hipLaunchKernelGGL((k_kv_cast<true, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_kv_cast<true, false>), grid, block, 0, stream, a);
    } else {
        if (rcp)
            hipLaunchKernelGGL((k_kv_cast<false, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_kv_cast<false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace launch
}  // namespace fp8q
