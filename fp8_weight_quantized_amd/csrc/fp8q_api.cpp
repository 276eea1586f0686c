// C ABI of the fp8q library: argument validation, device checks and kernel
// dispatch.  Nothing here allocates device memory or synchronizes; every
// kernel is enqueued on the caller's stream.  The operations are documented
// in include/fp8q.h.
#include "fp8q.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels/launch.hpp"

namespace {

thread_local char g_err[512] = "";

fp8q_status fail(fp8q_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fp8q_status ok()
{
    g_err[0] = '\0';
    return FP8Q_OK;
}

fp8q_status hip_fail(hipError_t e, const char *what)
{
    return fail(FP8Q_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- per-device property cache ---------------------------------------------
constexpr int kMaxDevices = 64;
struct DeviceInfo {
    bool known = false;
    bool gfx950 = false;
    char arch[64] = "";
};
std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

fp8q_status stream_device(hipStream_t stream, int *dev)
{
    hipDevice_t d = 0;
    hipError_t e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FP8Q_ERR_HIP, "cannot query the device of the stream: %s", hipGetErrorString(e));
    }
    *dev = (int)d;
    if (*dev < 0 || *dev >= kMaxDevices)
        return fail(FP8Q_ERR_UNSUPPORTED, "device ordinal %d out of range", *dev);
    return FP8Q_OK;
}

fp8q_status check_device(int dev)
{
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo &info = g_dev[dev];
    if (!info.known) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return hip_fail(e, "hipGetDeviceProperties");
        }
        std::snprintf(info.arch, sizeof(info.arch), "%s", prop.gcnArchName);
        info.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        info.known = true;
    }
    if (!info.gfx950)
        return fail(FP8Q_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev,
                    info.arch);
    return FP8Q_OK;
}

// The device of `stream`, checked to be a gfx950.
fp8q_status prepare(hipStream_t stream, int *dev)
{
    fp8q_status s = stream_device(stream, dev);
    if (s != FP8Q_OK)
        return s;
    return check_device(*dev);
}

// Device allocations this thread has already validated.  A pointer inside
// one of them skips the runtime query: hipPointerGetAttributes looks the
// address up among all of the process's allocations, which costs
// microseconds per pointer once a process holds many of them.  The last
// kKnownRanges allocations are remembered, replaced in turn.
// FP8Q_POINTER_CACHE=0 turns the memory off.  Not detected while a range is
// remembered: an allocation that is freed and whose address range is handed
// to host memory afterwards.
struct KnownRange {
    uintptr_t lo = 0, hi = 0;
    int dev = -1;
};
constexpr int kKnownRanges = 32;
thread_local KnownRange t_known[kKnownRanges];
thread_local int t_known_next = 0;

bool pointer_cache_on()
{
    static const bool on = [] {
        const char *e = std::getenv("FP8Q_POINTER_CACHE");
        return !(e != nullptr && std::strcmp(e, "0") == 0);
    }();
    return on;
}

bool known_device_pointer(uintptr_t q, int dev)
{
    for (const KnownRange &r : t_known)
        if (r.dev == dev && q >= r.lo && q < r.hi)
            return true;
    return false;
}

void remember_allocation(const void *p, int dev)
{
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) != hipSuccess || size == 0) {
        (void)hipGetLastError();
        return;
    }
    KnownRange &r = t_known[t_known_next];
    r.lo = reinterpret_cast<uintptr_t>(base);
    r.hi = r.lo + size;
    r.dev = dev;
    t_known_next = (t_known_next + 1) % kKnownRanges;
}

// A pointer the kernels will dereference: non-null, aligned, device memory
// on the stream's device.
fp8q_status check_ptr(const void *p, const char *name, int dev, size_t align)
{
    if (p == nullptr)
        return fail(FP8Q_ERR_INVALID_ARG, "%s is NULL", name);
    if (align > 1 && (reinterpret_cast<uintptr_t>(p) % align) != 0)
        return fail(FP8Q_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
    const bool cache = pointer_cache_on();
    if (cache && known_device_pointer(reinterpret_cast<uintptr_t>(p), dev))
        return FP8Q_OK;
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FP8Q_ERR_INVALID_ARG, "%s is not device memory (%s)", name, hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged && !attr.isManaged)
        return fail(FP8Q_ERR_INVALID_ARG, "%s is not device memory (memory type %d)", name,
                    (int)attr.type);
    if (attr.device != dev)
        return fail(FP8Q_ERR_INVALID_ARG, "%s lives on device %d but the stream is on device %d",
                    name, attr.device, dev);
    if (cache)
        remember_allocation(p, dev);
    return FP8Q_OK;
}

// The bytes [p, p + bytes) must lie inside one device allocation (the one
// hipMemGetAddressRange reports for p).  A runtime that cannot answer skips
// the check.
fp8q_status check_within_allocation(const void *p, size_t bytes, const char *name)
{
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    hipError_t e = hipMemGetAddressRange(&base, &size, const_cast<void *>(p));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return FP8Q_OK;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    if (q < b || q - b + bytes > size)
        return fail(FP8Q_ERR_INVALID_ARG, "%s: %zu bytes from this pointer run past its allocation",
                    name, bytes);
    return FP8Q_OK;
}

// Byte extent of a row-major [rows, cols] matrix with row stride ld.
size_t extent(int64_t rows, int64_t cols, int64_t ld, size_t elem)
{
    if (rows <= 0 || cols <= 0)
        return 0;
    return (size_t)((rows - 1) * ld + cols) * elem;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (na == 0 || nb == 0)
        return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

fp8q_status check_ld(int64_t ld, int64_t cols, int64_t multiple, const char *name)
{
    if (ld < cols)
        return fail(FP8Q_ERR_INVALID_ARG, "%s = %lld is smaller than the row length %lld", name,
                    (long long)ld, (long long)cols);
    if (ld % multiple != 0)
        return fail(FP8Q_ERR_INVALID_ARG, "%s = %lld is not a multiple of %lld", name,
                    (long long)ld, (long long)multiple);
    return FP8Q_OK;
}

#define FP8Q_TRY(expr)                   \
    do {                                 \
        fp8q_status _s = (expr);         \
        if (_s != FP8Q_OK)               \
            return _s;                   \
    } while (0)

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

extern "C" {

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

const char *fp8q_status_string(fp8q_status s)
{
    switch (s) {
    case FP8Q_OK: return "FP8Q_OK";
    case FP8Q_ERR_INVALID_ARG: return "FP8Q_ERR_INVALID_ARG: invalid argument";
    case FP8Q_ERR_UNSUPPORTED: return "FP8Q_ERR_UNSUPPORTED: device is not gfx950";
    case FP8Q_ERR_HIP: return "FP8Q_ERR_HIP: HIP runtime or launch error";
    case FP8Q_ERR_WORKSPACE: return "FP8Q_ERR_WORKSPACE: workspace missing or too small";
    default: break;
    }
    return "FP8Q: unknown status";
}

const char *fp8q_last_error(void) { return g_err; }

fp8q_status fp8q_quantize_weight(const uint16_t *w_bf16, int64_t n, int64_t k, int64_t ld_w,
                                 uint8_t *w_fp8, int64_t ld_q, float *w_scale,
                                 int32_t *nonfinite_flag, hipStream_t stream)
{
    if (n < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need n >= 0 and k >= 1 (n=%lld, k=%lld)", (long long)n,
                    (long long)k);
    FP8Q_TRY(check_ld(ld_w, k, 1, "ld_w"));
    FP8Q_TRY(check_ld(ld_q, k, 1, "ld_q"));
    if (n == 0)
        return ok();
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    FP8Q_TRY(check_ptr(w_bf16, "w_bf16", dev, 2));
    FP8Q_TRY(check_ptr(w_fp8, "w_fp8", dev, 1));
    FP8Q_TRY(check_ptr(w_scale, "w_scale", dev, 4));
    if (nonfinite_flag != nullptr)
        FP8Q_TRY(check_ptr(nonfinite_flag, "nonfinite_flag", dev, 4));
    const size_t ew = extent(n, k, ld_w, 2), eq = extent(n, k, ld_q, 1), es = (size_t)n * 4;
    if (overlap(w_fp8, eq, w_bf16, ew) || overlap(w_scale, es, w_bf16, ew) ||
        overlap(w_scale, es, w_fp8, eq))
        return fail(FP8Q_ERR_INVALID_ARG, "outputs overlap each other or the input");
    hipError_t e = fp8q::launch::quantize_weight(w_bf16, n, k, ld_w, w_fp8, ld_q, w_scale,
                                                 nonfinite_flag, stream);
    if (e != hipSuccess)
        return hip_fail(e, "weight quantization launch");
    return ok();
}

size_t fp8q_quantize_act_workspace_size(int64_t m, int64_t k)
{
    if (m < 0 || k < 1)
        return 0;
    return round_up((size_t)fp8q::launch::act_blocks(m, k) * sizeof(uint32_t), 256);
}

fp8q_status fp8q_quantize_act(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                              uint8_t *x_fp8, int64_t ld_q, float *x_scale,
                              void *workspace, size_t workspace_bytes,
                              int32_t *nonfinite_flag, hipStream_t stream)
{
    if (m < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need m >= 0 and k >= 1 (m=%lld, k=%lld)", (long long)m,
                    (long long)k);
    FP8Q_TRY(check_ld(ld_x, k, 1, "ld_x"));
    FP8Q_TRY(check_ld(ld_q, k, 1, "ld_q"));
    const size_t need = fp8q_quantize_act_workspace_size(m, k);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FP8Q_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                    workspace == nullptr ? (size_t)0 : workspace_bytes, need);
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    if (m > 0) {
        FP8Q_TRY(check_ptr(x_bf16, "x_bf16", dev, 2));
        FP8Q_TRY(check_ptr(x_fp8, "x_fp8", dev, 1));
    }
    FP8Q_TRY(check_ptr(x_scale, "x_scale", dev, 4));
    FP8Q_TRY(check_ptr(workspace, "workspace", dev, 16));
    if (nonfinite_flag != nullptr)
        FP8Q_TRY(check_ptr(nonfinite_flag, "nonfinite_flag", dev, 4));
    const size_t ex = extent(m, k, ld_x, 2), eq = extent(m, k, ld_q, 1);
    if (overlap(x_fp8, eq, x_bf16, ex) || overlap(x_scale, 4, x_bf16, ex) ||
        overlap(x_scale, 4, x_fp8, eq) || overlap(workspace, need, x_bf16, ex) ||
        overlap(workspace, need, x_fp8, eq) || overlap(workspace, need, x_scale, 4))
        return fail(FP8Q_ERR_INVALID_ARG, "outputs, workspace and input overlap");
    hipError_t e = fp8q::launch::quantize_act(x_bf16, m, k, ld_x, x_fp8, ld_q, x_scale,
                                              static_cast<uint32_t *>(workspace), nonfinite_flag,
                                              stream);
    if (e != hipSuccess)
        return hip_fail(e, "activation quantization launch");
    return ok();
}

fp8q_status fp8q_quantize_act_static(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                     const float *x_scale, uint8_t *x_fp8, int64_t ld_q,
                                     int32_t *nonfinite_flag, hipStream_t stream)
{
    if (m < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need m >= 0 and k >= 1 (m=%lld, k=%lld)", (long long)m,
                    (long long)k);
    FP8Q_TRY(check_ld(ld_x, k, 1, "ld_x"));
    FP8Q_TRY(check_ld(ld_q, k, 1, "ld_q"));
    if (m == 0)
        return ok();
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    FP8Q_TRY(check_ptr(x_bf16, "x_bf16", dev, 2));
    FP8Q_TRY(check_ptr(x_fp8, "x_fp8", dev, 1));
    FP8Q_TRY(check_ptr(x_scale, "x_scale", dev, 4));
    if (nonfinite_flag != nullptr)
        FP8Q_TRY(check_ptr(nonfinite_flag, "nonfinite_flag", dev, 4));
    const size_t ex = extent(m, k, ld_x, 2), eq = extent(m, k, ld_q, 1);
    if (overlap(x_fp8, eq, x_bf16, ex) || overlap(x_fp8, eq, x_scale, 4))
        return fail(FP8Q_ERR_INVALID_ARG, "x_fp8 overlaps the input or the scale");
    hipError_t e = fp8q::launch::quantize_act_static(x_bf16, m, k, ld_x, x_scale, x_fp8, ld_q,
                                                     nonfinite_flag, stream);
    if (e != hipSuccess)
        return hip_fail(e, "static activation quantization launch");
    return ok();
}

fp8q_status fp8q_quantize_act_ema(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                  uint8_t *x_fp8, int64_t ld_q, float *x_scale, float *state,
                                  float decay, float temperature, int seed,
                                  void *workspace, size_t workspace_bytes,
                                  int32_t *nonfinite_flag, hipStream_t stream)
{
    if (m < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need m >= 0 and k >= 1 (m=%lld, k=%lld)", (long long)m,
                    (long long)k);
    if (!(decay >= 0.0f && decay <= 1.0f))
        return fail(FP8Q_ERR_INVALID_ARG, "decay must lie in [0, 1] (got %g)", (double)decay);
    if (!(temperature >= 0.0f && temperature <= 3.0e38f))
        return fail(FP8Q_ERR_INVALID_ARG, "temperature must be finite and >= 0 (got %g)",
                    (double)temperature);
    FP8Q_TRY(check_ld(ld_x, k, 1, "ld_x"));
    FP8Q_TRY(check_ld(ld_q, k, 1, "ld_q"));
    const size_t need = fp8q_quantize_act_workspace_size(m, k);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FP8Q_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                    workspace == nullptr ? (size_t)0 : workspace_bytes, need);
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    if (m > 0) {
        FP8Q_TRY(check_ptr(x_bf16, "x_bf16", dev, 2));
        FP8Q_TRY(check_ptr(x_fp8, "x_fp8", dev, 1));
    }
    FP8Q_TRY(check_ptr(x_scale, "x_scale", dev, 4));
    FP8Q_TRY(check_ptr(state, "state", dev, 4));
    FP8Q_TRY(check_ptr(workspace, "workspace", dev, 16));
    if (nonfinite_flag != nullptr)
        FP8Q_TRY(check_ptr(nonfinite_flag, "nonfinite_flag", dev, 4));
    const size_t ex = extent(m, k, ld_x, 2), eq = extent(m, k, ld_q, 1);
    const void *outs[4] = {x_fp8, x_scale, state, workspace};
    const size_t lens[4] = {eq, 4, 4, need};
    for (int a = 0; a < 4; ++a) {
        if (overlap(outs[a], lens[a], x_bf16, ex))
            return fail(FP8Q_ERR_INVALID_ARG, "outputs, state and workspace must not overlap x");
        for (int b = a + 1; b < 4; ++b)
            if (overlap(outs[a], lens[a], outs[b], lens[b]))
                return fail(FP8Q_ERR_INVALID_ARG,
                            "x_fp8, x_scale, state and workspace must not overlap");
    }
    hipError_t e = fp8q::launch::quantize_act_ema(x_bf16, m, k, ld_x, x_fp8, ld_q, x_scale, state,
                                                  decay, temperature, seed != 0,
                                                  static_cast<uint32_t *>(workspace),
                                                  nonfinite_flag, stream);
    if (e != hipSuccess)
        return hip_fail(e, "EMA activation quantization launch");
    return ok();
}

size_t fp8q_kv_cache_workspace_size(int64_t tokens, int64_t heads, int64_t head_dim)
{
    if (tokens < 0 || heads < 1 || head_dim < 8)
        return 0;
    return round_up((size_t)2 * fp8q::launch::kv_blocks(tokens, heads, head_dim) * sizeof(uint32_t),
                    256);
}

fp8q_status fp8q_kv_cache_write(const uint16_t *k_bf16, const uint16_t *v_bf16, int64_t tokens,
                                int64_t heads, int64_t head_dim, int64_t ld,
                                const int64_t *slot, uint8_t *k_cache, uint8_t *v_cache,
                                int64_t slots, float *running_max, float *scale_out,
                                int calibrate, void *workspace, size_t workspace_bytes,
                                int32_t *flags, hipStream_t stream)
{
    if (tokens < 0 || heads < 1 || slots < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need tokens >= 0, heads >= 1 and slots >= 1");
    if (head_dim < 8 || head_dim % 8 != 0)
        return fail(FP8Q_ERR_INVALID_ARG, "head_dim must be a positive multiple of 8 (got %lld)",
                    (long long)head_dim);
    const int64_t width = heads * head_dim;
    if (width > ((int64_t)1 << 30) || slots > ((int64_t)1 << 40))
        return fail(FP8Q_ERR_INVALID_ARG, "heads * head_dim or slots too large");
    FP8Q_TRY(check_ld(ld, width, 8, "ld"));
    if (tokens > 0 && tokens > (((int64_t)1 << 31) - 1) / (width / 8))
        return fail(FP8Q_ERR_INVALID_ARG, "tokens * heads * head_dim / 8 must stay below 2^31");
    const size_t need = fp8q_kv_cache_workspace_size(tokens, heads, head_dim);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FP8Q_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                    workspace == nullptr ? (size_t)0 : workspace_bytes, need);
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    if (tokens > 0) {
        FP8Q_TRY(check_ptr(k_bf16, "k_bf16", dev, 16));
        FP8Q_TRY(check_ptr(v_bf16, "v_bf16", dev, 16));
        FP8Q_TRY(check_ptr(slot, "slot", dev, 8));
    }
    FP8Q_TRY(check_ptr(k_cache, "k_cache", dev, 8));
    FP8Q_TRY(check_ptr(v_cache, "v_cache", dev, 8));
    FP8Q_TRY(check_ptr(running_max, "running_max", dev, 4));
    FP8Q_TRY(check_ptr(scale_out, "scale_out", dev, 4));
    FP8Q_TRY(check_ptr(workspace, "workspace", dev, 16));
    if (flags != nullptr)
        FP8Q_TRY(check_ptr(flags, "flags", dev, 4));
    const size_t ein = tokens > 0 ? extent(tokens, width, ld, 2) : 0;
    const size_t ecache = (size_t)heads * (size_t)slots * (size_t)head_dim;
    FP8Q_TRY(check_within_allocation(k_cache, ecache, "k_cache"));
    FP8Q_TRY(check_within_allocation(v_cache, ecache, "v_cache"));
    const void *outs[5] = {k_cache, v_cache, running_max, scale_out, workspace};
    const size_t lens[5] = {ecache, ecache, 8, 8, need};
    const void *ins[3] = {k_bf16, v_bf16, slot};
    const size_t inl[3] = {ein, ein, tokens > 0 ? (size_t)tokens * 8 : 0};
    for (int a = 0; a < 5; ++a) {
        for (int b = 0; b < 3; ++b)
            if (inl[b] > 0 && overlap(outs[a], lens[a], ins[b], inl[b]))
                return fail(FP8Q_ERR_INVALID_ARG, "an output overlaps k, v or slot");
        for (int b = a + 1; b < 5; ++b)
            if (overlap(outs[a], lens[a], outs[b], lens[b]))
                return fail(FP8Q_ERR_INVALID_ARG,
                            "caches, running_max, scale_out and workspace must not overlap");
    }
    if (flags != nullptr)
        for (int a = 0; a < 5; ++a)
            if (overlap(flags, 4, outs[a], lens[a]))
                return fail(FP8Q_ERR_INVALID_ARG, "flags overlaps an output");
    hipError_t e = fp8q::launch::kv_cache_write(k_bf16, v_bf16, tokens, heads, head_dim, ld, slot,
                                                k_cache, v_cache, slots, running_max, scale_out,
                                                calibrate != 0, static_cast<uint32_t *>(workspace),
                                                flags, stream);
    if (e != hipSuccess)
        return hip_fail(e, "KV-cache write launch");
    return ok();
}

// W8A8 calls with this many activation rows or fewer run the decode kernels
// (E4M3 activations widened to bf16), where the prefill GEMM's 256-row tiles
// would leave most of the GPU idle.
constexpr int64_t kW8A8DecodeMaxM = 64;

namespace {

bool valid_group(int64_t group)
{
    return group == 64 || group == 128 || group == 256 || group == 512;
}

bool mid_rows_decode_cheaper(fp8q_mode mode, int64_t m, int64_t n, int64_t k, double gemm_scale);
size_t grouped_decode_workspace(fp8q_mode mode, int64_t m, int64_t n, int64_t k, int64_t group);

// Grouped fp8_w_fp8_a with more than the decode rows runs the FP8 MFMA GEMM,
// which folds group scales at its 128-k stages (groups of 128 k or more),
// except where the decode kernels are cheaper (the rule of rows_on_decode
// below, with the grouped GEMM's cost about 1.25x the per-channel one's).
bool grouped_uses_gemm(fp8q_mode mode, int64_t m, int64_t n, int64_t k, int64_t group)
{
    if (mode != FP8Q_W8A8 || m <= kW8A8DecodeMaxM || group < 128)
        return false;
    return !(mid_rows_decode_cheaper(mode, m, n, k, 1.25) &&
             grouped_decode_workspace(mode, m, n, k, group) <= ((size_t)4 << 20));
}

int act_type(fp8q_mode mode)
{
    return mode == FP8Q_W8A16       ? fp8q::launch::kW8A16ActBF16
           : mode == FP8Q_W8A16_F16 ? fp8q::launch::kW8A16ActF16
                                    : fp8q::launch::kW8A16ActF8;
}

// Whether a per-channel call runs the decode kernels rather than a prefill
// GEMM (the FP8 one for fp8_w_fp8_a, the 16-bit one for the other two modes).
// Up to 64 rows always.  From 65 to 1024 rows a GEMM whose grid is one round
// of a few 256 x 256 tiles keeps most CUs idle through its whole K loop,
// while the decode kernels run the rows as 64-row groups along their grid,
// each group streaming W (the later ones largely from L2).  The choice takes
// the cheaper of two cost estimates in microseconds, fitted to measurements
// on MI355X (K = 4096; N = 4096, 8192, 28672; M = 65..1024; HIP graphs with
// the weights rotated past the Infinity Cache):
//   decode kernels   5 + ceil(M / 64) * N * K / 3.5e6
//   FP8 GEMM         rounds * (K / 128) * 1.45
//   16-bit GEMM      rounds * (K / 64) * 1.4
// where rounds = ceil(256 x 256 tiles / 256).  E.g. N = K = 4096 at 128 rows:
// 18 us on the decode kernels against 44 us (FP8) and 85 us (16-bit) for the
// GEMMs; N = 28672 keeps the FP8 GEMM from 65 rows on.  Plans whose K-split
// scratch would pass 4 MiB keep the GEMM.
constexpr int64_t kMidRowsMax = 1024;
constexpr size_t kMidRowsMaxWorkspace = (size_t)4 << 20;

// the estimates above for 65..1024 rows; gemm_scale scales the GEMM's
bool mid_rows_decode_cheaper(fp8q_mode mode, int64_t m, int64_t n, int64_t k, double gemm_scale)
{
    if (m <= kW8A8DecodeMaxM || m > kMidRowsMax)
        return false;
    const double tiles = (double)((m + 255) / 256) * (double)((n + 255) / 256);
    const double rounds = (double)(int64_t)((tiles + 255.0) / 256.0);
    const double gemm = mode == FP8Q_W8A8 ? rounds * (double)k / 128.0 * 1.45
                                          : rounds * (double)k / 64.0 * 1.4;
    const double decode = 5.0 + (double)((m + 63) / 64) * (double)n * (double)k / 3.5e6;
    return decode < gemm * gemm_scale;
}

size_t grouped_decode_workspace(fp8q_mode mode, int64_t m, int64_t n, int64_t k, int64_t group)
{
    return fp8q::launch::plan_w8a16_grouped(m, n, k, group, act_type(mode)).workspace;
}

bool rows_on_decode(fp8q_mode mode, int64_t m, int64_t n, int64_t k)
{
    if (m <= kW8A8DecodeMaxM)
        return true;
    return mid_rows_decode_cheaper(mode, m, n, k, 1.0) &&
           fp8q::launch::plan_w8a16(m, n, k, act_type(mode)).workspace <= kMidRowsMaxWorkspace;
}

// group == 0: one weight scale per output row; else per-group scales
size_t linear_workspace(fp8q_mode mode, int64_t m, int64_t n, int64_t k, int64_t group)
{
    if (m <= 0 || n <= 0 || k < 1)
        return 0;
    if (group > 0) {
        if (!valid_group(group))
            return 0;
        if (grouped_uses_gemm(mode, m, n, k, group))
            return round_up(fp8q::launch::plan_w8a8(m, n, k).workspace, 256);
        return round_up(fp8q::launch::plan_w8a16_grouped(m, n, k, group, act_type(mode)).workspace,
                        256);
    }
    if (mode != FP8Q_W8A16 && mode != FP8Q_W8A16_F16 && mode != FP8Q_W8A8)
        return 0;
    if (rows_on_decode(mode, m, n, k))
        return round_up(fp8q::launch::plan_w8a16(m, n, k, act_type(mode)).workspace, 256);
    if (mode == FP8Q_W8A8)
        return round_up(fp8q::launch::plan_w8a8(m, n, k).workspace, 256);
    return 0;                       // the 16-bit prefill GEMM needs no scratch
}

fp8q_status linear_impl(fp8q_mode mode, const void *x, int64_t m, int64_t k, int64_t ld_x,
                        const float *x_scale, const uint8_t *w_fp8, int64_t n, int64_t ld_w,
                        const float *w_scale, int64_t group, uint16_t *y_bf16, int64_t ld_y,
                        void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (mode != FP8Q_W8A16 && mode != FP8Q_W8A8 && mode != FP8Q_W8A16_F16)
        return fail(FP8Q_ERR_INVALID_ARG, "unknown mode %d", (int)mode);
    const bool a16 = mode == FP8Q_W8A16 || mode == FP8Q_W8A16_F16;   // 16-bit activations
    if (m < 0 || n < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need m >= 0, n >= 0, k >= 1 (m=%lld, n=%lld, k=%lld)",
                    (long long)m, (long long)n, (long long)k);
    if (group != 0 && !valid_group(group))
        return fail(FP8Q_ERR_INVALID_ARG, "group must be 64, 128, 256 or 512 (got %lld)",
                    (long long)group);
    if (a16 && x_scale != nullptr)
        return fail(FP8Q_ERR_INVALID_ARG,
                    "fp8_w_bf16_a and fp8_w_fp16_a take no activation scale (x_scale must be NULL)");
    if (mode == FP8Q_W8A8 && x_scale == nullptr)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_w_fp8_a needs the activation scale (x_scale is NULL)");
    const size_t xelem = a16 ? 2 : 1;
    FP8Q_TRY(check_ld(ld_x, k, a16 ? 8 : 16, "ld_x"));
    FP8Q_TRY(check_ld(ld_w, k, 16, "ld_w"));
    FP8Q_TRY(check_ld(ld_y, n, 8, "ld_y"));
    if (!fp8q::launch::w8a16_supports_ld(ld_x, ld_w))
        return fail(FP8Q_ERR_INVALID_ARG, "ld_x and ld_w must be below 2^28 (got %lld, %lld)",
                    (long long)ld_x, (long long)ld_w);
    if (mode == FP8Q_W8A8 &&
        (!fp8q::launch::w8a8_supports_ld(ld_x) || !fp8q::launch::w8a8_supports_ld(ld_w)))
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_w_fp8_a needs ld_x and ld_w below 2^23 (got %lld, %lld)",
                    (long long)ld_x, (long long)ld_w);
    if (a16 && group == 0 && !rows_on_decode(mode, m, n, k) &&
        !fp8q::launch::w8a16_gemm_supports(ld_x, ld_w))
        return fail(FP8Q_ERR_INVALID_ARG,
                    "above 64 rows the 16-bit activation modes need ld_x below 2^22 and ld_w "
                    "below 2^23 (got %lld, %lld)", (long long)ld_x, (long long)ld_w);
    if ((a16 || group > 0) && (m + 63) / 64 > 65535)
        return fail(FP8Q_ERR_INVALID_ARG, "the decode kernels take at most 65535 * 64 rows");
    if (m == 0 || n == 0)
        return ok();
    const size_t need = linear_workspace(mode, m, n, k, group);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(FP8Q_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                    workspace == nullptr ? (size_t)0 : workspace_bytes, need);
    const size_t ex = extent(m, k, ld_x, xelem), ew = extent(n, k, ld_w, 1),
                 ey = extent(m, n, ld_y, 2);
    const size_t es = (size_t)n * 4 * (group > 0 ? (size_t)((k + group - 1) / group) : 1);
    if (overlap(y_bf16, ey, x, ex) || overlap(y_bf16, ey, w_fp8, ew) ||
        overlap(y_bf16, ey, w_scale, es) ||
        (x_scale != nullptr && overlap(y_bf16, ey, x_scale, 4)) ||
        (need > 0 && (overlap(workspace, need, y_bf16, ey) || overlap(workspace, need, x, ex) ||
                      overlap(workspace, need, w_fp8, ew) ||
                      overlap(workspace, need, w_scale, es) ||
                      (x_scale != nullptr && overlap(workspace, need, x_scale, 4)))))
        return fail(FP8Q_ERR_INVALID_ARG, "the output or workspace overlaps an input");
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    FP8Q_TRY(check_ptr(x, "x", dev, 16));
    FP8Q_TRY(check_ptr(w_fp8, "w_fp8", dev, 16));
    FP8Q_TRY(check_ptr(w_scale, "w_scale", dev, 4));
    FP8Q_TRY(check_ptr(y_bf16, "y_bf16", dev, 16));
    if (x_scale != nullptr)
        FP8Q_TRY(check_ptr(x_scale, "x_scale", dev, 4));
    if (need > 0)
        FP8Q_TRY(check_ptr(workspace, "workspace", dev, 16));
    if (group > 0)
        FP8Q_TRY(check_within_allocation(w_scale, es, "w_scale"));

    const int act = act_type(mode);
    hipError_t e;
    if (group > 0 && grouped_uses_gemm(mode, m, n, k, group)) {
        const auto plan = fp8q::launch::plan_w8a8(m, n, k);
        e = fp8q::launch::w8a8(plan, static_cast<const uint8_t *>(x), m, k, ld_x, x_scale, w_fp8,
                               n, ld_w, w_scale, y_bf16, ld_y, stream, group);
    } else if (group > 0) {
        const auto plan = fp8q::launch::plan_w8a16_grouped(m, n, k, group, act);
        e = fp8q::launch::w8a16(plan, act, x, m, k, ld_x, x_scale, w_fp8, n, ld_w, w_scale, y_bf16,
                                ld_y, workspace, stream);
    } else if (rows_on_decode(mode, m, n, k)) {
        const auto plan = fp8q::launch::plan_w8a16(m, n, k, act);
        e = fp8q::launch::w8a16(plan, act, x, m, k, ld_x, x_scale, w_fp8, n, ld_w, w_scale, y_bf16,
                                ld_y, workspace, stream);
    } else if (a16) {
        e = fp8q::launch::w8a16_gemm(mode == FP8Q_W8A16_F16, static_cast<const uint16_t *>(x), m, k,
                                     ld_x, w_fp8, n, ld_w, w_scale, y_bf16, ld_y, stream);
    } else {
        const auto plan = fp8q::launch::plan_w8a8(m, n, k);
        e = fp8q::launch::w8a8(plan, static_cast<const uint8_t *>(x), m, k, ld_x, x_scale, w_fp8,
                               n, ld_w, w_scale, y_bf16, ld_y, stream);
    }
    if (e != hipSuccess)
        return hip_fail(e, "linear launch");
    return ok();
}

}  // namespace

size_t fp8q_linear_workspace_size(fp8q_mode mode, int64_t m, int64_t n, int64_t k)
{
    return linear_workspace(mode, m, n, k, 0);
}

fp8q_status fp8q_linear(fp8q_mode mode,
                        const void *x, int64_t m, int64_t k, int64_t ld_x, const float *x_scale,
                        const uint8_t *w_fp8, int64_t n, int64_t ld_w, const float *w_scale,
                        uint16_t *y_bf16, int64_t ld_y,
                        void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return linear_impl(mode, x, m, k, ld_x, x_scale, w_fp8, n, ld_w, w_scale, 0, y_bf16, ld_y,
                       workspace, workspace_bytes, stream);
}

namespace {

// Up to this many rows fp8q_linear_w8a8_dynamic casts the activations inside
// the GEMM.  Every workgroup casts the activation rows it reads, and with 17..64
// rows each row is read by a whole column of 128-256 workgroups: one separate
// cast is then cheaper (measured on MI355X, Llama-3-8B q_proj in graphs: M = 32
// 36 us cast in the GEMM against 20 us for the quantizer + the GEMM on codes).
constexpr int64_t kDynamicFusedMaxM = 16;
// Up to this many activation values (64 KB of bf16) the panel kernel's
// workgroups each read the whole tensor for its maximum instead of taking the
// maxima of an absmax launch: an L2 read per workgroup against a launch.
constexpr int64_t kDynamicScanMaxElems = 32768;

bool dynamic_scans(const fp8q::launch::W8A16Plan &plan, int64_t m, int64_t k)
{
    return plan.kind == fp8q::launch::W8A16Plan::kPanel && m * k <= kDynamicScanMaxElems;
}

// Workspace of fp8q_linear_w8a8_dynamic: [0, 256) the scale slot (used when the
// caller passes no x_scale_out), then the absmax pass's maxima, then the
// decode plan's partial tiles (m <= 16), or the E4M3 codes [m, ldq] of the
// activations followed by the GEMM's scratch.
struct DynLayout {
    size_t part_off, part_bytes, rest_off, total, codes_bytes;
    int64_t ldq;
    bool fused;
};

DynLayout dyn_layout(int64_t m, int64_t n, int64_t k)
{
    DynLayout l{};
    l.part_off = 256;
    l.part_bytes = round_up((size_t)fp8q::launch::act_blocks(m, k) * sizeof(uint32_t), 256);
    l.rest_off = l.part_off + l.part_bytes;
    l.ldq = (k + 15) / 16 * 16;
    l.fused = m <= kDynamicFusedMaxM;
    size_t rest;
    if (l.fused) {
        rest = round_up(fp8q::launch::plan_w8a16(m, n, k, fp8q::launch::kW8A16ActQ).workspace, 256);
    } else {
        l.codes_bytes = round_up((size_t)m * (size_t)l.ldq, 256);
        rest = l.codes_bytes +
               round_up(rows_on_decode(FP8Q_W8A8, m, n, k)
                            ? fp8q::launch::plan_w8a16(m, n, k, fp8q::launch::kW8A16ActF8).workspace
                            : fp8q::launch::plan_w8a8(m, n, k).workspace,
                        256);
    }
    l.total = l.rest_off + rest;
    return l;
}

}  // namespace

size_t fp8q_linear_w8a8_dynamic_workspace_size(int64_t m, int64_t n, int64_t k)
{
    if (m <= 0 || n <= 0 || k < 1)
        return 0;
    return dyn_layout(m, n, k).total;
}

fp8q_status fp8q_linear_w8a8_dynamic(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                     const uint8_t *w_fp8, int64_t n, int64_t ld_w,
                                     const float *w_scale, uint16_t *y_bf16, int64_t ld_y,
                                     float *x_scale_out, void *workspace, size_t workspace_bytes,
                                     int32_t *nonfinite_flag, hipStream_t stream)
{
    if (m < 0 || n < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need m >= 0, n >= 0, k >= 1 (m=%lld, n=%lld, k=%lld)",
                    (long long)m, (long long)n, (long long)k);
    FP8Q_TRY(check_ld(ld_x, k, 8, "ld_x"));
    FP8Q_TRY(check_ld(ld_w, k, 16, "ld_w"));
    FP8Q_TRY(check_ld(ld_y, n, 8, "ld_y"));
    if (!fp8q::launch::w8a8_supports_ld(ld_w) || !fp8q::launch::w8a8_supports_ld((k + 15) / 16 * 16))
        return fail(FP8Q_ERR_INVALID_ARG, "ld_w and k must be below 2^23");
    if (m == 0 || n == 0)
        return ok();
    const DynLayout lay = dyn_layout(m, n, k);
    if (workspace == nullptr || workspace_bytes < lay.total)
        return fail(FP8Q_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                    workspace == nullptr ? (size_t)0 : workspace_bytes, lay.total);
    const size_t ex = extent(m, k, ld_x, 2), ew = extent(n, k, ld_w, 1), ey = extent(m, n, ld_y, 2),
                 es = (size_t)n * 4;
    const void *outs[4] = {y_bf16, workspace, x_scale_out, nonfinite_flag};
    const size_t olen[4] = {ey, lay.total, x_scale_out ? (size_t)4 : 0, nonfinite_flag ? (size_t)4 : 0};
    const void *ins[3] = {x_bf16, w_fp8, w_scale};
    const size_t ilen[3] = {ex, ew, es};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 3; ++b)
            if (overlap(outs[a], olen[a], ins[b], ilen[b]))
                return fail(FP8Q_ERR_INVALID_ARG, "an output or the workspace overlaps an input");
        for (int b = a + 1; b < 4; ++b)
            if (overlap(outs[a], olen[a], outs[b], olen[b]))
                return fail(FP8Q_ERR_INVALID_ARG,
                            "y, workspace, x_scale_out and nonfinite_flag must not overlap");
    }
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    FP8Q_TRY(check_ptr(x_bf16, "x_bf16", dev, 16));
    FP8Q_TRY(check_ptr(w_fp8, "w_fp8", dev, 16));
    FP8Q_TRY(check_ptr(w_scale, "w_scale", dev, 4));
    FP8Q_TRY(check_ptr(y_bf16, "y_bf16", dev, 16));
    FP8Q_TRY(check_ptr(workspace, "workspace", dev, 16));
    if (x_scale_out != nullptr)
        FP8Q_TRY(check_ptr(x_scale_out, "x_scale_out", dev, 4));
    if (nonfinite_flag != nullptr)
        FP8Q_TRY(check_ptr(nonfinite_flag, "nonfinite_flag", dev, 4));

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    float *scale = x_scale_out != nullptr ? x_scale_out : reinterpret_cast<float *>(ws);
    uint32_t *part = reinterpret_cast<uint32_t *>(ws + lay.part_off);
    void *rest = ws + lay.rest_off;
    hipError_t e;
    if (lay.fused) {
        const auto plan = fp8q::launch::plan_w8a16(m, n, k, fp8q::launch::kW8A16ActQ);
        if (dynamic_scans(plan, m, k)) {
            // one launch: every panel workgroup reads the whole (small) X for
            // its maximum
            e = fp8q::launch::w8a16_quant_act(plan, x_bf16, m, k, ld_x, nullptr, 0, scale,
                                              nonfinite_flag, w_fp8, n, ld_w, w_scale, y_bf16,
                                              ld_y, rest, stream);
        } else {
            e = fp8q::launch::act_amax(x_bf16, m, k, ld_x, part, stream);
            if (e == hipSuccess)
                e = fp8q::launch::w8a16_quant_act(plan, x_bf16, m, k, ld_x, part,
                                                  fp8q::launch::act_blocks(m, k), scale,
                                                  nonfinite_flag, w_fp8, n, ld_w, w_scale, y_bf16,
                                                  ld_y, rest, stream);
        }
    } else {
        uint8_t *codes = static_cast<uint8_t *>(rest);
        void *gemm_ws = static_cast<uint8_t *>(rest) + lay.codes_bytes;
        e = fp8q::launch::quantize_act(x_bf16, m, k, ld_x, codes, lay.ldq, scale, part,
                                       nonfinite_flag, stream);
        if (e == hipSuccess && rows_on_decode(FP8Q_W8A8, m, n, k))
            e = fp8q::launch::w8a16(fp8q::launch::plan_w8a16(m, n, k, fp8q::launch::kW8A16ActF8),
                                    fp8q::launch::kW8A16ActF8, codes, m, k, lay.ldq, scale, w_fp8,
                                    n, ld_w, w_scale, y_bf16, ld_y, gemm_ws, stream);
        else if (e == hipSuccess)
            e = fp8q::launch::w8a8(fp8q::launch::plan_w8a8(m, n, k), codes, m, k, lay.ldq, scale,
                                   w_fp8, n, ld_w, w_scale, y_bf16, ld_y, stream);
    }
    if (e != hipSuccess)
        return hip_fail(e, "dynamic W8A8 linear launch");
    return ok();
}

fp8q_status fp8q_linear_noalloc(fp8q_mode mode,
                                const void *x, int64_t m, int64_t k, int64_t ld_x,
                                const float *x_scale, const uint8_t *w_fp8, int64_t n,
                                int64_t ld_w, const float *w_scale,
                                uint16_t *y_bf16, int64_t ld_y, hipStream_t stream)
{
    if (m > 0 && n > 0 && k >= 1 && (mode == FP8Q_W8A16 || mode == FP8Q_W8A8 || mode == FP8Q_W8A16_F16)) {
        const size_t need = linear_workspace(mode, m, n, k, 0);
        if (need > fp8q::kNoallocScratchBytes)
            return fail(FP8Q_ERR_WORKSPACE,
                        "this shape needs %zu bytes of K-split scratch; the allocation-free "
                        "entry point has %zu (use fp8q_linear with a workspace)",
                        need, fp8q::kNoallocScratchBytes);
        if (need > 0) {
            int dev = 0;
            FP8Q_TRY(prepare(stream, &dev));
            void *scr = nullptr;
            hipError_t e = fp8q::launch::noalloc_scratch(dev, &scr);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return hip_fail(e, "resolving the device scratch (hipGetSymbolAddress)");
            }
            return linear_impl(mode, x, m, k, ld_x, x_scale, w_fp8, n, ld_w, w_scale, 0, y_bf16,
                               ld_y, scr, fp8q::kNoallocScratchBytes, stream);
        }
    }
    return linear_impl(mode, x, m, k, ld_x, x_scale, w_fp8, n, ld_w, w_scale, 0, y_bf16, ld_y,
                       nullptr, 0, stream);
}

size_t fp8q_linear_grouped_workspace_size(fp8q_mode mode, int64_t m, int64_t n, int64_t k,
                                          int64_t group)
{
    return valid_group(group) ? linear_workspace(mode, m, n, k, group) : 0;
}

fp8q_status fp8q_linear_grouped(fp8q_mode mode,
                                const void *x, int64_t m, int64_t k, int64_t ld_x,
                                const float *x_scale, const uint8_t *w_fp8, int64_t n,
                                int64_t ld_w, const float *w_scale, int64_t group,
                                uint16_t *y_bf16, int64_t ld_y,
                                void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!valid_group(group))
        return fail(FP8Q_ERR_INVALID_ARG, "group must be 64, 128, 256 or 512 (got %lld)",
                    (long long)group);
    return linear_impl(mode, x, m, k, ld_x, x_scale, w_fp8, n, ld_w, w_scale, group, y_bf16, ld_y,
                       workspace, workspace_bytes, stream);
}

fp8q_status fp8q_quantize_weight_grouped(const uint16_t *w_bf16, int64_t n, int64_t k,
                                         int64_t ld_w, int64_t group, uint8_t *w_fp8,
                                         int64_t ld_q, float *w_scale, int32_t *nonfinite_flag,
                                         hipStream_t stream)
{
    if (n < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "need n >= 0 and k >= 1 (n=%lld, k=%lld)", (long long)n,
                    (long long)k);
    if (!valid_group(group))
        return fail(FP8Q_ERR_INVALID_ARG, "group must be 64, 128, 256 or 512 (got %lld)",
                    (long long)group);
    FP8Q_TRY(check_ld(ld_w, k, 1, "ld_w"));
    FP8Q_TRY(check_ld(ld_q, k, 1, "ld_q"));
    if (n == 0)
        return ok();
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    FP8Q_TRY(check_ptr(w_bf16, "w_bf16", dev, 2));
    FP8Q_TRY(check_ptr(w_fp8, "w_fp8", dev, 1));
    FP8Q_TRY(check_ptr(w_scale, "w_scale", dev, 4));
    if (nonfinite_flag != nullptr)
        FP8Q_TRY(check_ptr(nonfinite_flag, "nonfinite_flag", dev, 4));
    const size_t ew = extent(n, k, ld_w, 2), eq = extent(n, k, ld_q, 1),
                 es = (size_t)n * (size_t)((k + group - 1) / group) * 4;
    FP8Q_TRY(check_within_allocation(w_scale, es, "w_scale"));
    if (overlap(w_fp8, eq, w_bf16, ew) || overlap(w_scale, es, w_bf16, ew) ||
        overlap(w_scale, es, w_fp8, eq))
        return fail(FP8Q_ERR_INVALID_ARG, "outputs overlap each other or the input");
    hipError_t e = fp8q::launch::quantize_weight_grouped(w_bf16, n, k, ld_w, group, w_fp8, ld_q,
                                                         w_scale, nonfinite_flag, stream);
    if (e != hipSuccess)
        return hip_fail(e, "grouped weight quantization launch");
    return ok();
}

fp8q_status fp8q_cast_f32_to_e4m3(const float *x, int64_t count, uint8_t *out, hipStream_t stream)
{
    if (count < 0)
        return fail(FP8Q_ERR_INVALID_ARG, "count < 0");
    if (count == 0)
        return ok();
    int dev = 0;
    FP8Q_TRY(prepare(stream, &dev));
    FP8Q_TRY(check_ptr(x, "x", dev, 16));
    FP8Q_TRY(check_ptr(out, "out", dev, 16));
    if (overlap(x, (size_t)count * 4, out, (size_t)count))
        return fail(FP8Q_ERR_INVALID_ARG, "out overlaps x");
    hipError_t e = fp8q::launch::cast_f32(x, count, out, stream);
    if (e != hipSuccess)
        return hip_fail(e, "cast launch");
    return ok();
}

}  // extern "C"

namespace {

void describe_w8a16(const fp8q::launch::W8A16Plan &p, char *buf, size_t len)
{
    char spg[16] = "";
    if (p.group > 0)
        std::snprintf(spg, sizeof spg, ", %lld", (long long)(p.group / 64));
    if (p.kind == fp8q::launch::W8A16Plan::kPanel)
        std::snprintf(buf, len,
                      "k_w8a16_panel<%d, %d, %d, %d, %d%s> grid=(%lld,%lld) block=%d staged_rows=%d "
                      "rows_per_workgroup=%d splits=1%s",
                      p.af, p.mb, p.steps, p.depth, p.waves, spg, (long long)p.grid_n,
                      (long long)p.grid_m, 64 * p.waves, p.xd, p.rpw > 0 ? p.rpw : 16 * p.mb,
                      p.group == 0 ? ""
                      : p.scale_stage == 2 ? " scales=preloaded" : " scales=per_chunk");
    else if (p.kind == fp8q::launch::W8A16Plan::kRows)
        std::snprintf(buf, len,
                      "k_w8a16_rows<%d, %d, %d, %d%s> rows=%d grid=(%lld,%lld,%lld) block=%d "
                      "kchunk=%lld splits=%lld%s",
                      p.af, p.mb, p.depth, p.waves, spg, p.rows, (long long)p.grid_n,
                      (long long)p.grid_m, (long long)p.splits, 64 * p.waves,
                      (long long)p.kchunk, (long long)p.splits,
                      p.splits > 1 ? " + k_w8a16_reduce" : "");
    else
        std::snprintf(buf, len,
                      "k_w8a16_tile<%d, %d, %d%s> grid=(%lld,%lld) block=256 splits=%lld kper=%lld%s",
                      p.mb, p.xd, p.steps, spg, (long long)p.grid_n, (long long)p.grid_m,
                      (long long)p.splits, (long long)p.kper,
                      p.splits > 1 ? " + k_w8a16_reduce" : "");
}

void describe_w8a8(int64_t m, int64_t n, int64_t k, bool grouped, char *buf, size_t len)
{
    const auto p = fp8q::launch::plan_w8a8(m, n, k);
    std::snprintf(buf, len, "k_w8a8%s tile=256x256x128 grid=%lld (%lldx%lld) block=512",
                  grouped ? "<true>" : "", (long long)(p.tiles_m * p.tiles_n),
                  (long long)p.tiles_m, (long long)p.tiles_n);
}

}  // namespace

extern "C" {

fp8q_status fp8q_linear_describe(fp8q_mode mode, int64_t m, int64_t n, int64_t k, char *buf,
                                 size_t len)
{
    if (buf == nullptr || len == 0)
        return fail(FP8Q_ERR_INVALID_ARG, "buf is NULL or empty");
    if (m < 0 || n < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "bad sizes");
    if (mode != FP8Q_W8A16 && mode != FP8Q_W8A16_F16 && mode != FP8Q_W8A8)
        return fail(FP8Q_ERR_INVALID_ARG, "unknown mode %d", (int)mode);
    if (rows_on_decode(mode, m, n, k))
        describe_w8a16(fp8q::launch::plan_w8a16(m, n, k, act_type(mode)), buf, len);
    else if (mode == FP8Q_W8A8)
        describe_w8a8(m, n, k, false, buf, len);
    else
        std::snprintf(buf, len, "k_w8a16_gemm<%s> tile=256x256x64 grid=%lld (%lldx%lld) block=512",
                      mode == FP8Q_W8A16_F16 ? "true" : "false",
                      (long long)(((m + 255) / 256) * ((n + 255) / 256)), (long long)((m + 255) / 256),
                      (long long)((n + 255) / 256));
    return ok();
}

fp8q_status fp8q_linear_w8a8_dynamic_describe(int64_t m, int64_t n, int64_t k, char *buf,
                                              size_t len)
{
    if (buf == nullptr || len == 0)
        return fail(FP8Q_ERR_INVALID_ARG, "buf is NULL or empty");
    if (m < 0 || n < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "bad sizes");
    if (!rows_on_decode(FP8Q_W8A8, m, n, k)) {
        char g[192];
        describe_w8a8(m, n, k, false, g, sizeof g);
        std::snprintf(buf, len, "k_act_amax + k_act_cast<0> + %s", g);
    } else if (m > kDynamicFusedMaxM) {
        char g[224];
        describe_w8a16(fp8q::launch::plan_w8a16(m, n, k, fp8q::launch::kW8A16ActF8), g, sizeof g);
        std::snprintf(buf, len, "k_act_amax + k_act_cast<0> + %s (E4M3 codes)", g);
    } else {
        char g[224];
        const auto plan = fp8q::launch::plan_w8a16(m, n, k, fp8q::launch::kW8A16ActQ);
        describe_w8a16(plan, g, sizeof g);
        if (dynamic_scans(plan, m, k))
            std::snprintf(buf, len, "%s (absmax and cast in the kernel)", g);
        else
            std::snprintf(buf, len, "k_act_amax + %s (activations cast in registers)", g);
    }
    return ok();
}

fp8q_status fp8q_linear_grouped_describe(fp8q_mode mode, int64_t m, int64_t n, int64_t k,
                                         int64_t group, char *buf, size_t len)
{
    if (buf == nullptr || len == 0)
        return fail(FP8Q_ERR_INVALID_ARG, "buf is NULL or empty");
    if (m < 0 || n < 0 || k < 1)
        return fail(FP8Q_ERR_INVALID_ARG, "bad sizes");
    if (mode != FP8Q_W8A16 && mode != FP8Q_W8A16_F16 && mode != FP8Q_W8A8)
        return fail(FP8Q_ERR_INVALID_ARG, "unknown mode %d", (int)mode);
    if (!valid_group(group))
        return fail(FP8Q_ERR_INVALID_ARG, "group must be 64, 128, 256 or 512 (got %lld)",
                    (long long)group);
    if (grouped_uses_gemm(mode, m, n, k, group))
        describe_w8a8(m, n, k, true, buf, len);
    else
        describe_w8a16(fp8q::launch::plan_w8a16_grouped(m, n, k, group, act_type(mode)), buf, len);
    return ok();
}

}  // extern "C"
