// W8A16 ("fp8_w_bf16_a", the write-up "Llama 3 精读" §3.1 step 3): E4M3
// weights with a per-output-channel scale, bf16 activations, bf16 output:
//   Y[m,n] = bf16_RNE( w_scale[n] * sum_k X[m,k] * dec(W[n,k]) ).
//
// This is the decode shape (a handful of tokens): the time is the weight
// stream from HBM (the deployment guide, "FP8量化与长上下文实测", §3.3: at
// batch 1 FP8 and BF16 are within 10% of each other because bandwidth is the
// limit).  Every weight byte is read exactly once.
//
// Both kernels widen the E4M3 codes to bf16 in registers (exact) and feed
// v_mfma_f32_16x16x32_bf16 with them as the A operand and the activations as
// B, fp32 accumulation.  The k order inside an MFMA is free as long as both
// operands use the same one, which lets one 16-byte weight load feed two
// MFMAs.  A lane streams 16 contiguous weight bytes per 64-k step with one
// non-temporal 16-byte load straight into registers; rows past N are clamped
// to a valid row and their outputs dropped, so every load is a plain
// unconditional dwordx4.  Nothing crosses workgroups inside a kernel: on
// MI355X the agent-scope release/acquire that would need (an L2 write-back
// and invalidate per workgroup) measured at 3-70 us per launch.
//
// k_w8a16_rows -- few activation rows on a small N.  A workgroup owns 4-32
//   weight rows and the whole K range; its waves split K and their fp32
//   partial tiles are summed through LDS in wave order.  Each wave loads its
//   own activation fragments straight into registers.
// k_w8a16_tile -- more activation rows, or an N large enough to fill the GPU
//   with 64-row tiles.  The 4 waves own 16 rows each and walk the same K
//   range, so the activations are staged once per workgroup through LDS (in
//   contiguous 1 KB row segments, double-buffered) and shared.  The
//   activation fragments the MFMA layout wants cover 16 rows x half a cache
//   line per load; fetched from L2 by every wave that way they cost about as
//   much as the weight stream itself at M = 12 and 3x more at M = 64.  When
//   N / 64 tiles cannot fill the GPU, K is split across workgroups: each
//   split writes an fp32 partial tile, and k_w8a16_reduce adds the splits in
//   split order (deterministic), scales and stores.
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "e4m3_div.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));


__device__ __forceinline__ v4u ldg_nt(const uint8_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
}

__device__ __forceinline__ v4u ldg(const void *p) { return *reinterpret_cast<const v4u *>(p); }

// 16 weight codes starting at k index kw of a row, zero past k.
__device__ __forceinline__ v4u load_w16_tail(const uint8_t *rowp, int64_t kw, int64_t k)
{
    uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        uint32_t b = (kw + e < k) ? (uint32_t)rowp[kw + e] : 0u;
        wd[e >> 2] |= b << (8 * (e & 3));
    }
    return v4u{wd[0], wd[1], wd[2], wd[3]};
}

// 8 bf16 activations starting at kx, zero past k.
__device__ __forceinline__ v4u load_x8_tail(const uint16_t *rowp, int64_t kx, int64_t k)
{
    uint32_t xd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t h = (kx + e < k) ? (uint32_t)rowp[kx + e] : 0u;
        xd[e >> 1] |= h << (16 * (e & 1));
    }
    return v4u{xd[0], xd[1], xd[2], xd[3]};
}

// s_waitcnt immediate for "at most n vector-memory loads outstanding" (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(N)); }

// Calls f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// The 16-bit activation types of the write-up's modes (§3.1 step 3):
// fp8_w_bf16_a and fp8_w_fp16_a.  Each gives the MFMA operand type, the
// exact widening of four E4M3 codes to it, the 16x16x32 MFMA and the RNE
// conversion of an fp32 output to the same 16-bit type.
// kActF8: E4M3 activations (fp8_w_fp8_a at decode sizes), widened exactly to
// bf16 and multiplied in bf16, bf16 output.
// kActQ: bf16 activations quantized per tensor as they are loaded (see
// QuantArgs below), then widened back to bf16 exactly for the MFMA.
enum { kActBF16 = 0, kActF16 = 1, kActF8 = 2, kActQ = 3 };
template <int AT> struct Act;

template <> struct Act<kActBF16> {
    typedef v8bf frag;
    static __device__ __forceinline__ frag cast(v4u v) { return __builtin_bit_cast(v8bf, v); }
    static __device__ __forceinline__ uint2 widen4(uint32_t codes) { return e4m3x4_to_bf16(codes); }
    static __device__ __forceinline__ v4f mfma(frag a, frag b, v4f c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
    static __device__ __forceinline__ uint16_t one(float v) { return (uint16_t)f32_to_bf16_rne(v); }
};

template <> struct Act<kActF16> {
    typedef v8h frag;
    static __device__ __forceinline__ frag cast(v4u v) { return __builtin_bit_cast(v8h, v); }
    // Four E4M3 codes -> four fp16 values (exact: E4M3 spans 2^-9 .. 448).
    static __device__ __forceinline__ uint2 widen4(uint32_t codes)
    {
        const v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, 1.0f, false);
        const v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, 1.0f, true);
        uint2 r;
        r.x = __builtin_bit_cast(uint32_t, lo);
        r.y = __builtin_bit_cast(uint32_t, hi);
        return r;
    }
    static __device__ __forceinline__ v4f mfma(frag a, frag b, v4f c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    // fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode)
    static __device__ __forceinline__ uint16_t one(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        return (uint32_t)one(lo) | ((uint32_t)one(hi) << 16);
    }
};

// The MFMA and output type used for an activation type.
template <int AT> constexpr int compute_type() { return AT == kActF8 || AT == kActQ ? kActBF16 : AT; }

// fp8_w_fp8_a with the dynamic per-tensor activation quantization folded into
// the GEMM (the deployment guide, "FP8量化与长上下文实测", §1.2 per-tensor
// activations and §3.1 scale formula).  An absmax pass over X left one
// maximum |x| key per block in part[0, npart).  Every workgroup folds them
// into s = max(fl32(amax / 448), 1e-12f), casts each activation it loads to
// E4M3 with E4M3Div (bit for bit the codes the per-tensor quantizer writes),
// and widens the codes back to bf16, which is exact; the epilogue multiplies
// by s * w_scale[n].  Workgroup (0, 0, 0) stores s to scale_out (read back by
// the K-split reduction) and raises *flag on a non-finite maximum.
struct QuantArgs {
    const uint32_t *part;
    int npart;
    float *scale_out;
    int32_t *flag;       // may be null
};

// Fold the absmax pass's maxima into the scale.  Contains __syncthreads: every
// thread of the workgroup calls it, at the start of the kernel.
__device__ __forceinline__ float fold_act_scale(const QuantArgs &qa)
{
    __shared__ uint32_t red[16];
    uint32_t key = 0;
    for (int j = threadIdx.x; j < qa.npart; j += blockDim.x)
        key = max(key, qa.part[j]);
    key = block_max_u32(key, red);
    const float s = scale_from_key(key);
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
        *qa.scale_out = s;
        if (qa.flag != nullptr && key >= 0x7F80u)
            *qa.flag = 1;
    }
    return s;
}

// The same scale from the activations themselves, for a tensor small enough
// that every workgroup reads all of it (at most a few tens of KB; the host
// passes no maxima then): the maximum is exact, so the scale is the same as
// from the absmax pass's maxima.  k is a multiple of 8 and the rows are
// 16-byte aligned.  Contains __syncthreads; called at the start of the
// kernel, before any direct load is in flight.
__device__ __forceinline__ float scan_act_scale(const uint16_t *x, int64_t m, int64_t k,
                                                int64_t ld_x, const QuantArgs &qa)
{
    __shared__ uint32_t red[16];
    uint32_t key = 0;
    const int cpr = (int)(k >> 3);
    const int chunks = (int)m * cpr;
    for (int i = threadIdx.x; i < chunks; i += blockDim.x) {
        const int row = i / cpr, c = i - row * cpr;
        key = max(key, key_max8(*reinterpret_cast<const uint4 *>(x + row * ld_x + 8 * c)));
    }
    key = block_max_u32(key, red);
    const float s = scale_from_key(key);
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
        *qa.scale_out = s;
        if (qa.flag != nullptr && key >= 0x7F80u)
            *qa.flag = 1;
    }
    return s;
}

// The scale the epilogue applies for activation type AT: 1 for 16-bit
// activations, *x_scale for E4M3 codes, the folded per-tensor scale for kActQ.
template <int AT>
__device__ __forceinline__ float act_scale(const float *x_scale, const QuantArgs &qa)
{
    if constexpr (AT == kActF8)
        return *x_scale;
    else if constexpr (AT == kActQ)
        return fold_act_scale(qa);
    else
        return 1.0f;
}

// Eight bf16 activations -> their E4M3 codes under div -> the codes' values
// as eight bf16 (exact), in the same order.
__device__ __forceinline__ v4u qdq8(v4u v, const E4M3Div &div)
{
    const uint2 c = div.codes8(uint4{v.x, v.y, v.z, v.w});
    const uint2 lo = e4m3x4_to_bf16(c.x), hi = e4m3x4_to_bf16(c.y);
    return v4u{lo.x, lo.y, hi.x, hi.y};
}

// Widen a lane's 16 weight codes into the A operands of two MFMA k-steps.
template <int AT>
__device__ __forceinline__ void widen(v4u wv, typename Act<AT>::frag &a0, typename Act<AT>::frag &a1)
{
    uint2 p0 = Act<AT>::widen4(wv.x), p1 = Act<AT>::widen4(wv.y);
    uint2 p2 = Act<AT>::widen4(wv.z), p3 = Act<AT>::widen4(wv.w);
    a0 = Act<AT>::cast(v4u{p0.x, p0.y, p1.x, p1.y});
    a1 = Act<AT>::cast(v4u{p2.x, p2.y, p3.x, p3.y});
}

// One 64-k step of a wave: widen the weight codes and issue the MFMAs.
// Rows past N (weights) or past M (activations) were clamped to a valid row
// when loading; they only feed output rows/columns that are never stored, so
// no masking is needed here.
// xv holds, per activation group, either 16 activation codes in xv[j][0]
// (E4M3) or two 8-value halves in xv[j][0..1] (16-bit types).
// SWAP puts the activations in the A operand and the weights in B, so each
// lane's 4 accumulators are 4 activation rows of one weight row (one output
// column) instead of 4 weight rows of one activation row.
template <int AF, int MB, int AT, bool SWAP = false>
__device__ __forceinline__ void step_mfma(const v4u (&wv)[AF], const v4u (&xv)[MB][2],
                                          v4f (&acc)[AF][MB], const E4M3Div &div)
{
    constexpr int CT = compute_type<AT>();
    typename Act<CT>::frag b[MB][2];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        if constexpr (AT == kActF8) {
            widen<CT>(xv[j][0], b[j][0], b[j][1]);
        } else if constexpr (AT == kActQ) {
            b[j][0] = Act<CT>::cast(qdq8(xv[j][0], div));
            b[j][1] = Act<CT>::cast(qdq8(xv[j][1], div));
        } else {
            b[j][0] = Act<CT>::cast(xv[j][0]);
            b[j][1] = Act<CT>::cast(xv[j][1]);
        }
    }
#pragma unroll
    for (int a = 0; a < AF; ++a) {
        typename Act<CT>::frag a0, a1;
        widen<CT>(wv[a], a0, a1);
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            if constexpr (SWAP) {
                acc[a][j] = Act<CT>::mfma(b[j][0], a0, acc[a][j]);
                acc[a][j] = Act<CT>::mfma(b[j][1], a1, acc[a][j]);
            } else {
                acc[a][j] = Act<CT>::mfma(a0, b[j][0], acc[a][j]);
                acc[a][j] = Act<CT>::mfma(a1, b[j][1], acc[a][j]);
            }
        }
    }
}

// AF: A fragments (16-row groups) per wave, so a block owns up to 16*AF rows;
// `rows` (<= 16*AF) is how many of them are real weight rows.
// MB: 16-column groups of activations (M <= 16*MB per block along grid.y).
// P:  pipeline depth -- 64-k steps whose loads are in flight while a step's
//     MFMAs run.  The pipelined span of a wave is a multiple of P steps; the
//     remaining steps (and a partial step at the end of K) run one by one.
// NW: waves per workgroup; wave w owns K range [w*kchunk, (w+1)*kchunk).
// AT: activation type (kActBF16, kActF16 or kActF8); x is then [m, ld_x]
// 16-bit values or E4M3 codes, and x_scale (E4M3 only) the activation scale.
// SPG: 0 for one scale per weight row; else per-group scales w_scale [n,
//     ngroups] for groups of 64*SPG k (the deployment guide §4.3), as in
//     k_w8a16_tile: the MFMA operands are swapped so a lane's accumulators
//     belong to one weight row, each group's sum is multiplied by its scale
//     as the group ends, and wave K ranges start on group boundaries (the
//     plan makes kchunk a multiple of 512, so each P = 8 round of 512 k is a
//     whole number of groups and the folds sit at fixed steps).  A group's
//     scale for the next round is loaded right after this round folds it.
template <int AF, int MB, int P, int NW, int AT, int SPG = 0>
__global__ __launch_bounds__(NW * kWave) void k_w8a16_rows(
    const void *__restrict__ xv, int64_t m, int64_t k, int64_t ld_x,
    const float *__restrict__ x_scale,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int rows, int64_t kchunk, int64_t kper, float *__restrict__ partial, int64_t ldp,
    int64_t ngroups, QuantArgs qa)
{
    constexpr bool GS = SPG > 0;
    constexpr int SPGD = GS ? SPG : 1;         // SPG as a divisor
    constexpr int GK = 64 * SPGD;              // k per scale group
    constexpr int GR = GS ? P / SPGD : 1;      // scale groups per pipelined round
    static_assert(!GS || P % SPGD == 0, "a round is a whole number of scale groups");
    constexpr bool F8 = AT == kActF8;
    constexpr int CT = compute_type<AT>();
    constexpr int ES = F8 ? 1 : 2;              // bytes per activation value
    constexpr int XS = F8 ? 1 : 2;              // activation loads per group per step
    constexpr int L = AF + XS * MB;             // loads per step
    __shared__ v4f red[NW][AF * MB][kWave];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int r = lane & 15;          // row of the A (weight) / B (activation) operand
    const int g = lane >> 4;          // which 16 k-values of a 64-k step this lane holds
    const int64_t n0 = (int64_t)blockIdx.x * rows;
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MB;
    // grid.z splits K into ranges of kper (a multiple of 64); within the
    // range the waves take kchunk each
    const int split = (int)blockIdx.z;
    const int64_t k_lo = (int64_t)split * kper;
    const int64_t k_hi = min(k, k_lo + kper);
    const int64_t kb = min(k_hi, k_lo + (int64_t)wave * kchunk);
    const int64_t ke = min(k_hi, kb + kchunk);

    const uint8_t *wp[AF];
#pragma unroll
    for (int a = 0; a < AF; ++a) {
        const int lr = 16 * a + r;
        const bool ok = lr < rows && n0 + lr < n;
        wp[a] = w + (ok ? n0 + lr : n0) * ld_w + 16 * g;
    }
    // byte pointers to this lane's 16 activation values of each group
    const uint8_t *xp[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const int64_t xr = m0 + 16 * j + r;
        xp[j] = static_cast<const uint8_t *>(xv) + ((xr < m ? xr : m0) * ld_x + 16 * g) * ES;
    }
    const float xs = act_scale<AT>(x_scale, qa);
    const E4M3Div div(AT == kActQ ? xs : 1.0f, true);

    v4f acc[2][AF][MB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int a = 0; a < AF; ++a)
#pragma unroll
            for (int j = 0; j < MB; ++j)
                acc[h][a][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // grouped: this lane's weight row of fragment a is its output column
    const float *srow[AF];
    v4f tot[AF][MB];
    float sc[GR][AF];
#pragma unroll
    for (int a = 0; a < AF; ++a) {
        srow[a] = w_scale + (GS ? min(n0 + min(16 * a + r, rows - 1), n - 1) * ngroups : 0);
#pragma unroll
        for (int j = 0; j < MB; ++j)
            tot[a][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    // close a scale group: each fragment's sum, times its row's scale
    auto fold = [&](const float (&s)[AF]) {
#pragma unroll
        for (int a = 0; a < AF; ++a)
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                tot[a][j] += s[a] * (acc[0][a][j] + acc[1][a][j]);
                acc[0][a][j] = v4f{0.f, 0.f, 0.f, 0.f};
                acc[1][a][j] = v4f{0.f, 0.f, 0.f, 0.f};
            }
    };
    auto load_sc = [&](int gi, int64_t k0) {      // group gi of the round starting at k0
#pragma unroll
        for (int a = 0; a < AF; ++a)
            sc[gi][a] = srow[a][(k0 + (int64_t)GK * gi) / GK];
    };

    const int64_t nfull = (ke - kb) / 64;          // whole 64-k steps
    const int64_t npipe = nfull - nfull % P;       // pipelined span
    int64_t kk = kb;
    if (npipe > 0) {
        v4u wb[P][AF];
        v4u xb[P][MB][2];
        auto issue = [&](int u, int64_t k0) {
#pragma unroll
            for (int a = 0; a < AF; ++a)
                wb[u][a] = ldg_nt(wp[a] + k0);
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                xb[u][j][0] = ldg(xp[j] + k0 * ES);
                if constexpr (!F8)
                    xb[u][j][1] = ldg(xp[j] + k0 * ES + 16);
            }
        };
        const int64_t kend = kb + 64 * npipe;
        if constexpr (GS) {
#pragma unroll
            for (int gi = 0; gi < GR; ++gi)
                load_sc(gi, kb);
        }
#pragma unroll
        for (int u = 0; u < P; ++u)
            issue(u, kb + 64 * u);
        __builtin_amdgcn_sched_barrier(0);
        for (; kk + 64 * P < kend; kk += 64 * P) {
            static_for<0, P>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                // loads retire in order: with (P-1) steps' loads still in
                // flight, step u's loads have landed (a scale load issued among
                // them only makes this wait for more)
                wait_vmcnt<(P - 1) * L>();
                __builtin_amdgcn_sched_barrier(0);
                step_mfma<AF, MB, AT, GS>(wb[u], xb[u], acc[u & 1], div);
                issue(u, kk + 64 * (P + u));
                if constexpr (GS && (u + 1) % SPGD == 0) {
                    fold(sc[u / SPGD]);
                    load_sc(u / SPGD, kk + 64 * P);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        // last pipelined round: no more loads to issue
        static_for<0, P>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            wait_vmcnt<(P - 1 - u) * L>();
            __builtin_amdgcn_sched_barrier(0);
            step_mfma<AF, MB, AT, GS>(wb[u], xb[u], acc[u & 1], div);
            if constexpr (GS && (u + 1) % SPGD == 0)
                fold(sc[u / SPGD]);
        });
        kk = kend;
    }
    // remaining steps one at a time; the last one may be partial (masked at k).
    // They start on a group boundary; a group's scale is read at its first
    // step and applied after its last (or at the end of the wave's range).
    float s_tail[AF];
    for (; kk < ke; kk += 64) {
        if constexpr (GS) {
            if ((kk - kb) % GK == 0) {
#pragma unroll
                for (int a = 0; a < AF; ++a)
                    s_tail[a] = srow[a][kk / GK];
            }
        }
        const int64_t kw = kk + 16 * g;
        v4u wv[AF];
        v4u xv[MB][2];
        if (kk + 64 <= k) {
#pragma unroll
            for (int a = 0; a < AF; ++a)
                wv[a] = ldg(wp[a] + kk);
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                xv[j][0] = ldg(xp[j] + kk * ES);
                if constexpr (!F8)
                    xv[j][1] = ldg(xp[j] + kk * ES + 16);
            }
        } else {
#pragma unroll
            for (int a = 0; a < AF; ++a)
                wv[a] = kw < k ? load_w16_tail(wp[a] - 16 * g, kw, k) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                const uint8_t *row0 = xp[j] - 16 * g * ES;     // the row's first value
                if constexpr (F8) {
                    xv[j][0] = kw < k ? load_w16_tail(row0, kw, k) : v4u{0u, 0u, 0u, 0u};
                } else {
                    const uint16_t *row16 = reinterpret_cast<const uint16_t *>(row0);
                    xv[j][0] = kw < k ? load_x8_tail(row16, kw, k) : v4u{0u, 0u, 0u, 0u};
                    xv[j][1] = kw + 8 < k ? load_x8_tail(row16, kw + 8, k) : v4u{0u, 0u, 0u, 0u};
                }
            }
        }
        step_mfma<AF, MB, AT, GS>(wv, xv, acc[0], div);
        if constexpr (GS) {
            if ((kk + 64 - kb) % GK == 0 || kk + 64 >= ke)
                fold(s_tail);
        }
    }

    // ---- sum the waves' partial tiles in wave order, then scale and store --
#pragma unroll
    for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int j = 0; j < MB; ++j)
            red[wave][a * MB + j][lane] = GS ? tot[a][j] : acc[0][a][j] + acc[1][a][j];
    __syncthreads();

    if constexpr (GS) {
        // lane slot sl holds D rows 4 * (sl >> 4) + v (activation rows) of
        // column sl & 15 (weight row 16a + (sl & 15)); group scales are applied
        for (int slot = threadIdx.x; slot < AF * MB * kWave; slot += blockDim.x) {
            const int f = slot / kWave;
            const int sl = slot % kWave;
            const int a = f / MB;
            const int j = f % MB;
            const int nl = 16 * a + (sl & 15);
            const int64_t nc = n0 + nl;
            if (nl >= rows || nc >= n)
                continue;
            v4f sum = red[0][f][sl];
            for (int wv = 1; wv < NW; ++wv)
                sum += red[wv][f][sl];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t mr = m0 + 16 * j + 4 * (sl >> 4) + v;
                if (mr >= m)
                    continue;
                if (gridDim.z > 1)
                    partial[((int64_t)split * m + mr) * ldp + nc] = sum[v];
                else
                    y[mr * ld_y + nc] = Act<CT>::one(sum[v] * xs);
            }
        }
        return;
    }

    // one thread per (fragment, lane) slot: 4 outputs of one row of Y
    for (int slot = threadIdx.x; slot < AF * MB * kWave; slot += blockDim.x) {
        const int f = slot / kWave;
        const int sl = slot % kWave;
        const int a = f / MB;
        const int j = f % MB;
        const int64_t mr = m0 + 16 * j + (sl & 15);
        const int nl = 16 * a + 4 * (sl >> 4);     // D rows 4g..4g+3 of this fragment
        const int64_t nb = n0 + nl;
        if (mr >= m || nl >= rows || nb >= n)
            continue;
        v4f sum = red[0][f][sl];
        for (int wv = 1; wv < NW; ++wv)
            sum += red[wv][f][sl];
        if (gridDim.z > 1) {
            // K split across workgroups: partial[split][m][ldp] (ldp >= n
            // rounded up to 4, so the 16 bytes fit); k_w8a16_reduce finishes
            *reinterpret_cast<v4f *>(partial + ((int64_t)split * m + mr) * ldp + nb) = sum;
            continue;
        }
        uint16_t *yp = y + mr * ld_y + nb;
        const int valid = (int)min<int64_t>(min<int64_t>(4, rows - nl), n - nb);
        if (valid == 4) {
            uint2 o;
            o.x = Act<CT>::pack2(sum[0] * (xs * w_scale[nb]), sum[1] * (xs * w_scale[nb + 1]));
            o.y = Act<CT>::pack2(sum[2] * (xs * w_scale[nb + 2]), sum[3] * (xs * w_scale[nb + 3]));
            *reinterpret_cast<uint2 *>(yp) = o;
        } else {
            for (int v = 0; v < valid; ++v)
                yp[v] = Act<CT>::one(sum[v] * (xs * w_scale[nb + v]));
        }
    }
}


// ---------------------------------------------------------------------------
// k_w8a16_tile
// ---------------------------------------------------------------------------

constexpr int kTileThreads = 256;              // 4 waves
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kTileN = 16 * kTileWaves;        // weight rows per workgroup

// Workgroup barrier after this wave's LDS writes have landed.  Written out
// because __syncthreads() also waits for every outstanding global load,
// which would drain the weight pipeline at each chunk boundary.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Scale 4 consecutive outputs of row mr and store them as bf16 (8 bytes when
// all 4 columns exist; the pointer is then 8-byte aligned).
// (xs: the activation scale of E4M3 activations, 1 otherwise -- 1 * w is
// exact, so the 16-bit modes round exactly as without it.)
template <int CT>
__device__ __forceinline__ void store_y4(uint16_t *__restrict__ y, int64_t ld_y,
                                         const float *__restrict__ w_scale, float xs, int64_t mr,
                                         int64_t nb, int64_t n, v4f s)
{
    uint16_t *yp = y + mr * ld_y + nb;
    // no w_scale: the group scales were applied inside the K loop
    auto ws = [&](int v) { return w_scale != nullptr ? w_scale[nb + v] : 1.0f; };
    if (nb + 4 <= n) {
        uint2 o;
        o.x = Act<CT>::pack2(s[0] * (xs * ws(0)), s[1] * (xs * ws(1)));
        o.y = Act<CT>::pack2(s[2] * (xs * ws(2)), s[3] * (xs * ws(3)));
        *reinterpret_cast<uint2 *>(yp) = o;
    } else {
        for (int v = 0; v < (int)(n - nb); ++v)
            yp[v] = Act<CT>::one(s[v] * (xs * ws(v)));
    }
}

// MB: 16-row groups of activations per workgroup (M <= 16*MB along grid.y).
// XD: activation rows each wave stages per chunk (4*XD rows are staged; rows
//     past M are clamped to row M-1; LDS rows past 4*XD are never written and
//     only feed output columns that are never stored).
// T:  64-k steps per chunk; a chunk's weights are loaded one chunk ahead.
// SPG: 0 for one scale per weight row (w_scale [n]); else per-group weight
//     scales, w_scale [n, ngroups] for groups of 64*SPG k (the deployment
//     guide §4.3): each group's products are summed on their own, multiplied
//     by the group's scale at the group's end and added to the row's total.
//     The MFMA operands are then swapped (activations in A, weights in B), so
//     every lane's accumulators belong to one weight row and one scale.
// Grid: x = tiles of 64 weight rows times K splits (split index fastest),
// y = groups of 16*MB activation rows.
template <int MB, int XD, int T, int AT, int SPG>
__global__ __launch_bounds__(kTileThreads) void k_w8a16_tile(
    const void *__restrict__ xv, int64_t m, int64_t k, int64_t ld_x,
    const float *__restrict__ x_scale,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int64_t kper, int splits, float *__restrict__ partial, int64_t ldp, int64_t ngroups,
    QuantArgs qa)
{
    constexpr bool GS = SPG > 0;
    constexpr int GK = 64 * (GS ? SPG : 1);    // k per scale group
    constexpr int SPGD = GS ? SPG : 1;         // SPG as a divisor
    constexpr int SC = GS ? T / SPGD : 0;      // scale groups per chunk
    // a chunk's scales are adjacent floats, which the compiler may merge into
    // fewer load instructions: the waits below count them as at least one
    // (a smaller count only waits for more)
    constexpr int SCL = GS ? 1 : 0;
    static_assert(!GS || T % SPG == 0, "a chunk is a whole number of scale groups");
    constexpr int XR = 16 * MB;                // LDS rows per buffer
    constexpr int CK = 64 * T;                 // k per chunk
    constexpr int RB = 2 * CK;                 // LDS bytes of one staged row
    constexpr int XH = T / 8;                  // 1 KB loads per staged row
    constexpr int XL = XD * XH;                // activation loads per wave per chunk
    static_assert(kTileWaves * XD <= XR, "staged rows exceed the buffer");
    static_assert(T % 8 == 0, "a chunk is a whole number of 1 KB row segments");
    constexpr bool F8 = AT == kActF8;
    constexpr int CT = compute_type<AT>();
    constexpr int ES = F8 ? 1 : 2;             // bytes per activation value
    // staged rows are always 16-bit (E4M3 activations are widened to bf16,
    // exactly, between their load and the LDS write)
    typedef typename std::conditional<F8, uint2, v4u>::type XReg;
    const uint8_t *x8 = static_cast<const uint8_t *>(xv);
    const float xs = act_scale<AT>(x_scale, qa);
    const E4M3Div div(AT == kActQ ? xs : 1.0f, true);
    __shared__ __attribute__((aligned(16))) uint8_t xlds[2 * XR * RB];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int r = lane & 15;          // row of the A (weight) / B (activation) operand
    const int g = lane >> 4;          // which 16 k-values of a 64-k step this lane holds
    const int split = (int)(blockIdx.x % (unsigned)splits);
    const int64_t tile_n = blockIdx.x / (unsigned)splits;
    const int64_t n0 = tile_n * kTileN + 16 * wave;    // this wave's first weight row
    const int64_t m0 = (int64_t)blockIdx.y * XR;
    const int64_t kb = (int64_t)split * kper;
    const int64_t ke = min(k, kb + kper);
    const int64_t nchunks = (ke - kb) / CK;

    const uint8_t *wrow = w + min(n0 + r, n - 1) * ld_w + 16 * g;
    const uint8_t *wp = wrow + kb;
    // grouped: this lane's weight row is its output column; its group scales
    const float *srow = w_scale + (GS ? min(n0 + r, n - 1) * ngroups : 0);
    v4f tot[MB];
    float sc_cur[SC > 0 ? SC : 1], sc_nxt[SC > 0 ? SC : 1];
#pragma unroll
    for (int j = 0; j < MB; ++j)
        tot[j] = v4f{0.f, 0.f, 0.f, 0.f};
    // scales of chunk c's groups (chunks start on group boundaries: kb and CK
    // are multiples of GK)
    auto load_sc = [&](int64_t c) {
#pragma unroll
        for (int i = 0; i < SC; ++i)
            sc_nxt[i] = srow[(kb + c * CK) / GK + i];
    };

    // LDS byte offset of 16-byte unit u of staged row rho.  The units of a row
    // are XOR-permuted by the row's low 4 bits, so the 16 rows one B-operand
    // read touches (same u) land in 16 different 4-bank groups.
    auto xs_off = [](int rho, int u) { return rho * RB + 16 * (u ^ (rho & 15)); };

    v4f acc[2][MB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < MB; ++j)
            acc[h][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // close a scale group: its sum, times its scale, joins the total
    auto fold = [&](float s) {
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            tot[j] += s * (acc[0][j] + acc[1][j]);
            acc[0][j] = v4f{0.f, 0.f, 0.f, 0.f};
            acc[1][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    };

    if (nchunks > 0) {
        // this wave stages activation rows wave, wave + 4, ...; lane l holds
        // 16-byte unit l of each 1 KB segment of the row's chunk
        const uint8_t *xsrc[XD];
#pragma unroll
        for (int i = 0; i < XD; ++i)
            xsrc[i] = x8 + (min(m0 + wave + kTileWaves * i, m - 1) * ld_x + kb + 8 * lane) * ES;
        XReg xr[XD][XH];
        v4u wr[T];
        auto load_x = [&](int64_t c) {
#pragma unroll
            for (int i = 0; i < XD; ++i)
#pragma unroll
                for (int h = 0; h < XH; ++h)
                    xr[i][h] = *reinterpret_cast<const XReg *>(xsrc[i] + (c * CK + 512 * h) * ES);
        };
        auto store_x = [&](int buf) {
            uint8_t *base = xlds + buf * (XR * RB);
#pragma unroll
            for (int i = 0; i < XD; ++i)
#pragma unroll
                for (int h = 0; h < XH; ++h)
                {
                    v4u v;
                    if constexpr (F8) {
                        const uint2 lo = Act<CT>::widen4(xr[i][h].x), hi = Act<CT>::widen4(xr[i][h].y);
                        v = v4u{lo.x, lo.y, hi.x, hi.y};
                    } else if constexpr (AT == kActQ) {
                        v = qdq8(xr[i][h], div);
                    } else {
                        v = xr[i][h];
                    }
                    *reinterpret_cast<v4u *>(base + xs_off(wave + kTileWaves * i, 64 * h + lane)) = v;
                }
        };
        auto compute = [&](int u, int buf, v4f(&a)[MB]) {
            typename Act<CT>::frag a0, a1;
            widen<CT>(wr[u], a0, a1);
            const uint8_t *base = xlds + buf * (XR * RB);
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                const v4u b0 = *reinterpret_cast<const v4u *>(base + xs_off(16 * j + r, 8 * u + 2 * g));
                const v4u b1 = *reinterpret_cast<const v4u *>(base + xs_off(16 * j + r, 8 * u + 2 * g + 1));
                if constexpr (GS) {
                    a[j] = Act<CT>::mfma(Act<CT>::cast(b0), a0, a[j]);
                    a[j] = Act<CT>::mfma(Act<CT>::cast(b1), a1, a[j]);
                } else {
                    a[j] = Act<CT>::mfma(a0, Act<CT>::cast(b0), a[j]);
                    a[j] = Act<CT>::mfma(a1, Act<CT>::cast(b1), a[j]);
                }
            }
        };

        // prologue: chunk 0's scales and activations, then its weights
        if constexpr (GS)
            load_sc(0);
        load_x(0);
        static_for<0, T>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            wr[u] = ldg_nt(wp + 64 * u);
        });
        wait_vmcnt<T>();                      // the scale and activation loads (issued first) landed
        __builtin_amdgcn_sched_barrier(0);
        store_x(0);
        if constexpr (GS) {
#pragma unroll
            for (int i = 0; i < SC; ++i)
                sc_cur[i] = sc_nxt[i];
        }
        lds_barrier();

        int64_t c = 0;
        for (; c + 1 < nchunks; ++c) {
            const int buf = (int)(c & 1);
            if constexpr (GS)
                load_sc(c + 1);
            load_x(c + 1);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, T>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                // loads retire in order; issued after this step's weights:
                // T-1 weight loads and the scale and XL activation loads of
                // chunk c+1
                wait_vmcnt<T - 1 + XL + SCL>();
                __builtin_amdgcn_sched_barrier(0);
                compute(u, buf, acc[u & 1]);
                wr[u] = ldg_nt(wp + (c + 1) * CK + 64 * u);
                if constexpr (GS && (u + 1) % SPGD == 0)
                    fold(sc_cur[u / SPGD]);
                __builtin_amdgcn_sched_barrier(0);
            });
            // chunk c+1's scales and activations: only its T weight loads were
            // issued after them
            wait_vmcnt<T>();
            __builtin_amdgcn_sched_barrier(0);
            store_x(buf ^ 1);     // that buffer was last read in chunk c-1, before the
            if constexpr (GS) {   // previous barrier
#pragma unroll
                for (int i = 0; i < SC; ++i)
                    sc_cur[i] = sc_nxt[i];
            }
            lds_barrier();
        }
        // last chunk: nothing more to load
        static_for<0, T>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            wait_vmcnt<T - 1 - u>();
            __builtin_amdgcn_sched_barrier(0);
            compute(u, (int)(c & 1), acc[u & 1]);
            if constexpr (GS && (u + 1) % SPGD == 0)
                fold(sc_cur[u / SPGD]);
        });
    }

    // K left after the whole chunks (less than one chunk, only in the last
    // split): one 64-k step at a time straight from global memory, the last
    // step masked at k.  It starts on a group boundary; a group's scale is
    // read at its first step and applied after its last (or K's end).
    float s_tail = 0.f;
    for (int64_t kk = kb + nchunks * CK; kk < ke; kk += 64) {
        if constexpr (GS) {
            if ((kk - kb) % GK == 0)
                s_tail = srow[kk / GK];
        }
        const int64_t kw = kk + 16 * g;
        v4u wv;
        v4u xv[MB][2];
        if (kk + 64 <= k) {
            wv = ldg(wrow + kk);
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                const uint8_t *xrow = x8 + (min(m0 + 16 * j + r, m - 1) * ld_x + kw) * ES;
                xv[j][0] = ldg(xrow);
                if constexpr (!F8)
                    xv[j][1] = ldg(xrow + 16);
            }
        } else {
            wv = kw < k ? load_w16_tail(wrow - 16 * g, kw, k) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                const uint8_t *xrow = x8 + min(m0 + 16 * j + r, m - 1) * ld_x * ES;
                if constexpr (F8) {
                    xv[j][0] = kw < k ? load_w16_tail(xrow, kw, k) : v4u{0u, 0u, 0u, 0u};
                } else {
                    const uint16_t *row16 = reinterpret_cast<const uint16_t *>(xrow);
                    xv[j][0] = kw < k ? load_x8_tail(row16, kw, k) : v4u{0u, 0u, 0u, 0u};
                    xv[j][1] = kw + 8 < k ? load_x8_tail(row16, kw + 8, k) : v4u{0u, 0u, 0u, 0u};
                }
            }
        }
        v4u wv1[1] = {wv};
        v4f acc1[1][MB];
#pragma unroll
        for (int j = 0; j < MB; ++j)
            acc1[0][j] = acc[0][j];
        step_mfma<1, MB, AT, GS>(wv1, xv, acc1, div);
#pragma unroll
        for (int j = 0; j < MB; ++j)
            acc[0][j] = acc1[0][j];
        if constexpr (GS) {
            if ((kk + 64 - kb) % GK == 0 || kk + 64 >= ke)
                fold(s_tail);
        }
    }

    if constexpr (GS) {
        // lane (r, g) holds D rows 4g..4g+3 (activation rows m0 + 16j + 4g..)
        // of column r (weight row n0 + r); every group is folded into tot
        const int64_t nc = n0 + r;
#pragma unroll
        for (int j = 0; j < MB; ++j) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t mr = m0 + 16 * j + 4 * g + v;
                if (mr >= m || nc >= n)
                    continue;
                if (splits == 1)
                    y[mr * ld_y + nc] = Act<CT>::one(tot[j][v] * xs);
                else
                    partial[((int64_t)split * m + mr) * ldp + nc] = tot[j][v];
            }
        }
        return;
    }

    // lane (r, g) holds D rows 4g..4g+3 (weight rows n0+4g..) of column r
    // (activation row m0 + 16j + r)
    const int64_t nb = n0 + 4 * g;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const int64_t mr = m0 + 16 * j + r;
        if (mr >= m || nb >= n)
            continue;
        const v4f s = acc[0][j] + acc[1][j];
        if (splits == 1)
            store_y4<CT>(y, ld_y, w_scale, xs, mr, nb, n, s);
        else      // partial[split][m][ldp]; ldp >= n rounded up to 4, so the 16 bytes fit
            *reinterpret_cast<v4f *>(partial + ((int64_t)split * m + mr) * ldp + nb) = s;
    }
}

// ---------------------------------------------------------------------------
// k_w8a16_panel
// ---------------------------------------------------------------------------
//
// One workgroup per output panel of 16*AF weight rows x 16*MB activation rows
// over the whole K range, so no partial sums leave the workgroup and a call
// is a single launch.  The NWV waves take 1/NWV of K each; their fp32 panels
// are added through LDS in wave order at the end.
//
// Both operands reach the MFMAs through LDS.  Each wave owns a ring of D
// chunk slots (CS 64-k steps per chunk) and fills them with direct
// global->LDS loads (global_load_lds_dwordx4): every load instruction moves
// 1 KB of whole row segments -- whole 128-byte lines -- and needs no
// registers, so D chunks stay in flight while the MFMAs consume an earlier
// one.  Loaded straight in the MFMA operand layout instead (16 rows x 64
// bytes per instruction), the weight stream touched twice as many cache lines
// per instruction and measured about 2 us slower per call on the Llama-3-8B
// q_proj at M = 32..64 (MI355X).  The 16-byte units of a staged row are
// XOR-swizzled by the row's low bits (global side: a lane fetches the unit
// that belongs at its LDS position), so the 16-row operand reads are free of
// bank conflicts.
//
// Every activation type arrives the same way.  16-bit activations are
// staged as they are; bf16 activations quantized on the fly (kActQ) are cast
// to E4M3 and widened back to bf16 in place in their slot (one read and one
// write per staged unit, by the wave that owns the slot) before the MFMAs
// read them; E4M3 activation codes (kActF8) are staged as codes and widened
// to bf16 after the operand read, as the weights are.  No value of the
// pipeline passes through a compiler-visible load: loaded into registers
// instead, the compiler guarded each use with its own vmcnt wait, counting
// only the loads it could see, and so waited for direct loads of later
// chunks too (the E4M3 decode took 8.6 us at M = 1 on q_proj against 5.7 us
// for bf16).
//
// XS: activation rows staged per chunk (the panel's first XS rows; the host
// plans XS >= the rows that exist).  Staging fewer rows than the panel has
// saves loads and, with activations quantized on the fly, the casts of rows
// that only feed output columns that are never stored; the LDS rows past XS
// are zeroed once.
//
// RPW: activation rows per workgroup along the grid's y (16 * MB unless a
// small weight needs more workgroups: the activation rows are then spread
// over more of them, each reading the same weight panel, which the other
// workgroups of its column find in L2).  Panel rows past RPW feed outputs
// that are never stored.
//
// GRP: per-group weight scales (the deployment guide, §4.3): w_scale [n,
// ngroups] for groups of 2^glog k (64..512).  The MFMAs accumulate a group's
// products on their own (accg); at the group's end the lane's 4 weight rows'
// scales multiply them into the running total.  GRP = 2: before the K loop
// each wave loads the scales of its whole K range, [WR rows][K range /
// group], into LDS beside the rings, each load instruction covering runs of
// consecutive groups of a few rows (the host plans it where that block fits).
// GRP = 1: the scales of a chunk's groups are staged with the chunk, one
// 4-byte direct load per row and group, which touches WR rows' cache lines
// per instruction and costs up to a third of the kernel's time on long K.
// The host plans either only where a wave's K range is a whole number of
// groups.
//
// The host plans this kernel only for K a multiple of NWV * 64 * CS with at
// least D chunks per wave.  Rows past N or M are clamped to a valid row when
// loading and their outputs are never stored.  A load instruction covers at
// most 8 weight rows or 4 activation rows, addressed from that group's first
// row, so the per-lane 32-bit offsets hold for row strides below 2^28 bytes
// (checked by the host).
// LDS of k_w8a16_panel's rings (NWV waves, D chunk slots each), and what a
// wave may take beside them for preloaded group scales within gfx950's 160 KB
// per workgroup (whole 256-byte loads).
constexpr int kPanelLdsBytes = 160 * 1024;
constexpr int panel_ring_bytes(int af, int mb, int cs, int d, int nwv, bool f8, bool chunk_scales)
{
    const int ck = 64 * cs, wr = 16 * af;
    const int xslot = 16 * mb * ck * (f8 ? 1 : 2);
    const int se = chunk_scales ? wr * (ck / 64) : 0;
    return nwv * d * (xslot + wr * ck + (se + 63) / 64 * 256);
}
constexpr int panel_scale_bytes(int ring, int nwv)
{
    return ring >= kPanelLdsBytes ? 0 : ((kPanelLdsBytes - ring) / nwv) & ~255;
}
// Preloaded group scales: not for E4M3 codes at 17..32 rows (two fragments,
// 4-step chunks), whose kernel then spills to scratch.
constexpr bool panel_preload_ok(int af, int cs, bool f8)
{
    return !(f8 && af == 2 && cs == 4);
}

template <int AF, int MB, int CS, int D, int NWV, int AT, int XS = 16 * MB, int RPW = 16 * MB,
          int GRP = 0>
__global__ __launch_bounds__(NWV * 64) void k_w8a16_panel(
    const void *__restrict__ xv, int64_t m, int64_t k, int64_t ld_x,
    const float *__restrict__ x_scale,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int glog, int64_t ngroups, QuantArgs qa)
{
    constexpr bool F8 = AT == kActF8;           // activations staged as E4M3 codes
    constexpr int CT = compute_type<AT>();
    constexpr int ES = F8 ? 1 : 2;              // bytes per activation value in memory and in LDS
    constexpr int XR = 16 * MB;                 // activation rows of the panel
    constexpr int WR = 16 * AF;                 // weight rows of the panel
    constexpr int CK = 64 * CS;                 // k per chunk
    constexpr int XU = CK * ES / 16;            // 16-byte units of an activation row segment
    constexpr int XRB = 16 * XU;                // bytes of a staged activation row segment
    constexpr int NI = XS * XU / kWave;         // activation loads per lane per chunk
    constexpr int XSW = XU >= 16 ? 15 : XU - 1; // activation unit swizzle mask
    constexpr int WU = CK / 16;                 // 16-byte units of a weight row segment
    constexpr int NW = WR * WU / kWave;         // weight loads per lane per chunk
    constexpr int WSW = WU >= 16 ? 15 : WU - 1; // weight unit swizzle mask
    // group scales staged per chunk: up to CK / 64 groups x WR rows, floats
    // [group][row], in whole 256-byte (64-lane) loads
    constexpr int SE = GRP == 1 ? WR * (CK / 64) : 0;
    constexpr int NS = (SE + kWave - 1) / kWave;
    constexpr int LC = NI + NW + NS;            // loads per lane per chunk
    constexpr int XSLOT = XR * XRB, WSLOT = WR * CK, SSLOT = NS * 4 * kWave;
    constexpr int SLOT = D * (XSLOT + WSLOT + SSLOT);
    constexpr int RED = (int)sizeof(v4f) * NWV * AF * MB * kWave;
    // GRP = 2: each wave's preloaded scales, in the LDS the rings leave free
    constexpr int SAB = GRP == 2 ? panel_scale_bytes(NWV * SLOT, NWV) : 0;
    static_assert(NWV * SLOT == panel_ring_bytes(AF, MB, CS, D, NWV, F8, GRP == 1),
                  "ring size as the host plans it");
    static_assert(GRP != 2 || SAB >= 256 * 4, "room for the preloaded scales");
    static_assert((XS * XU) % kWave == 0 && XS <= XR && XS > 0 && (XU & (XU - 1)) == 0,
                  "chunk shape");
    static_assert((WR * WU) % kWave == 0 && (WU & (WU - 1)) == 0, "weight chunk shape");
    static_assert(RPW > 0 && RPW <= XR, "activation rows per workgroup");
    static_assert(D >= 1 && D <= 4, "chunks in flight");
    // the waves' rings; after the K loop the same bytes hold the waves' fp32
    // panels for the reduction
    __shared__ __attribute__((aligned(16)))
    uint8_t xl[NWV * (SLOT + SAB) > RED ? NWV * (SLOT + SAB) : RED];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int r = lane & 15;          // row of the A (weight) / B (activation) operand
    const int g = lane >> 4;          // which 16 k-values of a 64-k step this lane holds
    const int64_t n0 = (int64_t)blockIdx.x * WR;
    const int64_t m0 = (int64_t)blockIdx.y * RPW;
    const int64_t kq = k / NWV;
    const int64_t kb = (int64_t)wave * kq;
    const int nch = (int)(kq / CK);
    uint8_t *xslot = xl + wave * SLOT;                  // D activation slots
    uint8_t *wslot = xslot + D * XSLOT;                 // D weight slots
    uint8_t *sslot = wslot + D * WSLOT;                 // D group-scale slots
    const uint32_t xslot_lds = (uint32_t)(uintptr_t)xslot;
    const uint32_t wslot_lds = (uint32_t)(uintptr_t)wslot;
    const uint32_t sslot_lds = (uint32_t)(uintptr_t)sslot;
    // kActQ without maxima from an absmax pass: the scale from the whole
    // (small) activation tensor, before the pipeline starts
    const float xs = AT == kActQ && qa.part == nullptr
                         ? scan_act_scale(static_cast<const uint16_t *>(xv), m, k, ld_x, qa)
                         : act_scale<AT>(x_scale, qa);
    const E4M3Div div(AT == kActQ ? xs : 1.0f, true);

    // load i of a chunk fills LDS bytes [1 KB i, 1 KB (i + 1)) of the slot:
    // for an operand of U units per row segment, rows (64 / U) i .. , lane l
    // at row l / U, position l % U, which holds global unit (l % U) ^ swizzle(row)
    constexpr int WPI = kWave / WU;
    uint32_t woff[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int rho = WPI * i + lane / WU, q = lane % WU;
        const int64_t row0 = min(n0 + WPI * i, n - 1);
        woff[i] = (uint32_t)((min(n0 + rho, n - 1) - row0) * ld_w + 16 * (q ^ (rho & WSW)));
    }
    auto wbase = [&](int i, int c) {
        return w + min(n0 + WPI * i, n - 1) * ld_w + kb + (int64_t)c * CK;
    };
    const uint8_t *x8 = static_cast<const uint8_t *>(xv);
    constexpr int XPI = kWave / XU;
    uint32_t xoff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int rho = XPI * i + lane / XU, q = lane % XU;
        const int64_t row0 = min(m0 + XPI * i, m - 1);
        xoff[i] = (uint32_t)((min(m0 + rho, m - 1) - row0) * ld_x * ES + 16 * (q ^ (rho & XSW)));
    }
    auto xbase = [&](int i, int c) {
        return x8 + (min(m0 + XPI * i, m - 1) * ld_x + kb + (int64_t)c * CK) * ES;
    };
    // group-scale load i: element e = 64 i + lane is group e / WR of the
    // chunk (clamped to the groups the chunk has), weight row e % WR
    uint32_t soff[NS > 0 ? NS : 1];
    if constexpr (GRP == 1) {
        const int gpc = CK >> glog > 0 ? CK >> glog : 1;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int e = kWave * i + lane;
            const int gi = min(e / WR, gpc - 1), row = e % WR;
            soff[i] = (uint32_t)(((min(n0 + row, n - 1) - n0) * ngroups + gi) * 4);
        }
    }
    auto sbase = [&](int c) {
        return w_scale + n0 * ngroups + ((kb + (int64_t)c * CK) >> glog);
    };

    if constexpr (XS < XR) {
#pragma unroll
        for (int u = 0; u < D; ++u)
#pragma unroll
            for (int o = XS * XRB + 16 * lane; o < XR * XRB; o += 16 * kWave)
                *reinterpret_cast<v4u *>(xslot + u * XSLOT + o) = v4u{0u, 0u, 0u, 0u};
    }

    v4f acc[AF][MB], accg[GRP ? AF : 1][GRP ? MB : 1];
    // GRP = 2: groups of the wave's K range, and its scales [WR][gw] in LDS
    const int gw = GRP == 2 ? (int)(kq >> glog) : 0;
    const float *sall = reinterpret_cast<const float *>(xl + NWV * SLOT + wave * SAB);
    if constexpr (GRP == 2) {
        // element e = row * gw + j (row of the panel, j-th group of the K
        // range), lane l of load i holding e = 64 i + l, so a load covers
        // 64 / gw rows' runs of consecutive groups; the lanes past the
        // block repeat its last element into the padding
        const uint32_t sall_lds = (uint32_t)(uintptr_t)sall;
        const float *sb = w_scale + n0 * ngroups + (kb >> glog);
        const int tot = WR * gw;
        for (int i = 0; i < tot; i += kWave) {
            const int e = min(i + lane, tot - 1);
            const int row = e / gw, j = e - row * gw;
            dma4(sb, (uint32_t)(((min(n0 + row, n - 1) - n0) * ngroups + j) * 4), sall_lds + 4 * i);
        }
    }
#pragma unroll
    for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int j = 0; j < MB; ++j)
            acc[a][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (GRP) {
#pragma unroll
        for (int a = 0; a < AF; ++a)
#pragma unroll
            for (int j = 0; j < MB; ++j)
                accg[a][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    auto issue = [&](int u, int c) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            dma16(xbase(i, c), xoff[i], xslot_lds + u * XSLOT + 1024 * i);
#pragma unroll
        for (int i = 0; i < NW; ++i)
            dma16_nt(wbase(i, c), woff[i], wslot_lds + u * WSLOT + 1024 * i);
        if constexpr (GRP == 1) {
#pragma unroll
            for (int i = 0; i < NS; ++i)
                dma4(sbase(c), soff[i], sslot_lds + u * SSLOT + 4 * kWave * i);
        }
    };
    // the wait for chunk c: loads retire in order, and the chunks issued after
    // it are min(D - 1, nch - 1 - c) whole chunks of LC loads each
    auto wait_chunk = [&](int c) {
        const int after = min(D - 1, nch - 1 - c);
        static_for<0, D>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if (after == j)
                wait_vmcnt<j * LC>();
        });
    };
    // kActQ: the staged bf16 units of slot u cast to E4M3 and widened back,
    // in place (elementwise, so the units' swizzled positions do not matter)
    auto quantize_slot = [&](int u) {
        if constexpr (AT == kActQ) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                v4u *p = reinterpret_cast<v4u *>(xslot + u * XSLOT + 1024 * i + 16 * lane);
                *p = qdq8(*p, div);
            }
        }
    };
    auto compute = [&](int u, int c) {
        const uint8_t *xs_ = xslot + u * XSLOT;
        const uint8_t *ws_ = wslot + u * WSLOT;
#pragma unroll
        for (int s = 0; s < CS; ++s) {
            typename Act<CT>::frag a0[AF], a1[AF];
#pragma unroll
            for (int a = 0; a < AF; ++a) {
                const int rho = 16 * a + r;
                const v4u wv = *reinterpret_cast<const v4u *>(ws_ + rho * CK + 16 * ((4 * s + g) ^ (rho & WSW)));
                widen<CT>(wv, a0[a], a1[a]);
            }
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                const int rho = 16 * j + r;
                typename Act<CT>::frag b0, b1;
                if constexpr (F8) {
                    // 16 codes: k = 64 s + 16 g .. + 15 of this row
                    const v4u cv = *reinterpret_cast<const v4u *>(xs_ + rho * XRB + 16 * ((4 * s + g) ^ (rho & XSW)));
                    widen<CT>(cv, b0, b1);
                } else {
                    const int u0 = 8 * s + 2 * g;
                    b0 = Act<CT>::cast(*reinterpret_cast<const v4u *>(xs_ + rho * XRB + 16 * (u0 ^ (rho & XSW))));
                    b1 = Act<CT>::cast(*reinterpret_cast<const v4u *>(xs_ + rho * XRB + 16 * ((u0 + 1) ^ (rho & XSW))));
                }
#pragma unroll
                for (int a = 0; a < AF; ++a) {
                    if constexpr (GRP) {
                        accg[a][j] = Act<CT>::mfma(a0[a], b0, accg[a][j]);
                        accg[a][j] = Act<CT>::mfma(a1[a], b1, accg[a][j]);
                    } else {
                        acc[a][j] = Act<CT>::mfma(a0[a], b0, acc[a][j]);
                        acc[a][j] = Act<CT>::mfma(a1[a], b1, acc[a][j]);
                    }
                }
            }
            if constexpr (GRP) {
                // the group ends with this step: its sums, times the lane's
                // 4 weight rows' scales, join the total
                if ((((c * CS + s + 1) << 6) & ((1 << glog) - 1)) == 0) {
                    const int gi = (s << 6) >> glog;
                    const int t = (((c * CS + s + 1) << 6) >> glog) - 1;
                    const float *sc = reinterpret_cast<const float *>(sslot + u * SSLOT) + gi * WR;
#pragma unroll
                    for (int a = 0; a < AF; ++a) {
                        v4f s4;
                        if constexpr (GRP == 2) {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                s4[v] = sall[(16 * a + 4 * g + v) * gw + t];
                        } else {
                            s4 = *reinterpret_cast<const v4f *>(sc + 16 * a + 4 * g);
                        }
#pragma unroll
                        for (int j = 0; j < MB; ++j) {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                acc[a][j][v] = __builtin_fmaf(s4[v], accg[a][j][v], acc[a][j][v]);
                            accg[a][j] = v4f{0.f, 0.f, 0.f, 0.f};
                        }
                    }
                }
            }
        }
    };

    // prologue: the first D chunks (nch >= D)
    static_for<0, D>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        issue(u, u);
    });
    for (int c0 = 0; c0 < nch; c0 += D) {
        static_for<0, D>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            const int c = c0 + u;
            if (c < nch) {
                wait_chunk(c);
                __builtin_amdgcn_sched_barrier(0);
                quantize_slot(u);
                compute(u, c);
                __builtin_amdgcn_sched_barrier(0);
                // slot u is free again: its operand reads fed the MFMAs above
                if (c + D < nch)
                    issue(u, c + D);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    }

    // ---- the waves' panels, added in wave order, then scaled and stored ----
    __syncthreads();
    v4f *red = reinterpret_cast<v4f *>(xl);     // [wave][AF * MB][lane]
#pragma unroll
    for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int j = 0; j < MB; ++j)
            red[(wave * AF * MB + a * MB + j) * kWave + lane] = acc[a][j];
    __syncthreads();
    // one thread per (fragment, lane) slot: weight rows 4g'..4g'+3 of
    // fragment a, activation row 16j + r' (lane layout of the MFMA result)
    for (int sl = threadIdx.x; sl < AF * MB * kWave; sl += blockDim.x) {
        const int f = sl / kWave;
        const int ln = sl % kWave;
        const int a = f / MB;
        const int j = f % MB;
        const int64_t mr = m0 + 16 * j + (ln & 15);
        const int64_t nb = n0 + 16 * a + 4 * (ln >> 4);
        if (mr >= m || nb >= n || 16 * j + (ln & 15) >= RPW)
            continue;
        v4f sum = red[f * kWave + ln];
#pragma unroll
        for (int wv = 1; wv < NWV; ++wv)
            sum += red[(wv * AF * MB + f) * kWave + ln];
        // grouped: the group scales are in the sums already
        store_y4<CT>(y, ld_y, GRP ? nullptr : w_scale, xs, mr, nb, n, sum);
    }
}

// Sum of the K splits' partial tiles in split order, scaled and stored as
// bf16: one thread per 4 consecutive outputs of a row.  w_scale == nullptr:
// the partials already carry the per-group weight scales.
template <int AT>
__global__ __launch_bounds__(256) void k_w8a16_reduce(
    const float *__restrict__ partial, int64_t m, int64_t n, int64_t ldp, int splits,
    const float *__restrict__ x_scale, const float *__restrict__ w_scale, uint16_t *__restrict__ y,
    int64_t ld_y)
{
    constexpr int CT = compute_type<AT>();
    const float xs = AT == kActF8 || AT == kActQ ? *x_scale : 1.0f;
    const int64_t q = ldp / 4;
    const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (slot >= m * q)
        return;
    const int64_t mr = slot / q;
    const int64_t nb = 4 * (slot % q);
    // every load is issued before the first add: the weight scales (clamped
    // to row n-1; only valid columns are stored) and up to 8 splits per
    // batch.  The sum still runs in split order.
    float ws[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        ws[v] = w_scale != nullptr ? w_scale[min(nb + v, n - 1)] : 1.0f;
    auto part = [&](int sp) {
        return *reinterpret_cast<const v4f *>(partial + ((int64_t)sp * m + mr) * ldp + nb);
    };
    constexpr int kBatch = 8;
    v4f s = part(0);
    for (int sb = 1; sb < splits; sb += kBatch) {
        v4f p[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (sb + i < splits)
                p[i] = part(sb + i);
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (sb + i < splits)
                s += p[i];
    }
    uint16_t *yp = y + mr * ld_y + nb;
    if (nb + 4 <= n) {
        uint2 o;
        o.x = Act<CT>::pack2(s[0] * (xs * ws[0]), s[1] * (xs * ws[1]));
        o.y = Act<CT>::pack2(s[2] * (xs * ws[2]), s[3] * (xs * ws[3]));
        *reinterpret_cast<uint2 *>(yp) = o;
    } else {
        for (int v = 0; v < (int)(n - nb); ++v)
            yp[v] = Act<CT>::one(s[v] * (xs * ws[v]));
    }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Device-resident scratch for callers that cannot allocate (fp8q_linear_noalloc):
// the K-split partial tiles of the decode kernels.  Each GPU holds its own copy
// from the library's load to the end of the process.  In host code the name
// `scratch` is only a stand-in for the device symbol; its device address comes
// from hipGetSymbolAddress, resolved once per device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace launch {

hipError_t noalloc_scratch(int device, void **ptr)
{
    static std::mutex mu;
    static void *addr[kNoallocMaxDevices] = {};
    if (device < 0 || device >= kNoallocMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[device] == nullptr) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != device ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess)
            return e;
        if (back != hipSuccess)
            return back;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        addr[device] = p;
    }
    *ptr = addr[device];
    return hipSuccess;
}

// Register-pipeline depth of the rows kernel: about 24-36 16-byte loads in
// flight per lane.
static int rows_depth(int af, int mb) { return (af + 2 * mb) <= 4 ? 8 : ((af + 2 * mb) <= 6 ? 4 : 2); }

// The tile kernel's part of a plan: rows staged per wave, chunk length, and
// the K split towards 256 workgroups.
static void plan_tile(W8A16Plan &p, int64_t m, int64_t k, int steps_mb1)
{
    const int64_t tiles = p.tiles_n * p.grid_m;
    p.kind = W8A16Plan::kTile;
    if (p.mb == 1) {
        // stage only the activation rows that exist: 4, 8 or 16 of the 16
        p.xd = (int)div_up(m, kTileWaves);
        p.steps = steps_mb1;
    } else {
        p.xd = 4 * p.mb;
        p.steps = 8;
    }
    // split K (in whole chunks) towards 256 workgroups, keeping at least two
    // chunks per split so each workgroup's pipeline gets past its prologue
    const int64_t chunk = 64 * p.steps;
    int64_t s = 256 / tiles;
    const int64_t s_max = k / (2 * chunk);
    s = s > s_max ? s_max : s;
    s = s < 1 ? 1 : s;
    p.kper = div_up(div_up(k, s), chunk) * chunk;
    p.splits = div_up(k, p.kper);
    p.workspace = p.splits > 1 ? (size_t)p.splits * m * p.ldp * sizeof(float) : 0;
    p.grid_n = p.tiles_n * p.splits;
}

// The panel kernel's plans (one launch, whole K per workgroup, no partial
// sums).  Measured on MI355X in graphs, weights rotating through 2 GiB:
//  - up to 16 activation rows, one activation group (MB = 1): AF weight
//    fragments per workgroup, AF in {1, 2, 3, 4, 7}, the AF with the least
//    rounds of 256 workgroups x (2 AF + 1) (the rule below; ties to the
//    larger AF); a weight of 256..1535 rows spreads the activation rows 4
//    per workgroup.  (Figures below are from before the non-temporal weight
//    loads, which took another 5-11% off.)
//    Llama-3-8B q_proj (4096 x 4096): M = 1 5.7 us, M = 8 5.9 us, M = 16
//    6.7 us against 5.8 / 7.0 / 8.3 us for the rows kernel; Llama-3-70B at
//    M = 12: q/o (8192 x 8192) 14.1 us, gate/up (28672 x 8192) 42.6 us,
//    down (8192 x 28672) 43.4 us against 51.1 us for the split tile kernel +
//    reduce; Llama-3-8B k/v (1024 x 4096) at M = 8 4.9 us on 64 workgroups
//    against 6.8 us for the split rows kernel + reduce (but 8.4 against 7.4
//    us for the 70B k/v, K = 8192).
//  - 17..32 activation rows: two activation groups of 16 rows along the grid
//    (MB = 1, AF = 2); 33..64 rows: 32-row groups (MB = 2, AF = 2); both only
//    where that makes 192..320 workgroups.  q_proj M = 24 7.2 us, M = 32 7.9
//    us, M = 64 9.6 us (12.0 us with the weights loaded straight into
//    registers).  E4M3 activation codes take chunks of 4 x 64 k there.
//  - E4M3 activation codes up to 16 rows: as 16-bit activations, 3 chunks
//    in flight (q_proj M = 1: 5.5 us; half the activation bytes).
// Activations cast on the fly (kActQ) stage only the rows that exist (4, 8 or
// 16).  Chunks of CS x 64 k, D of them in flight: the LDS of 4 waves' rings
// bounds CS * D * (activation + weight row bytes).
// grouped: per-group weight scales; the kernels with the most direct-load
// addresses (7 weight fragments; E4M3 codes at 33..64 rows) then run out of
// scalar registers, spill to scratch, and the compiler's waits for the spill
// loads stall the direct loads, so those shapes take at most 4 fragments or
// the rows / tile kernels.
static bool plan_panel(W8A16Plan &out, int64_t m, int64_t n, int64_t k, int act,
                       bool grouped = false)
{
    const bool f8 = act == kW8A16ActF8, q = act == kW8A16ActQ;
    if (m < 1 || m > 512 || n < 1 || k % 512 != 0 || k < 2048)
        return false;
    W8A16Plan p = out;
    p.kind = W8A16Plan::kPanel;
    p.waves = 4;
    p.splits = 1;
    p.workspace = 0;
    p.rpw = 0;
    p.kper = k;
    p.kchunk = k / 4;
    if (m > 64) {
        // 65..512 rows (a batched decode the host runs here instead of a
        // prefill GEMM): 64 weight rows x 32 activation rows per workgroup,
        // the tile that reads the least per CU for these shapes (K x (64 +
        // 2 x 32) bytes of operands per k for bf16).  Two 128-k chunks in
        // flight per wave where the grid is one round, else one (64 KB of
        // rings: two workgroups per CU).  Against the tile kernel, K = 4096,
        // graphs, weights rotated past the Infinity Cache:
        //   E4M3, N = 4096: 65..512 rows 10.8 / 11.0 / 16.7 / 23.8 / 34.8 us
        //     (65, 128, 256, 384, 512) against 16.7 / 18.0 / 21.3 / 40.5 /
        //     42.5; N = 8192: 19.2 / 19.3 / 27.7 / 40.5 (65..256) against
        //     23.0 / 22.7 / 41.5 / 44.1
        //   bf16, N = 4096: 11.9 / 12.1 / 19.4 / 35.8 / 39.7 against 16.3 /
        //     17.3 / 20.9 / 39.7 / 40.4; a grid of more than one round on a
        //     wider weight lost (N = 8192 at 128..512 rows 23.0..91.6 against
        //     21.8..80.2, N = 28672 at 128 rows 98.1 against 86.2) except at
        //     3 activation groups (65 rows: 20.0 against 21.7 at N = 8192,
        //     68.9 against 84.5 at N = 28672), so 16-bit activations take
        //     it only there.
        if (q || grouped)
            return false;
        const int64_t wgs = div_up(n, 64) * div_up(m, 32);
        if (wgs < 128 || (!f8 && wgs > 256 && n > 4096 && div_up(m, 32) > 3))
            return false;
        p.af = 4;
        p.mb = 2;
        p.steps = 2;
        p.depth = wgs <= 256 ? 2 : 1;
        p.xd = 32;
    } else if (m <= 16) {
        if (n < 256)
            return false;
        static const int kAf[5] = {1, 2, 3, 4, 7};
        int best = 0;
        int64_t best_cost = 0;
        for (int i = 0; i < (grouped ? 4 : 5); ++i) {
            // rounds of 256 workgroups, each as long as its fragments, plus
            // half a fragment per round for the pipeline's fill and drain
            // (M = 8, 28672 x 4096: 1 fragment, 7 rounds 32.6 us; 4 fragments,
            // 2 rounds 25.7 us; 7 fragments, 1 round 24.0 us)
            const int64_t rounds = div_up(div_up(n, 16 * kAf[i]), 256);
            const int64_t cost = rounds * (2 * kAf[i] + 1);
            if (i == 0 || cost < best_cost || (cost == best_cost && kAf[i] > kAf[best])) {
                best = i;
                best_cost = cost;
            }
        }
        // casting the activations on the fly needs many workgroups (1024 x
        // 8192: 24 us on 64 workgroups against 7.4 us for the split rows
        // kernel + reduce on bf16)
        if (q && n < 2048)
            return false;
        if (div_up(n, 16) < 96 && !q) {
            // a small weight (Llama-3 k/v, 1024 rows): 16-row panels, the
            // activation rows spread 4 per workgroup (each weight panel read
            // by div_up(m, 4) workgroups, from L2 after the first).  At M =
            // 12: 70B k/v (1024 x 8192) 6.8 us against 7.4 us for the split
            // rows kernel + reduce and 8.4 us for one workgroup per panel;
            // 8B k/v (1024 x 4096) 4.6 against 4.8 us.
            if (k % 1024 != 0)
                return false;
            p.af = 1;
            p.mb = 1;
            p.rpw = 4;
            p.steps = 4;
            p.depth = 2;
            p.xd = 4;
            p.rows = 16;
            p.grid_n = div_up(n, 16);
            p.grid_m = div_up(m, 4);
            out = p;
            return true;
        }
        p.af = kAf[best];
        p.mb = 1;
        p.steps = 2;
        p.depth = p.af == 7 ? 2 : (p.af > 2 || q || f8) ? 3 : 4;
        p.xd = q ? (m <= 4 ? 4 : m <= 8 ? 8 : 16) : 16;
    } else {
        if (q || (grouped && f8 && m > 32))
            return false;
        p.af = 2;
        p.mb = m > 32 ? 2 : 1;
        p.steps = f8 ? 4 : 2;
        // E4M3 codes at 17..32 rows: 3 chunks in flight where K has them
        p.depth = m > 32 || (f8 && k < 3 * 4 * 64 * p.steps) ? 2 : 3;
        p.xd = 16 * p.mb;
        const int64_t wgs = div_up(n, 32) * div_up(m, 16 * p.mb);
        const int64_t n64 = div_up(n, 64);
        if (wgs > 320 && m <= 32 && !grouped && n64 * 2 >= 192 && n64 * 2 <= 256) {
            // 17..32 rows on 6145..8192 weight rows: 64-row panels, two
            // 16-row activation groups, one round of workgroups (bf16, 8192
            // x 4096: 24 rows 10.5 us, 32 rows 10.8 us against 14.2 / 14.6
            // us for the tile kernel)
            p.af = 4;
            p.steps = 2;
            p.depth = 3;
            p.xd = 16;
        } else if (wgs > 320 && m <= 32 && !grouped && n64 >= 192 && n64 <= 256) {
            // 17..32 rows on 12289..16384 weight rows: 64 x 32 tiles, one
            // round (bf16, 14336 x 4096: 24 rows 14.4 us, 32 rows 15.0 us
            // against 19.8 / 20.1 us for the tile kernel)
            p.af = 4;
            p.mb = 2;
            p.steps = 2;
            p.depth = 2;
            p.xd = 32;
        } else if (wgs > 320 && m > 32 && !grouped && n64 * 2 <= 256) {
            // 33..64 rows on a weight of up to 8192 rows: the 64 x 32 tiles
            // of the 65..512-row plan, one round of workgroups (bf16, 8192 x
            // 4096: 48 rows 13.0 us, 64 rows 13.2 us against 16.7 / 18.8 us
            // for the tile kernel; at 14336 rows and more the panels tie
            // with the tile kernel or lose)
            p.af = 4;
            p.steps = 2;
            p.depth = 2;
            p.xd = 32;
        } else if (wgs < 192 || wgs > 320 || k % (4 * 64 * p.steps) != 0 ||
                   k / (4 * 64 * p.steps) < p.depth) {
            return false;
        }
    }
    p.rows = 16 * p.af;
    p.grid_n = div_up(n, 16 * p.af);
    p.grid_m = div_up(m, 16 * p.mb);
    out = p;
    return true;
}

// The rows / tile kernels' plans (the per-group weight scales use these too).
static W8A16Plan plan_rows_tile(int64_t m, int64_t n, int64_t k)
{
    W8A16Plan p{};
    const int64_t mgroups = div_up(m, 16);
    p.mb = (int)(mgroups >= 4 ? 4 : (mgroups < 1 ? 1 : mgroups));
    p.grid_m = div_up(m, 16 * p.mb);
    p.tiles_n = div_up(n, kTileN);
    p.splits = 1;
    p.workspace = 0;
    p.ldp = div_up(n, 4) * 4;
    // The rows kernel wins for up to 16 activation rows on a weight of up to
    // 4096 rows with K < 16K; a wider weight takes the split tile kernel
    // below, a long K, a small N or more activation rows the tile kernel
    // (measured on MI355X across the Llama-3 8B/70B decode shapes).
    const int64_t tiles = p.tiles_n * p.grid_m;
    const bool small_n_long_k = p.mb == 1 && tiles <= 32 && k >= 4096 && k < 16384;
    const bool tile = !small_n_long_k && (p.mb > 1 || tiles >= 256 || tiles <= 32 || k >= 16384);
    p.splits = 1;
    p.ldp = div_up(n, 4) * 4;
    if (small_n_long_k) {
        // a small N on a long K (e.g. the k/v projections): 16-row
        // workgroups, K split across workgroups towards 256 of them, each
        // wave keeping at least 512 k (one pipelined span)
        p.kind = W8A16Plan::kRows;
        p.rows = 16;
        p.af = 1;
        p.grid_n = div_up(n, 16);
        p.waves = 4;
        p.depth = rows_depth(p.af, p.mb);
        const int64_t span = 64 * p.depth * p.waves;        // one span per wave
        int64_t s = 256 / (p.grid_n * p.grid_m);
        const int64_t s_max = k / span;
        s = s > s_max ? s_max : s;
        s = s < 1 ? 1 : s;
        p.kper = div_up(div_up(k, s), span) * span;
        p.splits = div_up(k, p.kper);
        p.kchunk = p.kper / p.waves;
        if (p.splits > 1)
            p.workspace = (size_t)p.splits * m * p.ldp * sizeof(float);
        return p;
    }
    if (p.mb == 1 && p.tiles_n > 64 && k >= 8192 && k < 16384) {
        // up to 16 activation rows on a weight wider than 4096 rows with
        // 8K <= K < 16K (the Llama-3-70B q/o, fused qkv and gate/up at
        // decode): the tile kernel with K split 4 ways -- more, smaller
        // workgroups even out the CUs.  Measured on MI355X at M = 12: fused
        // qkv [10240, 8192] 25.9 us against 34.5 us for the rows kernel, gate
        // [28672, 8192] 55.7 us against 58.1 us unsplit.  At K = 4096 the
        // split chunks get too short and the unsplit plans below stay faster.
        p.kind = W8A16Plan::kTile;
        p.xd = (int)div_up(m, kTileWaves);
        p.steps = p.tiles_n >= 256 ? 16 : 8;
        const int64_t chunk = 64 * p.steps;
        int64_t s = 4;
        const int64_t s_max = k / (2 * chunk);
        s = s > s_max ? s_max : s;
        s = s < 1 ? 1 : s;
        p.kper = div_up(div_up(k, s), chunk) * chunk;
        p.splits = div_up(k, p.kper);
        p.workspace = p.splits > 1 ? (size_t)p.splits * m * p.ldp * sizeof(float) : 0;
        p.grid_n = p.tiles_n * p.splits;
        return p;
    }
    if (!tile) {
        p.kind = W8A16Plan::kRows;
        // rows per block: the most rows (up to 32) that still leave >= 256 blocks
        int rows = 32;
        while (rows > 4 && div_up(n, rows) * p.grid_m < 256)
            rows /= 2;
        p.rows = rows;
        p.af = rows > 16 ? 2 : 1;
        p.grid_n = div_up(n, rows);
        p.waves = 4;
        p.depth = rows_depth(p.af, p.mb);
        // the waves split K; a wave's range is a multiple of the pipelined span
        // (64 * depth) when K is large enough, else of 64
        const int64_t per = div_up(k, p.waves);
        const int64_t span = 64 * p.depth;
        p.kchunk = per >= span ? div_up(per, span) * span : div_up(per, 64) * 64;
        p.kper = p.kchunk * p.waves;
        return p;
    }
    plan_tile(p, m, k, (k >= 16384 || tiles >= 256) ? 16 : 8);
    return p;
}

W8A16Plan plan_w8a16(int64_t m, int64_t n, int64_t k, int act)
{
    W8A16Plan p = plan_rows_tile(m, n, k);
    plan_panel(p, m, n, k, act);
    return p;
}

W8A16Plan plan_w8a16_grouped(int64_t m, int64_t n, int64_t k, int64_t group, int act)
{
    // the panel kernel where it takes the per-channel call and every wave's K
    // range is a whole number of groups
    if (act != kW8A16ActQ) {
        W8A16Plan p = plan_rows_tile(m, n, k);
        if (plan_panel(p, m, n, k, act, true) && (k / p.waves) % group == 0) {
            p.group = group;
            // the wave's [rows][groups] scales, in whole 64-element loads,
            // beside the rings if they fit
            const int64_t elems = div_up(16 * p.af * (k / p.waves / group), 64) * 64;
            const int ring = panel_ring_bytes(p.af, p.mb, p.steps, p.depth, p.waves,
                                              act == kW8A16ActF8, false);
            p.scale_stage = panel_preload_ok(p.af, p.steps, act == kW8A16ActF8) &&
                                    elems * 4 <= panel_scale_bytes(ring, p.waves)
                                ? 2 : 1;
            return p;
        }
    }
    // where the per-channel plan takes the rows kernel, so does the grouped
    // one, with wave K ranges in whole 512-k rounds (so groups of up to 512 k
    // never straddle a round).  A K split (small N on a long K) already cuts
    // K into multiples of 4 waves x 512 k; unsplit, the wave ranges are
    // rounded up to 512 k.
    {
        W8A16Plan r = plan_rows_tile(m, n, k);
        if (r.kind == W8A16Plan::kRows && r.mb == 1 && r.depth == 8) {
            if (r.splits == 1) {
                r.kchunk = div_up(div_up(k, r.waves), 512) * 512;
                r.kper = r.kchunk * r.waves;
            }
            if (r.kchunk % 512 == 0) {
                r.group = group;
                return r;
            }
        }
    }
    // else the tile kernel, with the per-channel plan's chunks of 512 or
    // 1024 k (8 or 16 steps), each a whole number of groups of 64..512 k
    W8A16Plan p{};
    const int64_t mgroups = div_up(m, 16);
    p.mb = (int)(mgroups >= 4 ? 4 : (mgroups < 1 ? 1 : mgroups));
    p.grid_m = div_up(m, 16 * p.mb);
    p.tiles_n = div_up(n, kTileN);
    p.ldp = div_up(n, 4) * 4;
    p.group = group;
    const int64_t tiles = p.tiles_n * p.grid_m;
    plan_tile(p, m, k, (k >= 16384 || tiles >= 256) ? 16 : 8);
    if (p.mb == 1 && p.tiles_n > 64 && k >= 8192 && k < 16384) {
        // as the per-channel plan: wide weights split K 4 ways at decode
        p.steps = p.tiles_n >= 256 ? 16 : 8;
        const int64_t chunk = 64 * p.steps;
        int64_t s = 4;
        const int64_t s_max = k / (2 * chunk);
        s = s > s_max ? s_max : s;
        s = s < 1 ? 1 : s;
        p.kper = div_up(div_up(k, s), chunk) * chunk;
        p.splits = div_up(k, p.kper);
        p.workspace = p.splits > 1 ? (size_t)p.splits * m * p.ldp * sizeof(float) : 0;
        p.grid_n = p.tiles_n * p.splits;
    }
    return p;
}

template <int AF, int MB, int P, int NW, int AT, int SPG = 0>
static void launch_rows(const W8A16Plan &p, const void *x, int64_t m, int64_t k, int64_t ld_x,
                        const float *x_scale, const uint8_t *w, int64_t n, int64_t ld_w,
                        const float *w_scale, uint16_t *y, int64_t ld_y, void *workspace,
                        const QuantArgs &qa, hipStream_t stream)
{
    float *partial = static_cast<float *>(workspace);
    const dim3 grid((unsigned)p.grid_n, (unsigned)p.grid_m, (unsigned)p.splits);
    const int64_t ngroups = SPG > 0 ? div_up(k, 64 * SPG) : 0;
    hipLaunchKernelGGL((k_w8a16_rows<AF, MB, P, NW, AT, SPG>), grid, dim3(NW * kWave), 0, stream, x, m,
                       k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y, p.rows, p.kchunk, p.kper,
                       partial, p.ldp, ngroups, qa);
    if (p.splits > 1) {
        const int64_t slots = m * (p.ldp / 4);
        hipLaunchKernelGGL((k_w8a16_reduce<AT>), dim3((unsigned)div_up(slots, 256)), dim3(256), 0, stream,
                           partial, m, n, p.ldp, (int)p.splits,
                           AT == kActQ ? (const float *)qa.scale_out : x_scale,
                           SPG > 0 ? nullptr : w_scale, y, ld_y);
    }
}

template <int MB, int XD, int T, int AT, int SPG = 0>
static void launch_tile(const W8A16Plan &p, const void *x, int64_t m, int64_t k, int64_t ld_x,
                        const float *x_scale, const uint8_t *w, int64_t n, int64_t ld_w,
                        const float *w_scale, uint16_t *y, int64_t ld_y, float *partial,
                        const QuantArgs &qa, hipStream_t stream)
{
    const dim3 grid((unsigned)p.grid_n, (unsigned)p.grid_m);
    const int64_t ngroups = SPG > 0 ? div_up(k, 64 * SPG) : 0;
    hipLaunchKernelGGL((k_w8a16_tile<MB, XD, T, AT, SPG>), grid, dim3(kTileThreads), 0, stream, x,
                       m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y, p.kper, (int)p.splits,
                       partial, p.ldp, ngroups, qa);
    if (p.splits > 1) {
        const int64_t slots = m * (p.ldp / 4);
        hipLaunchKernelGGL((k_w8a16_reduce<AT>), dim3((unsigned)div_up(slots, 256)), dim3(256), 0, stream,
                           partial, m, n, p.ldp, (int)p.splits,
                           AT == kActQ ? (const float *)qa.scale_out : x_scale,
                           SPG > 0 ? nullptr : w_scale, y, ld_y);
    }
}

// k_w8a16_panel, 4 waves (the configurations plan_panel picks).  Per-group
// weight scales are instantiated only where plan_panel takes them (not with
// 7 weight fragments, nor with E4M3 codes at two 16-row blocks); false when
// the plan asks for a kernel that does not exist.
template <int AF, int MB, int CS, int D, int AT, int XS = 16 * MB, int RPW = 16 * MB>
static bool launch_panel(const W8A16Plan &p, const void *x, int64_t m, int64_t k, int64_t ld_x,
                         const float *x_scale, const uint8_t *w, int64_t n, int64_t ld_w,
                         const float *w_scale, uint16_t *y, int64_t ld_y, const QuantArgs &qa,
                         hipStream_t stream)
{
    constexpr bool kGrouped = AT != kActQ && AF != 7 && !(AT == kActF8 && MB == 2) &&
                              !(AF == 4 && MB == 2);
    const dim3 grid((unsigned)p.grid_n, (unsigned)p.grid_m);
    if (p.group > 0) {
        if constexpr (kGrouped) {
            const int glog = p.group == 64 ? 6 : p.group == 128 ? 7 : p.group == 256 ? 8 : 9;
            if constexpr (panel_preload_ok(AF, CS, AT == kActF8)) {
                if (p.scale_stage == 2) {
                    hipLaunchKernelGGL((k_w8a16_panel<AF, MB, CS, D, 4, AT, XS, RPW, 2>), grid,
                                       dim3(4 * kWave), 0, stream, x, m, k, ld_x, x_scale, w, n,
                                       ld_w, w_scale, y, ld_y, glog, div_up(k, p.group), qa);
                    return true;
                }
            }
            if (p.scale_stage == 1)
                hipLaunchKernelGGL((k_w8a16_panel<AF, MB, CS, D, 4, AT, XS, RPW, 1>), grid,
                                   dim3(4 * kWave), 0, stream, x, m, k, ld_x, x_scale, w, n, ld_w,
                                   w_scale, y, ld_y, glog, div_up(k, p.group), qa);
            return p.scale_stage == 1;
        }
        return false;
    }
    hipLaunchKernelGGL((k_w8a16_panel<AF, MB, CS, D, 4, AT, XS, RPW>), grid, dim3(4 * kWave), 0,
                       stream, x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y, 0,
                       (int64_t)0, qa);
    return true;
}

template <int AT>
static hipError_t dispatch(const W8A16Plan &p, const void *x, int64_t m, int64_t k,
                           int64_t ld_x, const float *x_scale, const uint8_t *w, int64_t n,
                           int64_t ld_w, const float *w_scale, uint16_t *y, int64_t ld_y,
                           void *workspace, const QuantArgs &qa, hipStream_t stream)
{
    float *partial = static_cast<float *>(workspace);
    if (p.kind == W8A16Plan::kPanel && (p.group == 0 || AT != kActQ)) {
#define FP8Q_PANEL_CASE(AF, MB, CS, D, XS)                                                    \
            if (p.af == AF && p.mb == MB && p.steps == CS && p.depth == D && p.waves == 4 &&    \
                p.xd == XS && p.rpw == 0) {                                                   \
                if (!launch_panel<AF, MB, CS, D, AT, XS>(p, x, m, k, ld_x, x_scale, w, n, ld_w,  \
                                                         w_scale, y, ld_y, qa, stream))       \
                    return hipErrorInvalidValue;                                              \
                return hipGetLastError();                                                     \
            }
#define FP8Q_PANEL_MB1(XS)                                                                    \
            FP8Q_PANEL_CASE(3, 1, 2, 3, XS) FP8Q_PANEL_CASE(4, 1, 2, 3, XS)                   \
            FP8Q_PANEL_CASE(7, 1, 2, 2, XS)
        if constexpr (AT == kActF8) {
            FP8Q_PANEL_CASE(1, 1, 2, 3, 16) FP8Q_PANEL_CASE(2, 1, 2, 3, 16) FP8Q_PANEL_MB1(16)
            FP8Q_PANEL_CASE(2, 1, 4, 3, 16)
            FP8Q_PANEL_CASE(2, 1, 4, 2, 16)
            FP8Q_PANEL_CASE(2, 2, 4, 2, 32)
            FP8Q_PANEL_CASE(4, 2, 2, 2, 32) FP8Q_PANEL_CASE(4, 2, 2, 1, 32)
        } else if constexpr (AT == kActQ) {
            // activations cast on the fly: stage (and cast) only the rows that exist
            FP8Q_PANEL_CASE(1, 1, 2, 3, 4) FP8Q_PANEL_CASE(2, 1, 2, 3, 4) FP8Q_PANEL_MB1(4)
            FP8Q_PANEL_CASE(1, 1, 2, 3, 8) FP8Q_PANEL_CASE(2, 1, 2, 3, 8) FP8Q_PANEL_MB1(8)
            FP8Q_PANEL_CASE(1, 1, 2, 3, 16) FP8Q_PANEL_CASE(2, 1, 2, 3, 16) FP8Q_PANEL_MB1(16)
        } else {
            FP8Q_PANEL_CASE(1, 1, 2, 4, 16) FP8Q_PANEL_CASE(2, 1, 2, 4, 16) FP8Q_PANEL_MB1(16)
            FP8Q_PANEL_CASE(2, 1, 2, 3, 16)
            FP8Q_PANEL_CASE(2, 2, 2, 2, 32)
            FP8Q_PANEL_CASE(4, 2, 2, 2, 32) FP8Q_PANEL_CASE(4, 2, 2, 1, 32)
        }
        if constexpr (AT != kActQ) {
            // a small weight: 4 activation rows per workgroup
            if (p.af == 1 && p.mb == 1 && p.steps == 4 && p.depth == 2 && p.waves == 4 &&
                p.xd == 4 && p.rpw == 4) {
                if (!launch_panel<1, 1, 4, 2, AT, 4, 4>(p, x, m, k, ld_x, x_scale, w, n, ld_w,
                                                        w_scale, y, ld_y, qa, stream))
                    return hipErrorInvalidValue;
                return hipGetLastError();
            }
        }
#undef FP8Q_PANEL_MB1
#undef FP8Q_PANEL_CASE
    } else if (p.group == 0 && p.kind == W8A16Plan::kRows) {
#define FP8Q_ROWS_CASE(AF, MB, P, NW)                                                         \
        if (p.af == AF && p.mb == MB && p.depth == P && p.waves == NW) {                      \
            launch_rows<AF, MB, P, NW, AT>(p, x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y,    \
                                           ld_y, workspace, qa, stream);                  \
            return hipGetLastError();                                                         \
        }
        FP8Q_ROWS_CASE(2, 1, 8, 4)
        FP8Q_ROWS_CASE(1, 1, 8, 4)
#undef FP8Q_ROWS_CASE
    } else if (p.group == 0) {
#define FP8Q_TILE_CASE(MB, XD, T)                                                             \
        if (p.mb == MB && p.xd == XD && p.steps == T) {                                       \
            launch_tile<MB, XD, T, AT>(p, x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y,  \
                                       partial, qa, stream);                                  \
            return hipGetLastError();                                                         \
        }
        FP8Q_TILE_CASE(1, 1, 8)
        FP8Q_TILE_CASE(1, 2, 8)
        FP8Q_TILE_CASE(1, 3, 8)
        FP8Q_TILE_CASE(1, 4, 8)
        FP8Q_TILE_CASE(1, 1, 16)
        FP8Q_TILE_CASE(1, 2, 16)
        FP8Q_TILE_CASE(1, 3, 16)
        FP8Q_TILE_CASE(1, 4, 16)
        FP8Q_TILE_CASE(2, 8, 8)
        FP8Q_TILE_CASE(3, 12, 8)
        FP8Q_TILE_CASE(4, 16, 8)
#undef FP8Q_TILE_CASE
    } else if constexpr (AT != kActQ) {
        // per-group weight scales (not with on-the-fly activation quantization)
        if (p.kind == W8A16Plan::kRows) {
#define FP8Q_GROUP_ROWS_CASE(AF, SPG)                                                         \
        if (p.af == AF && p.mb == 1 && p.depth == 8 && p.waves == 4 && p.group == 64 * SPG) {  \
            launch_rows<AF, 1, 8, 4, AT, SPG>(p, x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, \
                                              ld_y, workspace, qa, stream);                  \
            return hipGetLastError();                                                         \
        }
        FP8Q_GROUP_ROWS_CASE(1, 1) FP8Q_GROUP_ROWS_CASE(1, 2)
        FP8Q_GROUP_ROWS_CASE(1, 4) FP8Q_GROUP_ROWS_CASE(1, 8)
        FP8Q_GROUP_ROWS_CASE(2, 1) FP8Q_GROUP_ROWS_CASE(2, 2)
        FP8Q_GROUP_ROWS_CASE(2, 4) FP8Q_GROUP_ROWS_CASE(2, 8)
#undef FP8Q_GROUP_ROWS_CASE
        } else {
#define FP8Q_GROUP_CASE(MB, XD, T, SPG)                                                       \
        if (p.mb == MB && p.xd == XD && p.steps == T && p.group == 64 * SPG) {                \
            launch_tile<MB, XD, T, AT, SPG>(p, x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y,   \
                                            ld_y, partial, qa, stream);                       \
            return hipGetLastError();                                                         \
        }
#define FP8Q_GROUP_SIZES(MB, XD, T)                                                           \
        FP8Q_GROUP_CASE(MB, XD, T, 1) FP8Q_GROUP_CASE(MB, XD, T, 2)                           \
        FP8Q_GROUP_CASE(MB, XD, T, 4) FP8Q_GROUP_CASE(MB, XD, T, 8)
        FP8Q_GROUP_SIZES(1, 1, 8)
        FP8Q_GROUP_SIZES(1, 2, 8)
        FP8Q_GROUP_SIZES(1, 3, 8)
        FP8Q_GROUP_SIZES(1, 4, 8)
        FP8Q_GROUP_SIZES(1, 1, 16)
        FP8Q_GROUP_SIZES(1, 2, 16)
        FP8Q_GROUP_SIZES(1, 3, 16)
        FP8Q_GROUP_SIZES(1, 4, 16)
        FP8Q_GROUP_SIZES(2, 8, 8)
        FP8Q_GROUP_SIZES(3, 12, 8)
        FP8Q_GROUP_SIZES(4, 16, 8)
#undef FP8Q_GROUP_SIZES
#undef FP8Q_GROUP_CASE
        }
    }
    return hipErrorInvalidValue;
}

hipError_t w8a16(const W8A16Plan &p, int act, const void *x, int64_t m, int64_t k, int64_t ld_x,
                 const float *x_scale, const uint8_t *w, int64_t n, int64_t ld_w,
                 const float *w_scale, uint16_t *y, int64_t ld_y, void *workspace,
                 hipStream_t stream)
{
    const QuantArgs none{nullptr, 0, nullptr, nullptr};
    switch (act) {
    case kActBF16:
        return dispatch<kActBF16>(p, x, m, k, ld_x, nullptr, w, n, ld_w, w_scale, y, ld_y,
                                  workspace, none, stream);
    case kActF16:
        return dispatch<kActF16>(p, x, m, k, ld_x, nullptr, w, n, ld_w, w_scale, y, ld_y,
                                 workspace, none, stream);
    case kActF8:
        return dispatch<kActF8>(p, x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y,
                                workspace, none, stream);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t w8a16_quant_act(const W8A16Plan &p, const uint16_t *x, int64_t m, int64_t k,
                           int64_t ld_x, const uint32_t *act_part, int npart, float *x_scale_out,
                           int32_t *flag, const uint8_t *w, int64_t n, int64_t ld_w,
                           const float *w_scale, uint16_t *y, int64_t ld_y, void *workspace,
                           hipStream_t stream)
{
    // without maxima only the panel kernel (which scans x itself) applies
    if (p.group != 0 || (act_part == nullptr && p.kind != W8A16Plan::kPanel))
        return hipErrorInvalidValue;
    const QuantArgs qa{act_part, npart, x_scale_out, flag};
    return dispatch<kActQ>(p, x, m, k, ld_x, nullptr, w, n, ld_w, w_scale, y, ld_y, workspace, qa,
                           stream);
}

}  // namespace launch
}  // namespace fp8q
