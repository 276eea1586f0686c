// W8A16 ("fp8_w_bf16_a", the write-up "Llama 3 精读" §3.1 step 3): E4M3
// weights with a per-output-channel scale, bf16 activations, bf16 output:
//   Y[m,n] = bf16_RNE( w_scale[n] * sum_k X[m,k] * dec(W[n,k]) ).
//
// This is the decode shape (a handful of tokens): the time is the weight
// stream from HBM (the deployment guide, "FP8量化与长上下文实测", §3.3: at
// batch 1 FP8 and BF16 are within 10% of each other because bandwidth is the
// limit).  Every weight byte is read exactly once.
//
// Design (gfx950):
//   * one launch, no second pass: a workgroup owns R weight rows (R = 4, 8,
//     16 or 32, chosen so that N/R workgroups cover the 256 CUs) and the
//     whole K range; its waves split K between them and their fp32 partial
//     tiles are summed through LDS in wave order (deterministic);
//   * a lane streams 16 contiguous weight bytes per 64-k step with one
//     16-byte load straight into registers (non-temporal: weights are read
//     once, activations stay in L2); rows past N or past R are clamped to a
//     valid row and zeroed after the load, so every load is a plain
//     unconditional dwordx4;
//   * the codes are widened to bf16 in registers (exact) and fed to
//     v_mfma_f32_16x16x32_bf16 as the A operand, the activations as B, fp32
//     accumulation.  The k order inside an MFMA is free as long as both
//     operands use the same one, which lets one 16-byte weight load feed two
//     MFMAs and one 32-byte activation load match it.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;    // 4 waves split K

__device__ __forceinline__ v8bf as_v8bf(v4u v) { return __builtin_bit_cast(v8bf, v); }

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

// Widen a lane's 16 weight codes into the A operands of two MFMA k-steps.
__device__ __forceinline__ void widen(v4u wv, v8bf &a0, v8bf &a1)
{
    uint2 p0 = e4m3x4_to_bf16(wv.x), p1 = e4m3x4_to_bf16(wv.y);
    uint2 p2 = e4m3x4_to_bf16(wv.z), p3 = e4m3x4_to_bf16(wv.w);
    a0 = as_v8bf(v4u{p0.x, p0.y, p1.x, p1.y});
    a1 = as_v8bf(v4u{p2.x, p2.y, p3.x, p3.y});
}

// One 64-k step of a wave: widen the weight codes and issue the MFMAs.
// Rows past N (weights) or past M (activations) were clamped to a valid row
// when loading; they only feed output rows/columns that are never stored, so
// no masking is needed here.
template <int AF, int MB>
__device__ __forceinline__ void step_mfma(const v4u (&wv)[AF], const v4u (&xv)[MB][2],
                                          v4f (&acc)[AF][MB])
{
#pragma unroll
    for (int a = 0; a < AF; ++a) {
        v8bf a0, a1;
        widen(wv[a], a0, a1);
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_v8bf(xv[j][0]), acc[a][j], 0, 0, 0);
            acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_v8bf(xv[j][1]), acc[a][j], 0, 0, 0);
        }
    }
}

// AF: A fragments (16-row groups) per wave, so a block owns up to 16*AF rows;
// `rows` (<= 16*AF) is how many of them are real weight rows.
// MB: 16-column groups of activations (M <= 16*MB per block along grid.y).
// P:  pipeline depth -- 64-k steps whose loads are in flight while a step's
//     MFMAs run.  The pipelined span of a wave is a multiple of P steps; the
//     remaining steps (and a partial step at the end of K) run one by one.
template <int AF, int MB, int P>
__global__ __launch_bounds__(kThreads) void k_w8a16(
    const uint16_t *__restrict__ x, int64_t m, int64_t k, int64_t ld_x,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int rows, int64_t kchunk)
{
    constexpr int L = AF + 2 * MB;    // loads per step
    __shared__ v4f red[kThreads / kWave][AF * MB][kWave];

    const int nwaves = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int r = lane & 15;          // row of the A (weight) / B (activation) operand
    const int g = lane >> 4;          // which 16 k-values of a 64-k step this lane holds
    const int64_t n0 = (int64_t)blockIdx.x * rows;
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MB;
    const int64_t kb = min(k, (int64_t)wave * kchunk);
    const int64_t ke = min(k, kb + kchunk);

    const uint8_t *wp[AF];
#pragma unroll
    for (int a = 0; a < AF; ++a) {
        const int lr = 16 * a + r;
        const bool ok = lr < rows && n0 + lr < n;
        wp[a] = w + (ok ? n0 + lr : n0) * ld_w + 16 * g;
    }
    const uint16_t *xp[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const int64_t xr = m0 + 16 * j + r;
        xp[j] = x + (xr < m ? xr : m0) * ld_x + 16 * g;
    }

    v4f acc[2][AF][MB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int a = 0; a < AF; ++a)
#pragma unroll
            for (int j = 0; j < MB; ++j)
                acc[h][a][j] = v4f{0.f, 0.f, 0.f, 0.f};

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
                xb[u][j][0] = ldg(xp[j] + k0);
                xb[u][j][1] = ldg(xp[j] + k0 + 8);
            }
        };
        const int64_t kend = kb + 64 * npipe;
#pragma unroll
        for (int u = 0; u < P; ++u)
            issue(u, kb + 64 * u);
        __builtin_amdgcn_sched_barrier(0);
        for (; kk + 64 * P < kend; kk += 64 * P) {
            static_for<0, P>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                // loads retire in order: with (P-1) steps' loads still in
                // flight, step u's loads have landed
                wait_vmcnt<(P - 1) * L>();
                __builtin_amdgcn_sched_barrier(0);
                step_mfma<AF, MB>(wb[u], xb[u], acc[u & 1]);
                issue(u, kk + 64 * (P + u));
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        // last pipelined round: no more loads to issue
        static_for<0, P>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            wait_vmcnt<(P - 1 - u) * L>();
            __builtin_amdgcn_sched_barrier(0);
            step_mfma<AF, MB>(wb[u], xb[u], acc[u & 1]);
        });
        kk = kend;
    }
    // remaining steps one at a time; the last one may be partial (masked at k)
    for (; kk < ke; kk += 64) {
        const int64_t kw = kk + 16 * g;
        v4u wv[AF];
        v4u xv[MB][2];
        if (kk + 64 <= k) {
#pragma unroll
            for (int a = 0; a < AF; ++a)
                wv[a] = ldg(wp[a] + kk);
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                xv[j][0] = ldg(xp[j] + kk);
                xv[j][1] = ldg(xp[j] + kk + 8);
            }
        } else {
#pragma unroll
            for (int a = 0; a < AF; ++a)
                wv[a] = kw < k ? load_w16_tail(wp[a] - 16 * g, kw, k) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                xv[j][0] = kw < k ? load_x8_tail(xp[j] - 16 * g, kw, k) : v4u{0u, 0u, 0u, 0u};
                xv[j][1] = kw + 8 < k ? load_x8_tail(xp[j] - 16 * g, kw + 8, k) : v4u{0u, 0u, 0u, 0u};
            }
        }
        step_mfma<AF, MB>(wv, xv, acc[0]);
    }

    // ---- sum the waves' partial tiles in wave order, then scale and store --
#pragma unroll
    for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int j = 0; j < MB; ++j)
            red[wave][a * MB + j][lane] = acc[0][a][j] + acc[1][a][j];
    __syncthreads();

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
        for (int wv = 1; wv < nwaves; ++wv)
            sum += red[wv][f][sl];
        uint16_t *yp = y + mr * ld_y + nb;
        const int valid = (int)min<int64_t>(min<int64_t>(4, rows - nl), n - nb);
        if (valid == 4) {
            uint2 o;
            o.x = pack_bf16x2(sum[0] * w_scale[nb], sum[1] * w_scale[nb + 1]);
            o.y = pack_bf16x2(sum[2] * w_scale[nb + 2], sum[3] * w_scale[nb + 3]);
            *reinterpret_cast<uint2 *>(yp) = o;
        } else {
            for (int v = 0; v < valid; ++v)
                yp[v] = (uint16_t)f32_to_bf16_rne(sum[v] * w_scale[nb + v]);
        }
    }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Pipeline depth (64-k steps in flight per wave) for a tile shape: about 24-36
// outstanding 16-byte loads per lane, within the register budget.
constexpr int w8a16_depth(int af, int mb) { return (af + 2 * mb) <= 4 ? 8 : ((af + 2 * mb) <= 6 ? 4 : 2); }

namespace launch {

W8A16Plan plan_w8a16(int64_t m, int64_t n, int64_t k)
{
    W8A16Plan p{};
    const int64_t mgroups = div_up(m, 16);
    p.mb = (int)(mgroups >= 4 ? 4 : (mgroups < 1 ? 1 : mgroups));
    p.grid_m = div_up(m, 16 * p.mb);
    // rows per block: the most rows (up to 32) that still leave >= 256 blocks
    int rows = 32;
    while (rows > 4 && div_up(n, rows) * p.grid_m < 256)
        rows /= 2;
    if (rows == 32 && p.mb > 1)
        rows = 16;                       // keep the register pipeline within budget
    p.rows = rows;
    p.af = rows > 16 ? 2 : 1;
    p.grid_n = div_up(n, rows);
    // the 4 waves split K; a wave's range is a multiple of the pipelined span
    // (64 * depth) when K is large enough, else of 64
    p.waves = kThreads / kWave;
    const int64_t per = div_up(k, p.waves);
    const int64_t span = 64 * w8a16_depth(p.af, p.mb);
    p.kchunk = per >= span ? div_up(per, span) * span : div_up(per, 64) * 64;
    p.splits = 1;
    p.np = n;
    p.workspace = 0;
    return p;
}

template <int AF, int MB>
static void launch_t(const W8A16Plan &p, const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                     const uint8_t *w, int64_t n, int64_t ld_w, const float *w_scale,
                     uint16_t *y, int64_t ld_y, hipStream_t stream)
{
    constexpr int P = w8a16_depth(AF, MB);
    const dim3 grid((unsigned)p.grid_n, (unsigned)p.grid_m);
    hipLaunchKernelGGL((k_w8a16<AF, MB, P>), grid, dim3(kThreads), 0, stream, x, m, k,
                       ld_x, w, n, ld_w, w_scale, y, ld_y, p.rows, p.kchunk);
}

hipError_t w8a16(const W8A16Plan &p, const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                 const uint8_t *w, int64_t n, int64_t ld_w, const float *w_scale,
                 uint16_t *y, int64_t ld_y, float *partial, hipStream_t stream)
{
    (void)partial;
    if (p.af == 2) {
        launch_t<2, 1>(p, x, m, k, ld_x, w, n, ld_w, w_scale, y, ld_y, stream);
    } else {
        switch (p.mb) {
        case 1: launch_t<1, 1>(p, x, m, k, ld_x, w, n, ld_w, w_scale, y, ld_y, stream); break;
        case 2: launch_t<1, 2>(p, x, m, k, ld_x, w, n, ld_w, w_scale, y, ld_y, stream); break;
        case 3: launch_t<1, 3>(p, x, m, k, ld_x, w, n, ld_w, w_scale, y, ld_y, stream); break;
        default: launch_t<1, 4>(p, x, m, k, ld_x, w, n, ld_w, w_scale, y, ld_y, stream); break;
        }
    }
    return hipGetLastError();
}

}  // namespace launch
}  // namespace fp8q
