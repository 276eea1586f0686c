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
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 16;

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

__device__ __forceinline__ v4u mask(v4u v, bool keep) { return keep ? v : v4u{0u, 0u, 0u, 0u}; }

// Widen a lane's 16 weight codes into the A operands of two MFMA k-steps.
__device__ __forceinline__ void widen(v4u wv, v8bf &a0, v8bf &a1)
{
    uint2 p0 = e4m3x4_to_bf16(wv.x), p1 = e4m3x4_to_bf16(wv.y);
    uint2 p2 = e4m3x4_to_bf16(wv.z), p3 = e4m3x4_to_bf16(wv.w);
    a0 = as_v8bf(v4u{p0.x, p0.y, p1.x, p1.y});
    a1 = as_v8bf(v4u{p2.x, p2.y, p3.x, p3.y});
}

// AF: A fragments (16-row groups) per wave, so a block owns up to 16*AF rows;
// `rows` (<= 16*AF) is how many of them are real weight rows.
// MB: 16-column groups of activations (M <= 16*MB per block along grid.y).
// UNR: 64-k steps whose loads are issued together.
template <int AF, int MB, int UNR>
__global__ __launch_bounds__(1024) void k_w8a16(
    const uint16_t *__restrict__ x, int64_t m, int64_t k, int64_t ld_x,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int rows, int64_t kchunk)
{
    __shared__ v4f red[kMaxWaves][AF * MB][kWave];

    const int nwaves = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int r = lane & 15;          // row of the A (weight) / B (activation) operand
    const int g = lane >> 4;          // which 16 k-values of a 64-k step this lane holds
    const int64_t n0 = (int64_t)blockIdx.x * rows;
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MB;
    const int64_t kb = (int64_t)wave * kchunk;
    const int64_t ke = min(k, kb + kchunk);

    const uint8_t *wp[AF];
    bool wvalid[AF];
#pragma unroll
    for (int a = 0; a < AF; ++a) {
        const int lr = 16 * a + r;
        wvalid[a] = lr < rows && n0 + lr < n;
        wp[a] = w + (wvalid[a] ? n0 + lr : n0) * ld_w;
    }
    const uint16_t *xp[MB];
    bool xvalid[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const int64_t xr = m0 + 16 * j + r;
        xvalid[j] = xr < m;
        xp[j] = x + (xvalid[j] ? xr : m0) * ld_x;
    }

    v4f acc[AF][MB];
#pragma unroll
    for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int j = 0; j < MB; ++j)
            acc[a][j] = v4f{0.f, 0.f, 0.f, 0.f};

    int64_t kk = kb;
    for (; kk + 64 * UNR <= ke; kk += 64 * UNR) {
        v4u wv[UNR][AF];
        v4u xv[UNR][MB][2];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t kw = kk + 64 * u + 16 * g;
#pragma unroll
            for (int a = 0; a < AF; ++a)
                wv[u][a] = ldg_nt(wp[a] + kw);
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                xv[u][j][0] = ldg(xp[j] + kw);
                xv[u][j][1] = ldg(xp[j] + kw + 8);
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            v8bf b0[MB], b1[MB];
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                b0[j] = as_v8bf(mask(xv[u][j][0], xvalid[j]));
                b1[j] = as_v8bf(mask(xv[u][j][1], xvalid[j]));
            }
#pragma unroll
            for (int a = 0; a < AF; ++a) {
                v8bf a0, a1;
                widen(mask(wv[u][a], wvalid[a]), a0, a1);
#pragma unroll
                for (int j = 0; j < MB; ++j) {
                    acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0[j], acc[a][j], 0, 0, 0);
                    acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1[j], acc[a][j], 0, 0, 0);
                }
            }
        }
    }
    // remainder steps, masked at k
    for (; kk < ke; kk += 64) {
        const int64_t kw = kk + 16 * g;
        const bool full = kw + 16 <= k;
        v8bf b0[MB], b1[MB];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            v4u x0 = v4u{0u, 0u, 0u, 0u}, x1 = x0;
            if (full) {
                x0 = ldg(xp[j] + kw);
                x1 = ldg(xp[j] + kw + 8);
            } else if (kw < k) {
                x0 = load_x8_tail(xp[j], kw, k);
                x1 = load_x8_tail(xp[j], kw + 8, k);
            }
            b0[j] = as_v8bf(mask(x0, xvalid[j]));
            b1[j] = as_v8bf(mask(x1, xvalid[j]));
        }
#pragma unroll
        for (int a = 0; a < AF; ++a) {
            v4u wv = v4u{0u, 0u, 0u, 0u};
            if (full)
                wv = ldg(wp[a] + kw);
            else if (kw < k)
                wv = load_w16_tail(wp[a], kw, k);
            v8bf a0, a1;
            widen(mask(wv, wvalid[a]), a0, a1);
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0[j], acc[a][j], 0, 0, 0);
                acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1[j], acc[a][j], 0, 0, 0);
            }
        }
    }

    // ---- sum the waves' partial tiles in wave order, then scale and store --
#pragma unroll
    for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int j = 0; j < MB; ++j)
            red[wave][a * MB + j][lane] = acc[a][j];
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
        v4f s = red[0][f][sl];
        for (int wv = 1; wv < nwaves; ++wv)
            s += red[wv][f][sl];
        uint16_t *yp = y + mr * ld_y + nb;
        const int valid = (int)min<int64_t>(min<int64_t>(4, rows - nl), n - nb);
        if (valid == 4) {
            uint2 o;
            o.x = pack_bf16x2(s[0] * w_scale[nb], s[1] * w_scale[nb + 1]);
            o.y = pack_bf16x2(s[2] * w_scale[nb + 2], s[3] * w_scale[nb + 3]);
            *reinterpret_cast<uint2 *>(yp) = o;
        } else {
            for (int v = 0; v < valid; ++v)
                yp[v] = (uint16_t)f32_to_bf16_rne(s[v] * w_scale[nb + v]);
        }
    }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

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
    if (rows == 32 && p.mb > 2)
        rows = 16;                       // keep the LDS reduction buffer <= 64 KB
    p.rows = rows;
    p.af = rows > 16 ? 2 : 1;
    p.grid_n = div_up(n, rows);
    // waves split K, each taking a multiple of 64 and at least 256 k values
    int64_t waves = div_up(k, 256);
    if (waves > kMaxWaves)
        waves = kMaxWaves;
    if (waves < 1)
        waves = 1;
    p.kchunk = div_up(div_up(k, waves), 64) * 64;
    p.waves = (int)div_up(k, p.kchunk);
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
    constexpr int UNR = (AF * 1 + MB * 2) <= 4 ? 4 : 2;
    const dim3 grid((unsigned)p.grid_n, (unsigned)p.grid_m);
    hipLaunchKernelGGL((k_w8a16<AF, MB, UNR>), grid, dim3(64 * p.waves), 0, stream, x, m, k,
                       ld_x, w, n, ld_w, w_scale, y, ld_y, p.rows, p.kchunk);
}

hipError_t w8a16(const W8A16Plan &p, const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                 const uint8_t *w, int64_t n, int64_t ld_w, const float *w_scale,
                 uint16_t *y, int64_t ld_y, float *partial, hipStream_t stream)
{
    (void)partial;
    if (p.af == 2) {
        switch (p.mb) {
        case 1: launch_t<2, 1>(p, x, m, k, ld_x, w, n, ld_w, w_scale, y, ld_y, stream); break;
        default: launch_t<2, 2>(p, x, m, k, ld_x, w, n, ld_w, w_scale, y, ld_y, stream); break;
        }
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
