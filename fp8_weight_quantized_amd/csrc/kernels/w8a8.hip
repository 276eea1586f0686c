// W8A8 ("fp8_w_fp8_a", the write-up "Llama 3 精读" §3.1 step 3): E4M3
// activations with one per-tensor scale, E4M3 weights with per-output-channel
// scales, bf16 output:
//   Y[m,n] = bf16_RNE( x_scale * w_scale[n] * sum_k dec(X[m,k]) * dec(W[n,k]) ).
//
// This is the prefill shape (thousands of tokens): the time is matrix-core
// compute.  Products of two E4M3 values are exact in fp32 and the sum is
// accumulated in fp32 by the MFMA; both scales are applied once, in the
// epilogue.
//
// Design (gfx950, 256 CUs in 8 XCDs, 160 KB LDS per CU):
//   * 256 x 256 output tile per workgroup of 8 waves (2 x 4); each wave owns a
//     128 x 64 sub-tile = 4 x 2 blocks of v_mfma_scale_f32_32x32x64_f8f6f4
//     (E4M3 x E4M3, unit E8M0 scales), 128 fp32 accumulators per lane;
//   * K advances 64 bytes per stage; X and W stage tiles are loaded with
//     16-byte global loads into registers, then written to LDS rows padded to
//     80 bytes (so the 16-byte fragment reads of 8 or 16 consecutive rows hit
//     distinct banks), double buffered: the global loads of stage s+1 are in
//     flight while stage s feeds the MFMAs, with one barrier per stage;
//   * the k order inside an MFMA is free as long as X and W use the same
//     one, so a lane simply takes 32 contiguous bytes of its row;
//   * tile order: consecutive workgroups are dealt round-robin to the 8 XCDs,
//     so the tile index is remapped to give each XCD a contiguous band of
//     tiles, grouped 8 tile-rows high so that concurrent tiles share X and W
//     panels in that XCD's L2.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;               // bytes (= k values) per stage
constexpr int kThreads = 512;        // 8 waves
constexpr int kWavesM = 2;
constexpr int kWavesN = 4;
constexpr int WM = BM / kWavesM;     // 128
constexpr int WN = BN / kWavesN;     // 64
constexpr int TM = WM / 32;          // 4 MFMA blocks along M per wave
constexpr int TN = WN / 32;          // 2 MFMA blocks along N per wave
constexpr int kRowBytes = BK + 16;   // padded LDS row
constexpr int kTileBytes = BM * kRowBytes;        // one operand, one stage (20 KB)
constexpr int kStageBytes = 2 * kTileBytes;       // X + W
constexpr int kLdsBytes = 2 * kStageBytes;        // double buffered (80 KB)
constexpr int kChunksPerRow = BK / 16;            // 16-byte chunks per stage row
constexpr int kLoadsPerThread = BM * kChunksPerRow / kThreads;   // 2 per operand
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

static_assert(BM == BN, "one loader layout serves both operands");
static_assert(kLoadsPerThread * kThreads == BM * kChunksPerRow, "loader covers the tile");

// 16 codes of a row at k index kc, zero past k (only on a K tail).
__device__ __forceinline__ uint4 load16_tail(const uint8_t *rowp, int64_t kc, int64_t k)
{
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        uint32_t b = (kc + e < k) ? (uint32_t)rowp[kc + e] : 0u;
        d[e >> 2] |= b << (8 * (e & 3));
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
}

struct TileLoader {
    const uint8_t *row[kLoadsPerThread];
    bool valid[kLoadsPerThread];
    int lds_off[kLoadsPerThread];
    int col[kLoadsPerThread];

    __device__ void init(const uint8_t *base, int64_t row0, int64_t rows, int64_t ld, int tid)
    {
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; ++i) {
            const int c = tid + i * kThreads;
            const int r = c / kChunksPerRow;
            col[i] = (c % kChunksPerRow) * 16;
            const int64_t gr = row0 + r;
            valid[i] = gr < rows;
            row[i] = base + (valid[i] ? gr : 0) * ld;
            lds_off[i] = r * kRowBytes + col[i];
        }
    }

    __device__ void load(uint4 *regs, int64_t k0, int64_t k, bool full_k) const
    {
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; ++i) {
            const int64_t kc = k0 + col[i];
            if (!valid[i])
                regs[i] = make_uint4(0u, 0u, 0u, 0u);
            else if (full_k || kc + 16 <= k)
                regs[i] = *reinterpret_cast<const uint4 *>(row[i] + kc);
            else if (kc < k)
                regs[i] = load16_tail(row[i], kc, k);
            else
                regs[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    __device__ void store(uint8_t *lds, const uint4 *regs) const
    {
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; ++i)
            *reinterpret_cast<uint4 *>(lds + lds_off[i]) = regs[i];
    }
};

__device__ __forceinline__ v8i lds_frag(const uint8_t *tile, int row, int half)
{
    const uint8_t *p = tile + row * kRowBytes + half * 32;
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    uint4 b = *reinterpret_cast<const uint4 *>(p + 16);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__global__ __launch_bounds__(kThreads, 1) void k_w8a8(
    const uint8_t *__restrict__ x, int64_t m, int64_t k, int64_t ld_x,
    const float *__restrict__ x_scale,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int tiles_m, int tiles_n)
{
    __shared__ __align__(16) uint8_t lds[kLdsBytes];

    // ---- tile order: XCD bands, then groups of kGroupM tile-rows ----------
    const int nblocks = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if (nblocks % kXcds == 0) {
        const int per_xcd = nblocks / kXcds;
        pid = (pid % kXcds) * per_xcd + pid / kXcds;
    }
    const int group = kGroupM * tiles_n;
    const int first_m = (pid / group) * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (pid % group) % gm;
    const int tn = (pid % group) / gm;

    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int wm = wave / kWavesN;
    const int wn = wave % kWavesN;
    const int lr = lane & 31;        // row of the MFMA operand this lane feeds
    const int lh = lane >> 5;        // which 32-byte half of the 64-byte k step

    TileLoader lx, lw;
    lx.init(x, m0, m, ld_x, tid);
    lw.init(w, n0, n, ld_w, tid);

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.f;

    const int64_t ksteps = (k + BK - 1) / BK;
    uint4 rx[kLoadsPerThread], rw[kLoadsPerThread];
    lx.load(rx, 0, k, BK <= k);
    lw.load(rw, 0, k, BK <= k);
    lx.store(lds, rx);
    lw.store(lds + kTileBytes, rw);
    __syncthreads();

    for (int64_t ks = 0; ks < ksteps; ++ks) {
        const int cur = (int)(ks & 1);
        const bool more = ks + 1 < ksteps;
        if (more) {
            const int64_t k0 = (ks + 1) * BK;
            const bool full = k0 + BK <= k;
            lx.load(rx, k0, k, full);
            lw.load(rw, k0, k, full);
        }
        const uint8_t *tx = lds + cur * kStageBytes;
        const uint8_t *tw = tx + kTileBytes;
        v8i bf[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bf[j] = lds_frag(tw, wn * WN + j * 32 + lr, lh);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const v8i af = lds_frag(tx, wm * WM + i * 32 + lr, lh);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af, bf[j], acc[i][j], 0, 0, 0, 127, 0, 127);
        }
        if (more) {
            uint8_t *nx = lds + (cur ^ 1) * kStageBytes;
            lx.store(nx, rx);
            lw.store(nx + kTileBytes, rw);
        }
        __syncthreads();
    }

    // ---- epilogue: D[i][j] at lane (col j = lane % 32), rows
    //      8 * (v / 4) + 4 * (lane / 32) + v % 4 of each 32 x 32 block --------
    const float xs = *x_scale;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + wn * WN + j * 32 + lr;
        if (col >= n)
            continue;
        const float s = xs * w_scale[col];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t rbase = m0 + wm * WM + i * 32 + 4 * lh;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t rr = rbase + 8 * (v / 4) + (v % 4);
                if (rr < m)
                    y[rr * ld_y + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v] * s);
            }
        }
    }
}

}  // namespace

namespace launch {

W8A8Plan plan_w8a8(int64_t m, int64_t n, int64_t k)
{
    (void)k;
    W8A8Plan p{};
    p.tiles_m = (m + BM - 1) / BM;
    p.tiles_n = (n + BN - 1) / BN;
    p.workspace = 0;
    return p;
}

hipError_t w8a8(const W8A8Plan &p, const uint8_t *x, int64_t m, int64_t k, int64_t ld_x,
                const float *x_scale, const uint8_t *w, int64_t n, int64_t ld_w,
                const float *w_scale, uint16_t *y, int64_t ld_y, hipStream_t stream)
{
    const int64_t blocks = p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL(k_w8a8, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y,
                       (int)p.tiles_m, (int)p.tiles_n);
    return hipGetLastError();
}

}  // namespace launch
}  // namespace fp8q
