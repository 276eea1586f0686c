// Prefill GEMM for the 16-bit activation modes of the write-up ("Llama 3
// 精读" §3.1 step 3): fp8_w_fp16_a (fp16 activations, fp16 output) and
// fp8_w_bf16_a (bf16 activations, bf16 output), E4M3 weights with one scale
// per output channel (the deployment guide, "FP8量化与长上下文实测", §1.2):
//   Y[m,n] = out_RNE( w_scale[n] * sum_k X[m,k] * dec(W[n,k]) ).
//
// At prefill sizes the time is matrix-core work, so W is widened in registers
// to the activation type (exact: every E4M3 value is a 16-bit float) and fed
// to the 16-bit MFMA, v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulation; the
// weight scale is applied once, in the epilogue.
//
// Design (gfx950, 256 CUs in 8 XCDs, 160 KB LDS per CU):
//   * 256 x 256 output tile per workgroup of 8 waves (2 x 4); each wave owns a
//     128 x 64 sub-tile = 4 x 2 blocks of 32 x 32, 128 fp32 accumulators per
//     lane; the weights are the MFMA's A operand and the activations its B
//     operand, so the accumulator holds Y^T;
//   * K advances 64 values per stage: a 32 KB activation tile (256 rows of
//     128 bytes) and a 16 KB code tile (256 rows of 64 bytes), filled by
//     direct global->LDS loads two stages ahead through a 3-slot, 144 KB ring,
//     one barrier per stage;
//   * the k order inside an MFMA is free as long as both operands use the same
//     one: a lane takes 16 contiguous k values of its row per pair of MFMA
//     k-steps (32 bytes of activations, 16 bytes of codes);
//   * LDS rows are XOR-swizzled in 16-byte chunks so that the 16 lanes a
//     ds_read_b128 serves per clock hit 16 distinct bank groups: chunk c of a
//     128-byte row r sits at c ^ ((r >> 1) & 7), of a 64-byte row at
//     c ^ ((r >> 2) & 3) (four rows share one 256-byte bank line there);
//   * tile order and epilogue as the FP8 GEMM: XCD-banded tiles grouped 8
//     tile-rows high, and the scaled output tile staged row-major in the ring
//     and written as whole 512-byte rows with non-temporal stores.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BKV = 64;                          // k values per stage
constexpr int kStages = 3;                       // LDS ring; loads run kStages-1 stages ahead
constexpr int kThreads = 512;                    // 8 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kWavesM = 2;
constexpr int kWavesN = 4;
constexpr int WM = BM / kWavesM;                 // 128 activation rows per wave
constexpr int WN = BN / kWavesN;                 // 64 weight rows per wave
constexpr int TM = WM / 32;
constexpr int TN = WN / 32;
constexpr int kXRow = 2 * BKV;                   // bytes of an activation tile row (128)
constexpr int kWRow = BKV;                       // bytes of a code tile row (64)
constexpr int kXTile = BM * kXRow;               // 32 KB
constexpr int kWTile = BN * kWRow;               // 16 KB
constexpr int kStageBytes = kXTile + kWTile;     // 48 KB
constexpr int kLdsBytes = kStages * kStageBytes; // 144 KB
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

// LDS chunk position of logical 16-byte chunk c of row r, for RB-byte rows.
template <int RB>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (RB == 128)
        return (r >> 1) & 7;
    else
        return (r >> 2) & 3;
}

// One operand's per-lane share of a stage: RB-byte tile rows, ES bytes per
// value.  A wave instruction fills 1 KB of LDS (1024 / RB rows); lane l
// writes slot l, i.e. row l / (RB / 16) at chunk position l % (RB / 16), so it
// fetches logical chunk (l % (RB / 16)) ^ swz(row).
template <int RB, int ES>
struct Loader {
    static constexpr int kChunks = RB / 16;
    static constexpr int kRowsPerInst = kWave / kChunks;
    static constexpr int kInst = BM / kRowsPerInst / kWaves;
    static_assert(kInst * kRowsPerInst * kWaves == BM, "loader covers the tile");

    const uint8_t *base;          // the tile's first row (uniform)
    uint32_t off[kInst];          // (row - row0) * ld bytes + chunk offset; rows past the end clamp to row0
    uint32_t lds_off[kInst];      // wave-uniform LDS offset of the 1 KB block
    bool ok[kInst];

    __device__ void init(const uint8_t *mat, int64_t row0, int64_t rows, int64_t ld_bytes,
                         int wave, int lane)
    {
        base = mat + row0 * ld_bytes;
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int blk = wave * kInst + i;
            const int r = blk * kRowsPerInst + lane / kChunks;
            ok[i] = row0 + r < rows;
            off[i] = (uint32_t)((ok[i] ? (int64_t)r * ld_bytes : 0) +
                                ((lane % kChunks) ^ swz<RB>(r)) * 16);
            lds_off[i] = (uint32_t)(blk * kRowsPerInst * RB);
        }
    }

    // a stage wholly inside K: exactly kInst direct loads (the wait counts
    // rely on it); rows past the end read their clamped row and only feed
    // outputs that are never stored
    __device__ void load_full(uint32_t tile_lds, int64_t k0) const
    {
        const uint8_t *stage = base + k0 * ES;
#pragma unroll
        for (int i = 0; i < kInst; ++i)
            dma16(stage, off[i], tile_lds + lds_off[i]);
    }

    // the stage that crosses k, through registers: values at and past k, and
    // rows past the end, read 0
    __device__ void load_tail(uint8_t *tile, int64_t k0, int64_t k, int wave, int lane) const
    {
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int r = (wave * kInst + i) * kRowsPerInst + lane / kChunks;
            const uint32_t cofs = ((lane % kChunks) ^ swz<RB>(r)) * 16;
            const int64_t kc = k0 + cofs / ES;                 // first k value of this chunk
            const uint8_t *rowp = base + (off[i] - cofs);
            uint32_t d[4] = {0u, 0u, 0u, 0u};
            if (ok[i]) {
                if (kc + 16 / ES <= k) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(rowp + kc * ES);
                    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
                } else {
                    for (int e = 0; e < 16 / ES; ++e)
                        if (kc + e < k) {
                            uint32_t val = ES == 2 ? (uint32_t)reinterpret_cast<const uint16_t *>(rowp)[kc + e]
                                                   : (uint32_t)rowp[kc + e];
                            d[(e * ES) >> 2] |= val << (8 * ((e * ES) & 3));
                        }
                }
            }
            *reinterpret_cast<uint4 *>(tile + lds_off[i] + lane * 16) = make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
};

// The 16-bit activation types: MFMA operand, exact widening of 4 E4M3 codes,
// the 32x32x16 MFMA and the RNE output conversion.
template <bool F16> struct T16;
template <> struct T16<true> {
    typedef v8h frag;
    static __device__ __forceinline__ uint2 widen4(uint32_t codes)
    {
        const v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, 1.0f, false);
        const v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, 1.0f, true);
        return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
    static __device__ __forceinline__ v16f mfma(frag a, frag b, v16f c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    }
};
template <> struct T16<false> {
    typedef v8bf frag;
    static __device__ __forceinline__ uint2 widen4(uint32_t codes) { return e4m3x4_to_bf16(codes); }
    static __device__ __forceinline__ v16f mfma(frag a, frag b, v16f c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
};

// s_waitcnt immediate: at most n vector-memory operations and no LDS
// operations outstanding (vmcnt bits 3:0 and 15:14, expcnt 6:4 at max,
// lgkmcnt 11:8 = 0).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

template <bool F16>
__global__ __launch_bounds__(kThreads, 1) void k_w8a16_gemm(
    const uint16_t *__restrict__ x, int64_t m, int64_t k, int64_t ld_x,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int tiles_m, int tiles_n)
{
    typedef T16<F16> T;
    typedef Loader<kXRow, 2> XLoader;
    typedef Loader<kWRow, 1> WLoader;
    constexpr int kOps = XLoader::kInst + WLoader::kInst;   // direct loads per wave per stage
    __shared__ __align__(16) uint8_t lds[kLdsBytes];
    __shared__ __align__(16) float wsl[BN];

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
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int wm = wave / kWavesN;
    const int wn = wave % kWavesN;
    const int lr = lane & 31;        // row of the MFMA operand this lane feeds
    const int lh = lane >> 5;        // which 16 k values of a 32-k pair of MFMA steps

    XLoader lx;
    WLoader lw;
    lx.init(reinterpret_cast<const uint8_t *>(x), m0, m, ld_x * 2, wave, lane);
    lw.init(w, n0, n, ld_w, wave, lane);
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);

    v16f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.f;

    auto compute = [&](int64_t st) {
        const uint8_t *tx = lds + (int)(st % kStages) * kStageBytes;
        const uint8_t *tw = tx + kXTile;
#pragma unroll
        for (int sub = 0; sub < BKV / 32; ++sub) {
            // activations: k [32 sub + 16 lh, +16) of each of the wave's rows,
            // two 16-byte chunks = the B operands of two MFMA k-steps
            typename T::frag xf[TM][2];
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int r = wm * WM + j * 32 + lr;
                const uint8_t *rp = tx + r * kXRow;
                const int c0 = 4 * sub + 2 * lh;
                const v4u a = *reinterpret_cast<const v4u *>(rp + (c0 ^ swz<kXRow>(r)) * 16);
                const v4u b = *reinterpret_cast<const v4u *>(rp + ((c0 + 1) ^ swz<kXRow>(r)) * 16);
                xf[j][0] = __builtin_bit_cast(typename T::frag, a);
                xf[j][1] = __builtin_bit_cast(typename T::frag, b);
            }
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                // codes of the same 16 k values, widened exactly
                const int r = wn * WN + i * 32 + lr;
                const int c = 2 * sub + lh;
                const v4u cw = *reinterpret_cast<const v4u *>(tw + r * kWRow + (c ^ swz<kWRow>(r)) * 16);
                const uint2 p0 = T::widen4(cw.x), p1 = T::widen4(cw.y);
                const uint2 p2 = T::widen4(cw.z), p3 = T::widen4(cw.w);
                const typename T::frag w0 = __builtin_bit_cast(typename T::frag, v4u{p0.x, p0.y, p1.x, p1.y});
                const typename T::frag w1 = __builtin_bit_cast(typename T::frag, v4u{p2.x, p2.y, p3.x, p3.y});
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    acc[i][j] = T::mfma(w0, xf[j][0], acc[i][j]);
                    acc[i][j] = T::mfma(w1, xf[j][1], acc[i][j]);
                }
            }
        }
    };
    auto issue_full = [&](int64_t st) {
        const uint32_t t = lds_base + (uint32_t)((st % kStages) * kStageBytes);
        lx.load_full(t, st * BKV);
        lw.load_full(t + kXTile, st * BKV);
    };

    const int64_t nfull = k / BKV;
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
        if (st < nfull)
            issue_full(st);
    if (tid < BN)
        wsl[tid] = w_scale[min(n0 + tid, n - 1)];

    for (int64_t ks = 0; ks < nfull; ++ks) {
        // this wave's loads of stage ks have landed once only the later stages
        // already issued (up to kStages-2, kOps loads each) are outstanding; the
        // barrier makes every wave's part visible and ends all reads of the
        // slot the next issue overwrites (stage ks-1)
        const int64_t later = min<int64_t>(kStages - 2, nfull - 1 - ks);
        if (later >= 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(kOps));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
        barrier_no_fence();
        if (ks + kStages - 1 < nfull)
            issue_full(ks + kStages - 1);
        compute(ks);
    }
    if (k % BKV != 0) {
        // every direct load has landed (the last iteration waited for
        // vmcnt(0)); the tail's slot was last read by stage nfull - kStages,
        // and this barrier also covers the reads of the last full stage
        barrier_no_fence();
        uint8_t *t = lds + (int)(nfull % kStages) * kStageBytes;
        lx.load_tail(t, nfull * BKV, k, wave, lane);
        lw.load_tail(t + kXTile, nfull * BKV, k, wave, lane);
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
        barrier_no_fence();
        compute(nfull);
    }

    // ---- epilogue: lane (col = lane % 32, h = lane / 32) of a 32 x 32 block
    // holds D rows 8 (v / 4) + 4 h + v % 4; D = Y^T, so 4 consecutive output
    // columns of row m = col.  The scaled tile is staged row-major in the ring
    // (chunk c of row r at c ^ (r & 31)) and written as whole rows.
    constexpr int kRowBytes = BN * 2;
    constexpr int kRowChunks = kRowBytes / 16;
    static_assert(BM * kRowBytes <= kLdsBytes, "the output tile fits the ring");
    auto out_off = [](int r, int c) { return r * kRowBytes + ((c ^ (r & (kRowChunks - 1))) * 16); };
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));   // lgkmcnt(0)
    barrier_no_fence();
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int r = wm * WM + j * 32 + lr;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * WN + i * 32 + 8 * q + 4 * lh;
                const v16f &a = acc[i][j];
                uint2 o;
                o.x = T::pack2(a[4 * q + 0] * wsl[nl + 0], a[4 * q + 1] * wsl[nl + 1]);
                o.y = T::pack2(a[4 * q + 2] * wsl[nl + 2], a[4 * q + 3] * wsl[nl + 3]);
                *reinterpret_cast<uint2 *>(lds + out_off(r, nl / 8) + (nl & 4) * 2) = o;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));   // lgkmcnt(0)
    barrier_no_fence();
    constexpr int kRowsPerPass = kThreads / kRowChunks;
    const int c = tid % kRowChunks;
#pragma unroll 4
    for (int r = tid / kRowChunks; r < BM; r += kRowsPerPass) {
        const int64_t mr = m0 + r;
        const int64_t nb = n0 + 8 * c;
        if (mr >= m || nb >= n)
            continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(lds + out_off(r, c));
        uint16_t *yp = y + mr * ld_y + nb;
        if (nb + 8 <= n) {
            __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u *>(yp));
        } else {
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < (int)(n - nb); ++e)
                yp[e] = (uint16_t)(d[e >> 1] >> (16 * (e & 1)));
        }
    }
}

}  // namespace

namespace launch {

// Per-lane load offsets are 32-bit: a 256-row tile must span < 2^31 bytes.
bool w8a16_gemm_supports(int64_t ld_x, int64_t ld_w)
{
    return ld_x > 0 && ld_w > 0 && ld_x * 2 * BM < ((int64_t)1 << 31) &&
           ld_w * BN < ((int64_t)1 << 31);
}

hipError_t w8a16_gemm(bool f16, const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                      const uint8_t *w, int64_t n, int64_t ld_w, const float *w_scale,
                      uint16_t *y, int64_t ld_y, hipStream_t stream)
{
    const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    if (f16)
        hipLaunchKernelGGL(k_w8a16_gemm<true>, grid, dim3(kThreads), 0, stream, x, m, k, ld_x, w, n,
                           ld_w, w_scale, y, ld_y, (int)tiles_m, (int)tiles_n);
    else
        hipLaunchKernelGGL(k_w8a16_gemm<false>, grid, dim3(kThreads), 0, stream, x, m, k, ld_x, w,
                           n, ld_w, w_scale, y, ld_y, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace launch
}  // namespace fp8q
