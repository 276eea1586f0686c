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
//     128 x 64 sub-tile = 4 x 2 blocks of v_mfma_f32_32x32x64_f8f6f4 (E4M3 x
//     E4M3; the scaled builtin with zero scale operands selects the unscaled
//     instruction, about 2% faster here than unit E8M0 scales), 128 fp32
//     accumulators per lane, two waves per SIMD so one wave's LDS reads
//     overlap the other's MFMAs;
//   * the weights are the MFMA's A operand and the activations its B
//     operand, so the accumulator D holds Y^T: each lane ends up with runs of
//     4 consecutive output columns, stored as 8-byte bf16 packets;
//   * K advances 128 bytes per stage (two MFMA k-steps) through a 2-slot,
//     128 KB LDS ring filled by direct global->LDS loads
//     (global_load_lds_dwordx4) issued one stage ahead, with one barrier per
//     stage.  128-byte stages halve the barriers and waits per MFMA against
//     64-byte stages with a 4-slot ring (7% faster here).  The direct loads are issued from
//     inline assembly: the compiler cannot tell the ring slots apart, and if
//     it sees the loads it waits for every one of them before each LDS read,
//     which serializes the pipeline.  The kernel's own s_waitcnt (each wave
//     waits for its loads of the stage it is about to read) and barrier
//     provide the ordering instead;
//   * a direct load writes a wave's 64 lanes to 1 KB of consecutive LDS (8
//     rows of 128 bytes), so the bank-conflict-avoiding layout is an XOR
//     swizzle of the 16-byte chunks of each row, applied by choosing which
//     global chunk each lane fetches;
//   * the k order inside an MFMA is free as long as X and W use the same
//     one, so a lane simply takes 32 contiguous bytes of its row per k-step;
//   * tile order: consecutive workgroups are dealt round-robin to the 8 XCDs,
//     so the tile index is remapped to give each XCD a contiguous band of
//     tiles, grouped 8 tile-rows high so that concurrent tiles share X and W
//     panels in that XCD's L2.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {
namespace {

using namespace dev;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;              // bytes (= k values) per stage
constexpr int kStages = 2;           // LDS ring; loads run kStages-1 stages ahead
constexpr int kThreads = 512;        // 8 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kWavesM = 2;
constexpr int kWavesN = 4;
constexpr int WM = BM / kWavesM;     // 128 activation rows per wave
constexpr int WN = BN / kWavesN;     // 64 weight rows per wave
constexpr int TM = WM / 32;          // 4 MFMA blocks along M per wave
constexpr int TN = WN / 32;          // 2 MFMA blocks along N per wave
constexpr int kTileBytes = BM * BK;               // one operand, one stage (16 KB)
constexpr int kStageBytes = 2 * kTileBytes;       // X + W
constexpr int kLdsBytes = kStages * kStageBytes;  // 128 KB
constexpr int kRowsPerInst = kWave * 16 / BK;     // rows one wave load instruction fills (8)
constexpr int kInst = BM / kRowsPerInst / kWaves; // load instructions per operand per wave (4)
constexpr int kOps = 2 * kInst;                   // vector-memory operations per full stage
constexpr int kChunks = BK / 16;                  // 16-byte chunks per tile row
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

static_assert(BM == BN, "one loader layout serves both operands");
static_assert(kInst * kRowsPerInst * kWaves == BM, "loader covers the tile");

// LDS layout of a stage tile: rows of BK = 128 bytes; the eight 16-byte
// chunks of row r are stored at chunk positions c ^ swz(r).  gfx950 serves a
// ds_read_b128 16 lanes (256 bytes, all 64 banks) per clock, and a fragment
// read has 16 consecutive rows read the same logical chunk: rows r and r+1
// sit in different 128-byte halves of the bank space, and XOR-ing the chunk
// with (r >> 1) & 7 spreads the 8 rows of equal parity over the 8 chunk
// positions, so the 16 reads hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// 16 bytes of a row starting at k index kc, zero-filled at and past k.
__device__ __forceinline__ uint4 tail16(const uint8_t *rowp, int64_t kc, int64_t k)
{
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        uint32_t b = (kc + e < k) ? (uint32_t)rowp[kc + e] : 0u;
        d[e >> 2] |= b << (8 * (e & 3));
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// One operand's per-lane share of a stage load.  The wave fills 1 KB blocks
// (16 rows x 64 bytes) of the stage tile; lane l writes LDS slot l of a block,
// i.e. row l / 4 at chunk position l % 4, so it fetches logical chunk
// (l % 4) ^ swz(row).  Addresses are a wave-uniform base (the tile's first
// row) plus a 32-bit per-lane offset, to keep the register footprint small;
// a tile spans fewer than 2^31 bytes (256 rows x ld, checked by the host).
struct StageLoader {
    const uint8_t *base;          // row0 of the operand (uniform)
    uint32_t off[kInst];          // (row - row0) * ld + chunk offset; rows past the end clamp to row0
    uint32_t lds_off[kInst];      // wave-uniform LDS offset of the 1 KB block
    bool ok[kInst];               // row exists (only the register path needs it)

    __device__ void init(const uint8_t *mat, int64_t row0, int64_t rows, int64_t ld, int wave, int lane)
    {
        base = mat + row0 * ld;
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int blk = wave * kInst + i;
            const int r = blk * kRowsPerInst + lane / kChunks;
            ok[i] = row0 + r < rows;
            off[i] = (uint32_t)((ok[i] ? (int64_t)r * ld : 0) + ((lane % kChunks) ^ swz(r)) * 16);
            lds_off[i] = (uint32_t)(blk * kRowsPerInst * BK);
        }
    }

    // A stage wholly inside K: exactly kInst direct loads, which the caller's
    // wait counts rely on.  Rows past the end read their clamped row and only
    // feed outputs that are never stored.
    __device__ void load_full(uint32_t tile_lds, int64_t k0) const
    {
        const uint8_t *stage = base + k0;
#pragma unroll
        for (int i = 0; i < kInst; ++i)
            dma16(stage, off[i], tile_lds + lds_off[i]);
    }

    // The stage that crosses k goes through registers with zero fill (bytes
    // past k, and rows past the end, read 0).
    __device__ void load_tail(uint8_t *tile, int64_t k0, int64_t k, int wave, int lane) const
    {
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int r = (wave * kInst + i) * kRowsPerInst + lane / kChunks;
            const uint32_t kofs = ((lane % kChunks) ^ swz(r)) * 16;
            const int64_t kc = k0 + kofs;                    // this lane's logical chunk start
            const uint8_t *rowp = base + (off[i] - kofs);
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (ok[i] && kc < k)
                v = kc + 16 <= k ? *reinterpret_cast<const uint4 *>(rowp + kc) : tail16(rowp, kc, k);
            *reinterpret_cast<uint4 *>(tile + lds_off[i] + lane * 16) = v;
        }
    }
};

// The 32 bytes lane (r, half) feeds an MFMA: logical chunks 2*half, 2*half+1 of row r.
__device__ __forceinline__ v8i lds_frag(const uint8_t *tile, int r, int half, int sub)
{
    const uint8_t *rp = tile + r * BK;
    const int s = swz(r);
    const uint4 a = *reinterpret_cast<const uint4 *>(rp + ((4 * sub + 2 * half) ^ s) * 16);
    const uint4 b = *reinterpret_cast<const uint4 *>(rp + ((4 * sub + 2 * half + 1) ^ s) * 16);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// s_waitcnt immediate for "at most n vector-memory operations and no LDS
// operations outstanding" (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4 left at max, lgkmcnt 11:8 = 0).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

// Workgroup barrier without a memory fence.  __syncthreads() would wait for
// every outstanding global load (vmcnt(0)) -- including the prefetches of
// later stages -- so the pipeline uses an explicit s_waitcnt for the data it
// needs and this bare barrier; the "memory" clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// GS: per-group weight scales (the deployment guide §4.3), w_scale
// [n, ngroups] for groups of 128 << gshift k, so a group is a whole number of
// stages.  The accumulators then hold the running sum in units of the
// current group's scale: when stage ks opens group g, every accumulator of
// weight row n is multiplied by s[n][g-1] / s[n][g] before the stage's
// MFMAs add to it, and the epilogue multiplies by the last group's scale.  That is
// sum_g s_g * P_g with one accumulator set (a second set would not fit the
// register file next to the 256 x 256 tile).  The ratios use the hardware
// reciprocal (about 1 ulp); group scales come through a 4-slot LDS ring of
// the tile's 256 rows, loaded two stages ahead.  The two waves of a SIMD
// (waves w and w + 4, which own different halves of the tile's M) multiply at
// different times: the first half at the start of the stage that opens the
// group, the second at the end of the stage before it, after its MFMAs, so
// one wave's multiplies can overlap the other's MFMAs (2-3% faster with
// groups of 128 than both at the start of the stage).
template <bool GS>
__global__ __launch_bounds__(kThreads, 1) void k_w8a8(
    const uint8_t *__restrict__ x, int64_t m, int64_t k, int64_t ld_x,
    const float *__restrict__ x_scale,
    const uint8_t *__restrict__ w, int64_t n, int64_t ld_w,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ld_y,
    int tiles_m, int tiles_n, int64_t ngroups, int gshift)
{
    __shared__ __align__(16) uint8_t lds[kLdsBytes];
    __shared__ __align__(16) float gsc[GS ? 4 * BN : 4];
    // grouped: s[n][g-1] / s[n][g] of the tile's rows, slot g & 3
    __shared__ __align__(16) float gratio[GS ? 4 * BN : 4];
    // per-row scales: xs * w_scale[n] of the tile's 256 weight rows, fetched
    // into LDS before the main loop hides the load; read by the epilogue
    __shared__ __align__(16) float wsl[GS ? 4 : BN];

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
    // the wave index is uniform across the wave; saying so keeps the LDS
    // addresses of the direct loads in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int wm = wave / kWavesN;
    const int wn = wave % kWavesN;
    const int lr = lane & 31;        // row of the MFMA operand this lane feeds
    const int lh = lane >> 5;        // which 32-byte half of the 64-byte k step

    StageLoader lx, lw;
    lx.init(x, m0, m, ld_x, wave, lane);
    lw.init(w, n0, n, ld_w, wave, lane);
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);

    // acc[i][j] = D^T block: rows n (i-th 32-row block of the wave's W rows),
    // columns m (j-th 32-row block of the wave's X rows)
    v16f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.f;

    // grouped: the scale of tile row tid (< BN) for group g, loaded into a
    // register two stages ahead and written to LDS slot g & 3 before the
    // barrier of the stage before the one that opens group g (group 0 and the
    // group of stage 1 are loaded before the loop and written in stage 0)
    // Stage indices are 32-bit (K < 2^31) and group boundaries a shift and a
    // mask: 64-bit divisions here cost over a hundred scalar instructions
    // each, per stage and wave, on the scalar unit the CU's waves share.
    const int last_stage = (int)(k / BK) - (k % BK == 0 ? 1 : 0);
    const int gmask = (1 << gshift) - 1;
    const float *srow = w_scale + (GS ? min(n0 + tid, n - 1) * ngroups : 0);
    float pend = 0.f, prev = 0.f, pend0 = 0.f;
    int pend_g = -1;
    bool have0 = false;
    auto fetch_scale = [&](int st) {
        if constexpr (GS) {
            if (st <= last_stage && (st & gmask) == 0) {
                pend_g = st >> gshift;
                if (tid < BN)
                    pend = srow[pend_g];
            }
        }
    };
    auto store_scale = [&]() {
        if constexpr (GS) {
            if (have0) {
                if (tid < BN) {
                    gsc[tid] = pend0;
                    prev = pend0;
                }
                have0 = false;
            }
            if (pend_g >= 0) {
                if (tid < BN) {
                    gsc[(pend_g & 3) * BN + tid] = pend;
                    // the ratio each lane holding this row multiplies by
                    // when group pend_g opens (hardware reciprocal, ~1 ulp)
                    gratio[(pend_g & 3) * BN + tid] = prev * __builtin_amdgcn_rcpf(pend);
                    prev = pend;
                }
                pend_g = -1;
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));   // lgkmcnt(0): the write is done
        }
    };
    // stage st opens group g > 0: bring the accumulators from units of
    // s[g-1] to units of s[g] before the stage's MFMAs.  Lane (col, h) of a
    // 32 x 32 block holds rows 8 * q + 4 * h + e (e = 0..3) of W block i, so
    // one ratio serves the TM blocks of that row; the thread that stores a
    // row's group scale also stores its ratio, once per workgroup instead of
    // once per lane.  (Interleaving these multiplies with the stage's MFMAs
    // measured slower: each then waits for the previous stage's last MFMA
    // on its block, and the ratios held live cost 27 registers.)
    auto rescale = [&](int st) {
        if constexpr (GS) {
            if (st == 0 || (st & gmask) != 0)
                return;
            const int g = st >> gshift;
            const float *rt = gratio + (g & 3) * BN;
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = wn * WN + i * 32 + 8 * q + 4 * lh;
                    const float4 r4 = *reinterpret_cast<const float4 *>(rt + r);
                    const float ra[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                    for (int j = 0; j < TM; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j][4 * q + e] *= ra[e];
                }
        }
    };

    // after_first_reads runs once the stage's first activation fragments
    // have been read from LDS (the grouped kernel issues the next stage's
    // loads there)
    auto compute = [&](int st, auto after_first_reads) {
        if (!GS || wm == 0)
            rescale(st);
        const uint8_t *tx = lds + (int)(st % kStages) * kStageBytes;
        const uint8_t *tw = tx + kTileBytes;
#pragma unroll
        for (int sub = 0; sub < BK / 64; ++sub) {
            v8i xf[TM];
#pragma unroll
            for (int j = 0; j < TM; ++j)
                xf[j] = lds_frag(tx, wm * WM + j * 32 + lr, lh, sub);
            if (sub == 0)
                after_first_reads();
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const v8i wf = lds_frag(tw, wn * WN + i * 32 + lr, lh, sub);
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        wf, xf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
            }
        }
        if (GS && wm == 1 && st < last_stage)
            rescale(st + 1);
    };
    auto issue_full = [&](int st) {
        const uint32_t t = lds_base + (uint32_t)((st % kStages) * kStageBytes);
        lx.load_full(t, (int64_t)st * BK);
        lw.load_full(t + kTileBytes, (int64_t)st * BK);
    };

    // Full stages run through the ring, loaded kStages-1 stages ahead; a
    // partial last stage (k not a multiple of BK) is peeled off after the loop.
    const int nfull = (int)(k / BK);
    if constexpr (GS) {
        if (tid < BN)
            pend0 = srow[0];
        have0 = true;
        fetch_scale(1);
    }
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
        if (st < nfull)
            issue_full(st);
    // (its LDS write is visible after the first barrier of the loop; with K
    // under one stage, after the tail stage's barrier)
    if constexpr (!GS) {
        if (tid < BN)
            wsl[tid] = *x_scale * w_scale[min(n0 + tid, n - 1)];
    }

    for (int ks = 0; ks < nfull; ++ks) {
        // This wave's loads for stage ks have landed once no more than the
        // loads of the later stages already issued (up to kStages-2 of them,
        // exactly kOps each) are outstanding.  The barrier then makes every
        // wave's part of the stage visible, and guarantees that all waves are
        // done with stage ks-1, whose slot the next issue overwrites.
        const int later = min(kStages - 2, nfull - 1 - ks);
        if (later >= 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(2 * kOps));
        else if (later == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(kOps));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
        // (grouped: the scale load issued one stage earlier, or before the
        // loop, has landed with this wait; its LDS write goes before the
        // barrier)
        store_scale();
        barrier_no_fence();
        // grouped: the next stage's loads go out after this stage's first
        // fragment reads, and after the rescale where it comes first (5-6%
        // faster with groups of 128 than issuing them first; per channel 2.5%
        // slower, so there they go first)
        auto issue_next = [&] {
            if (ks + kStages - 1 < nfull)
                issue_full(ks + kStages - 1);
        };
        if constexpr (!GS)
            issue_next();
        fetch_scale(ks + 2);
        if constexpr (GS)
            compute(ks, issue_next);
        else
            compute(ks, [] {});
    }
    if (k % BK != 0) {
        // All direct loads have landed (the last loop iteration waited for
        // vmcnt(0)).  The partial stage's slot was last read by stage
        // nfull - kStages, finished by every wave before an earlier barrier;
        // this barrier also covers the reads of the last full stage.
        barrier_no_fence();
        uint8_t *t = lds + (int)(nfull % kStages) * kStageBytes;
        lx.load_tail(t, (int64_t)nfull * BK, k, wave, lane);
        lw.load_tail(t + kTileBytes, (int64_t)nfull * BK, k, wave, lane);
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
        store_scale();
        barrier_no_fence();
        compute(nfull, [] {});
    }

    // ---- epilogue.  In a 32 x 32 block, lane (col = lane % 32, h = lane / 32)
    // holds D rows 8 * (v / 4) + 4 * h + v % 4, v = 0..15.  D = Y^T here, so
    // the lane holds Y[m = col][n = ... + 4 consecutive]: 8 bytes in each of
    // 32 rows per store instruction, which measured at about 2.3 TB/s of
    // output (15 us per tile at M = 8192).  Instead the scaled bf16 tile is
    // staged row-major in the LDS ring, free once every wave is past its last
    // stage, and written out as whole rows: each lane stores 16 bytes and a
    // wave covers two 512-byte rows.  A staged row is 32 chunks of 16 bytes,
    // chunk c of row r stored at c ^ (r & 31), so the 32 rows of one write
    // instruction and the 32 chunks of one row's read spread over the banks.
    const float xs = *x_scale;
    // grouped: the last group's scales (every group's LDS write preceded a
    // barrier that every wave has passed)
    const float *slast = gsc + (GS ? ((last_stage >> gshift) & 3) * BN : 0);
    // xs * w_scale of output column nb + v
    auto wsc = [&](int64_t nb, int v) {
        if constexpr (GS)
            return xs * slast[nb - n0 + v];
        else
            return wsl[nb - n0 + v];
    };
    constexpr int kRowBytes = BN * 2;             // one staged output row (512 bytes)
    constexpr int kRowChunks = kRowBytes / 16;    // 32
    static_assert(BM * kRowBytes <= kLdsBytes, "the output tile fits the ring");
    auto out_off = [](int r, int c) { return r * kRowBytes + ((c ^ (r & (kRowChunks - 1))) * 16); };
    // every wave's reads of the last stage have returned before any wave
    // overwrites the ring (the direct loads all landed with the last vmcnt(0))
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));   // lgkmcnt(0)
    barrier_no_fence();
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int r = wm * WM + j * 32 + lr;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * WN + i * 32 + 8 * q + 4 * lh;   // multiple of 4
                const int64_t nb = n0 + nl;
                const v16f &a = acc[i][j];
                uint2 o;
                o.x = pack_bf16x2(a[4 * q + 0] * wsc(nb, 0), a[4 * q + 1] * wsc(nb, 1));
                o.y = pack_bf16x2(a[4 * q + 2] * wsc(nb, 2), a[4 * q + 3] * wsc(nb, 3));
                *reinterpret_cast<uint2 *>(lds + out_off(r, nl / 8) + (nl & 4) * 2) = o;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));   // lgkmcnt(0)
    barrier_no_fence();
    constexpr int kRowsPerPass = kThreads / kRowChunks;   // 16
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
            // non-temporal: the output (470 MB for Llama-3-8B gate+up at 8192
            // tokens) streams past the caches instead of evicting the X and W
            // panels later tiles re-read (about 5% at M = 8192)
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
bool w8a8_supports_ld(int64_t ld) { return ld > 0 && ld * BM < ((int64_t)1 << 31); }

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
                const float *w_scale, uint16_t *y, int64_t ld_y, hipStream_t stream,
                int64_t group)
{
    const int64_t blocks = p.tiles_m * p.tiles_n;
    if (group > 0) {
        // groups of 128 << gshift k (128, 256 or 512)
        const int gshift = group == BK ? 0 : group == 2 * BK ? 1 : group == 4 * BK ? 2 : -1;
        if (gshift < 0 || k >= ((int64_t)1 << 31))
            return hipErrorInvalidValue;
        const int64_t ngroups = (k + group - 1) / group;
        hipLaunchKernelGGL(k_w8a8<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y,
                           (int)p.tiles_m, (int)p.tiles_n, ngroups, gshift);
    } else {
        if (k >= ((int64_t)1 << 31))
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_w8a8<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           x, m, k, ld_x, x_scale, w, n, ld_w, w_scale, y, ld_y,
                           (int)p.tiles_m, (int)p.tiles_n, (int64_t)0, 0);
    }
    return hipGetLastError();
}

}  // namespace launch
}  // namespace fp8q
