// Internal launchers of the fp8q kernels (host side).  Each returns the HIP
// error of its launches; argument validation happens before, in the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8q {

// Upper bound on the blocks of the activation passes (also the number of
// partial maxima kept in the workspace).
constexpr int kActMaxBlocks = 1024;

// The allocation-free linear layer's device scratch: 8 MiB per GPU, which
// holds the K-split partial tiles of the Llama-3 8B/70B decode shapes (at
// most 5.5 MB, the 70B gate/up projection at 12 rows).
constexpr size_t kNoallocScratchBytes = (size_t)8 << 20;
constexpr int kNoallocMaxDevices = 64;

namespace launch {

hipError_t quantize_weight(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                           uint8_t *q, int64_t ld_q, float *scale, int32_t *flag,
                           hipStream_t stream);

int act_blocks(int64_t m, int64_t k);
// The absmax pass alone: act_blocks(m, k) maxima |x| (as bf16 magnitude keys)
// into partial.
hipError_t act_amax(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x, uint32_t *partial,
                    hipStream_t stream);
hipError_t quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                        uint8_t *q, int64_t ld_q, float *x_scale, uint32_t *partial,
                        int32_t *flag, hipStream_t stream);

// Per-group weight quantization: scale [n, ceil(k / group)], group 64..512
// (a power of two).
hipError_t quantize_weight_grouped(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                                   int64_t group, uint8_t *q, int64_t ld_q, float *scale,
                                   int32_t *flag, hipStream_t stream);

// Per-tensor quantization with a held scale (*scale, device), one pass.
hipError_t quantize_act_static(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                               const float *scale, uint8_t *q, int64_t ld_q, int32_t *flag,
                               hipStream_t stream);

// EMA-scaled quantization.  seed: the dynamic quantization, whose scale also
// goes to *state.  Otherwise the cast uses *state (and reports it in
// *x_scale), then a one-workgroup kernel steps *state towards this tensor's
// dynamic scale.  partial: act_blocks(m, k) words of scratch.
hipError_t quantize_act_ema(const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                            uint8_t *q, int64_t ld_q, float *x_scale, float *state,
                            float decay, float temperature, bool seed, uint32_t *partial,
                            int32_t *flag, hipStream_t stream);

hipError_t cast_f32(const float *x, int64_t count, uint8_t *out, hipStream_t stream);

// ---- FP8 KV cache ------------------------------------------------------------
// Blocks per tensor of the KV kernels (the workspace holds 2 * that many words).
int kv_blocks(int64_t tokens, int64_t heads, int64_t head_dim);
hipError_t kv_cache_write(const uint16_t *k, const uint16_t *v, int64_t tokens, int64_t heads,
                          int64_t head_dim, int64_t ld, const int64_t *slot, uint8_t *k_cache,
                          uint8_t *v_cache, int64_t slots, float *running, float *scale_out,
                          bool calibrate, uint32_t *partial, int32_t *flags, hipStream_t stream);

// ---- W8A16 (fp8_w_bf16_a) skinny GEMM --------------------------------------
struct W8A16Plan {
    enum Kind { kRows = 0, kTile = 1, kPanel = 2 };
    int kind;
    int mb;            // 16-row activation groups per workgroup (1..4)
    int64_t grid_m;    // workgroups along M (16 * mb activation rows each)
    int64_t grid_n;    // workgroups along N (times the K splits for the tile kernel)
    // k_w8a16_rows
    int rows;          // weight rows per workgroup (4, 8, 16 or 32)
    int af;            // 16-row MFMA fragments per wave (2 when rows == 32)
    int waves;         // waves per workgroup; they split K
    int depth;         // 64-k steps of loads in flight per wave
    int64_t kchunk;    // K range per wave
    // k_w8a16_tile (and k_w8a16_panel: steps, and depth = chunks in flight)
    int xd;            // activation rows each of the 4 waves stages per chunk
    int steps;         // 64-k steps per staged chunk
    int64_t tiles_n;   // tiles of 64 weight rows
    // both kernels (+ k_w8a16_reduce when splits > 1)
    int64_t splits;    // K splits across workgroups
    int64_t kper;      // K range per split (a multiple of 64)
    int64_t ldp;       // row stride of the fp32 partial tiles (n rounded up to 4)
    size_t workspace;  // scratch bytes: the partial tiles [splits][m][ldp] (0 if no split)
    int64_t group;     // 0: one weight scale per row; else k per weight-scale group
    int rpw;           // k_w8a16_panel: activation rows per workgroup (0: 16 * mb)
    int scale_stage;   // k_w8a16_panel with groups: 2 = each wave's group scales
                       // preloaded into LDS, 1 = staged per chunk
};
// act: the activation type (kW8A16Act* below).
W8A16Plan plan_w8a16(int64_t m, int64_t n, int64_t k, int act = 0);
// Per-group weight scales (w_scale [n, ceil(k / group)]); group is 64, 128,
// 256 or 512; act as for plan_w8a16 (not kW8A16ActQ).  The panel kernel where
// the per-channel plan takes it and the groups divide the waves' K ranges,
// else the rows or tile kernel.
W8A16Plan plan_w8a16_grouped(int64_t m, int64_t n, int64_t k, int64_t group, int act = 0);
// act: the activation type -- 0 bf16 (fp8_w_bf16_a, bf16 out), 1 fp16
// (fp8_w_fp16_a, fp16 out), 2 E4M3 codes with *x_scale (fp8_w_fp8_a at decode
// sizes, bf16 out).  ld_x counts activation values.
// 3: bf16 activations quantized per tensor on the fly (fp8_w_fp8_a with the
// dynamic activation quantization folded in): see w8a16_quant_act.
constexpr int kW8A16ActBF16 = 0, kW8A16ActF16 = 1, kW8A16ActF8 = 2, kW8A16ActQ = 3;
// Row strides the decode kernels take (elements of x, bytes of w): a load
// instruction addresses a few rows from one base with 32-bit lane offsets.
inline bool w8a16_supports_ld(int64_t ld_x, int64_t ld_w)
{
    return ld_x < ((int64_t)1 << 28) && ld_w < ((int64_t)1 << 28);
}
hipError_t w8a16(const W8A16Plan &p, int act, const void *x, int64_t m, int64_t k, int64_t ld_x,
                 const float *x_scale, const uint8_t *w, int64_t n, int64_t ld_w,
                 const float *w_scale, uint16_t *y, int64_t ld_y, void *workspace,
                 hipStream_t stream);
// fp8_w_fp8_a on bf16 activations, quantized per tensor inside the GEMM: the
// plan is plan_w8a16(m, n, k, kW8A16ActQ); act_part holds the npart maxima of
// act_amax over x, or is null with a panel plan, whose workgroups then each
// read all of x for its maximum (for tensors of a few tens of KB).  The scale used goes to *x_scale_out (always written;
// the K-split reduction reads it back), a non-finite maximum raises *flag.
// workspace: the plan's partial tiles.
hipError_t w8a16_quant_act(const W8A16Plan &p, const uint16_t *x, int64_t m, int64_t k,
                           int64_t ld_x, const uint32_t *act_part, int npart, float *x_scale_out,
                           int32_t *flag, const uint8_t *w, int64_t n, int64_t ld_w,
                           const float *w_scale, uint16_t *y, int64_t ld_y, void *workspace,
                           hipStream_t stream);

// Device address of this GPU's kNoallocScratchBytes scratch array, looked up
// (hipGetSymbolAddress, with `device` made current for the call) on the first
// request for that device and kept.
hipError_t noalloc_scratch(int device, void **ptr);

// ---- prefill GEMM for 16-bit activations (fp8_w_fp16_a / fp8_w_bf16_a) ------
// Y = X . dequant(W)^T on v_mfma_f32_32x32x16_{f16,bf16}, 256 x 256 tiles; x is
// fp16 (f16) or bf16 [m, ld_x], y the same type.  No scratch.
bool w8a16_gemm_supports(int64_t ld_x, int64_t ld_w);
hipError_t w8a16_gemm(bool f16, const uint16_t *x, int64_t m, int64_t k, int64_t ld_x,
                      const uint8_t *w, int64_t n, int64_t ld_w, const float *w_scale,
                      uint16_t *y, int64_t ld_y, hipStream_t stream);

// ---- W8A8 (fp8_w_fp8_a) GEMM on FP8 MFMA -----------------------------------
struct W8A8Plan {
    int64_t tiles_m, tiles_n;
    size_t workspace;
};
W8A8Plan plan_w8a8(int64_t m, int64_t n, int64_t k);
bool w8a8_supports_ld(int64_t ld);
hipError_t w8a8(const W8A8Plan &p, const uint8_t *x, int64_t m, int64_t k, int64_t ld_x,
                const float *x_scale, const uint8_t *w, int64_t n, int64_t ld_w,
                const float *w_scale, uint16_t *y, int64_t ld_y, hipStream_t stream,
                int64_t group = 0);

}  // namespace launch
}  // namespace fp8q
