// Device helpers shared by the fp8q kernels (gfx950 / CDNA4 only).
//
// E4M3 here is the OCP "e4m3fn" encoding the deployment guide
// ("FP8量化与长上下文实测：Llama 3 70B部署优化指南", §1.1) describes: 4 exponent
// bits with bias 7, 3 mantissa bits, largest finite value 448, smallest
// subnormal 2^-9, no infinities.  gfx950 converts to and from this encoding
// in hardware (v_cvt_pk_fp8_f32, v_cvt_scalef32_pk_bf16_fp8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp8q {
namespace dev {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Largest finite E4M3 magnitude (the range is [-448, 448]).
constexpr float kE4M3Max = 448.0f;
// Lower clamp of a scale, as an fp32 constant (the fp32 value nearest 1e-12).
constexpr float kScaleFloor = 1e-12f;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// |bf16| as an unsigned key: for non-NaN values the order of the keys is the
// order of the magnitudes; NaN keys sort above +Inf (0x7F80).
__device__ __forceinline__ uint32_t abs_key_max2(uint32_t pair)
{
    uint32_t lo = pair & 0x7FFFu;
    uint32_t hi = (pair >> 16) & 0x7FFFu;
    return lo > hi ? lo : hi;
}

// Largest |bf16| key of a 16-byte chunk (8 values).
__device__ __forceinline__ uint32_t key_max8(uint4 v)
{
    return max(max(abs_key_max2(v.x), abs_key_max2(v.y)), max(abs_key_max2(v.z), abs_key_max2(v.w)));
}

// Scale from an absolute maximum given as a |bf16| key:
// s = max(fl32(amax / 448), 1e-12f), with an IEEE division.
__device__ __forceinline__ float scale_from_key(uint32_t key)
{
    float amax = __uint_as_float(key << 16);
    float s = amax / kE4M3Max;
    return s < kScaleFloor ? kScaleFloor : s;
}

// Four fp32 values -> four E4M3 codes packed little-endian in a dword.
// Round to nearest even; |t| >= 448 saturates to +-448 (the clamp runs first
// because the hardware conversion is not saturating by itself).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
    c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
    d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return (uint32_t)v;
}

// Eight bf16 values (a uint4) divided by s, cast to eight E4M3 codes (a uint2).
__device__ __forceinline__ uint2 quantize8(uint4 v, float s)
{
    uint2 r;
    r.x = e4m3x4(bf16_lo(v.x) / s, bf16_hi(v.x) / s, bf16_lo(v.y) / s, bf16_hi(v.y) / s);
    r.y = e4m3x4(bf16_lo(v.z) / s, bf16_hi(v.z) / s, bf16_lo(v.w) / s, bf16_hi(v.w) / s);
    return r;
}

// Four E4M3 codes (a dword) -> four bf16 values (two dwords).  Exact: every
// E4M3 value is representable in bf16.
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t codes)
{
    v2bf lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, 1.0f, false);
    v2bf hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, 1.0f, true);
    uint2 r;
    r.x = __builtin_bit_cast(uint32_t, lo);
    r.y = __builtin_bit_cast(uint32_t, hi);
    return r;
}

// Two fp32 values -> two bf16 bit patterns (lo in bits 15:0), round to
// nearest even: one v_cvt_pk_bf16_f32 (gfx950), where the integer rounding it
// replaced took about five instructions per value -- enough to show in the
// epilogues of the GEMMs (a 256 x 256 tile is 128 values per lane).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}

// fp32 -> bf16 bit pattern, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// Wave-wide unsigned max (64 lanes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

// Unsigned max over aligned groups of L lanes (L = 2..64, a power of two);
// every lane of a group gets the group's maximum.  Within a row of 16 lanes
// the exchanges are DPP moves (quad permutes, then the half-row and row
// mirrors, which pair each lane with one in the other half); 32-lane groups
// add a swizzle that swaps the two rows of each half-wave, 64-lane groups a
// permute across the halves.
template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v)
{
    static_assert(L >= 2 && L <= kWave && (L & (L - 1)) == 0, "group size");
    auto dpp_max = [](uint32_t x, auto ctrl) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value,
                                                                 0xF, 0xF, false);
        return o > x ? o : x;
    };
    v = dpp_max(v, std::integral_constant<int, 0xB1>{});       // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (L >= 4)
        v = dpp_max(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (L >= 8)
        v = dpp_max(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
    if constexpr (L >= 16)
        v = dpp_max(v, std::integral_constant<int, 0x140>{});  // row_mirror
    if constexpr (L >= 32) {
        // swizzle, bit mode: and 0x1F, xor 0x10 (lane ^ 16 within 32)
        const uint32_t o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
        v = o > v ? o : v;
    }
    if constexpr (L >= 64) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, 32, kWave);
        v = o > v ? o : v;
    }
    return v;
}

// Block-wide unsigned max; every thread gets the result.  `red` is LDS of
// at least blockDim.x / 64 words.  Contains __syncthreads: call uniformly.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red)
{
    v = wave_max_u32(v);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (lane == 0)
        red[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    for (int i = 0; i < nw; ++i)
        r = red[i] > r ? red[i] : r;
    __syncthreads();
    return r;
}

// One direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at LDS address lds + 16 * l.  `base` is wave-uniform (an
// SGPR pair), `off` the lane's 32-bit byte offset from it, `lds` a
// wave-uniform LDS byte address.  The instruction takes its LDS address from
// M0, which the asm sets; no other code in these kernels uses M0 (gfx950 LDS
// instructions do not), so the clobber is harmless and the compiler's warning
// about clobbering a reserved register is silenced.  The load counts in
// vmcnt like any other; once vmcnt has dropped past it, its bytes are in LDS.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const uint8_t *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// 16 bytes loaded / 8 bytes stored with the non-temporal hint: for data that
// streams through once (a weight matrix being quantized, the last read of
// an activation tensor), so that it does not displace what is re-read.
__device__ __forceinline__ uint4 ld_nt16(const void *p)
{
    const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt8(void *p, uint2 v)
{
    __builtin_nontemporal_store(v2u32{v.x, v.y}, reinterpret_cast<v2u32 *>(p));
}

// The same as dma16 with the non-temporal hint, for data read once (a
// stream of weights): streaming reads this way measured about 6.0 TB/s
// against 5.6 TB/s with the default policy on MI355X.
__device__ __forceinline__ void dma16_nt(const uint8_t *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "global_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane l's dword lands
// at LDS address lds + 4 * l.  `base` must be wave-uniform; it is read from
// the first lane (the compiler does not always prove such an address uniform,
// and the instruction takes it from an SGPR pair).  Each half goes through
// uint32_t, so the signed result of readfirstlane is not sign-extended.
__device__ __forceinline__ void dma4(const void *base, uint32_t off, uint32_t lds)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const void *ub = reinterpret_cast<const void *>(((uint64_t)hi << 32) | (uint64_t)lo);
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "global_load_lds_dword %0, %1"
                 :
                 : "v"(off), "s"(ub), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace dev
}  // namespace fp8q
