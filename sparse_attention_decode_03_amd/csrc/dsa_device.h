// dsa_device.h -- small device-side helpers shared by the gfx950 kernels of
// the DSA decode path (vector types, matrix-core wrappers, number formats,
// the order-preserving score key and block-wide scans).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on gfx9-family chips: 32-bit data format,
// no swizzle, no stride; with stride 0 the range check compares the byte
// offset with the record count, and a load past it returns zeros.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of the buffer load builtins: the non-temporal bit.
constexpr int kCachePolicyNT = 2;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16). Lane l supplies row l%16 of
// A and column l%16 of B, eight consecutive k each (k block l/16); it receives
// D[4*(l/16) + v][l%16] in element v.
__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16). Lane l supplies row l%32 of
// A and column l%32 of B (k block l/32); it receives
// D[8*(v/4) + 4*(l/32) + v%4][l%32] in element v.
__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two OCP E4M3 bytes (byte pair HI of `word`) -> two bf16 packed in a dword.
// Every E4M3 value is exactly representable in bf16, so the conversion through
// fp32 is exact; the bf16 code is the upper half of the fp32 code.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t word)
{
    typedef float float2_t __attribute__((ext_vector_type(2)));
    float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(word, HI);
    uint32_t lo_bits = __float_as_uint(f.x);
    uint32_t hi_bits = __float_as_uint(f.y);
    return (hi_bits & 0xFFFF0000u) | (lo_bits >> 16);
}

// The same conversion in one gfx950 instruction (scaled FP8 -> packed bf16
// with scale 1.0; exact, as every E4M3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2_exact(uint32_t word)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> bf16, round to nearest even; a NaN stays a (quiet) NaN. Written
// as a select so it compiles to straight-line code.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x0040u;
    return (uint16_t)(((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet : rounded);
}

// Two fp32 -> packed bf16, round to nearest even, in one gfx950 instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float float2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}

// Order-preserving unsigned key of an fp32 score: a > b  <=>  key(a) > key(b)
// for non-NaN a, b, with -0.0 mapped onto +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Data-parallel lane moves (VALU, no LDS round trip). Controls: quad
// permutations xor 1 and xor 2, mirror inside each half-row of 8 lanes and
// inside each row of 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Wave-wide reductions and scan through DPP row moves plus three readlanes
// (no LDS round trip): the sum / max / min of all 64 lanes in every lane, and
// the inclusive prefix sum of lanes 0..lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shift_in_zero(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan_add(uint32_t x)
{
    x += dpp_shift_in_zero<0x111>(x); // row_shr:1
    x += dpp_shift_in_zero<0x112>(x); // row_shr:2
    x += dpp_shift_in_zero<0x114>(x); // row_shr:4
    x += dpp_shift_in_zero<0x118>(x); // row_shr:8 -> prefix within each row of 16
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}
// Pairwise combination of lanes l and l ^ 32 (and of l and l ^ 16 within
// each 32-lane half) through the gfx950 lane-swap instructions, with no LDS
// round trip. Every lane receives op(own, partner); each op here is
// commutative, so the result is bit-identical to op(x, shuffle_xor(x, d)).
__device__ __forceinline__ float add_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<kDppQuadXor1>(v));
    v = max(v, dpp_u32<kDppQuadXor2>(v));
    v = max(v, dpp_u32<kDppRowHalfMirror>(v));
    v = max(v, dpp_u32<kDppRowMirror>(v));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
// Sum over the wave, the same in every lane (after each step every lane of a
// group holds the group's sum, so the mirror steps add disjoint halves).
__device__ __forceinline__ float wave_total_f32(float x)
{
    x += __uint_as_float(dpp_u32<kDppQuadXor1>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<kDppQuadXor2>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<kDppRowMirror>(__float_as_uint(x)));
    const int b = __float_as_int(x);
    return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = min(v, dpp_u32<kDppQuadXor1>(v));
    v = min(v, dpp_u32<kDppQuadXor2>(v));
    v = min(v, dpp_u32<kDppRowHalfMirror>(v));
    v = min(v, dpp_u32<kDppRowMirror>(v));
    return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               min((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Block-wide exclusive prefix sum of one value per thread (blockDim.x == NT).
// `scratch` holds NT/64 + 1 words of LDS. Returns the exclusive prefix; the
// block total lands in *total.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch,
                                                         uint32_t *total)
{
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x % kWave;
    const int wid = threadIdx.x / kWave;
    const uint32_t x = wave_incl_scan_add(v);
    if (lane == kWave - 1)
        scratch[wid] = x;
    __syncthreads();
    uint32_t base = 0;
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        const uint32_t s = scratch[w];
        base += (w < wid) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

} // namespace dsa
