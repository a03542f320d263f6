// Device helpers shared by the gfx950 attention kernels: vector types, bf16 bit handling, MFMA
// wrappers and wavefront reductions.  wave64 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// 16-byte vector load / store (one dwordx4 per lane).
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even); lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// D[16x16] += A[16x32] B[32x16], bf16 in, fp32 accumulate.
// Lane l holds A row l%16 and B column l%16, k = 8(l/16)..+8; D column l%16, rows 4(l/16)..+4.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D[32x32] += A[32x16] B[16x32], bf16 in, fp32 accumulate.
// Lane l holds A row l%32 and B column l%32, k = 8(l/32)..+8; D column l%32, register i holds
// row 8(i/4) + 4(l/32) + i%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Max / sum of v over lanes l and l ^ 32, by v_permlane32_swap (a VALU op; no LDS round trip).  The
// swap exchanges the upper half of its first operand with the lower half of its second: with both set
// to v, lane l ends up holding {own, other} (l < 32) or {other, own} (l >= 32).
__device__ __forceinline__ float max_halves(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same over lanes l and l ^ 16 by v_permlane16_swap, which exchanges the odd 16-lane rows of its
// first operand with the even rows of its second.
__device__ __forceinline__ float max_rows16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_rows16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions across the four 16-lane groups that share lane%16 (VALU lane swaps, no LDS round trip).
__device__ __forceinline__ float max_across_groups16(float v) { return max_halves(max_rows16(v)); }
__device__ __forceinline__ float sum_across_groups16(float v) { return sum_halves(sum_rows16(v)); }

// Full-wave reductions.
__device__ __forceinline__ float wave_max(float v)
{
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

} // namespace attn
