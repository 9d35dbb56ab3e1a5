// device.h -- gfx950 (CDNA4) device helpers shared by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blasst {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lane layout (wave64):
// A[m][k]: lane = m + 32*(k/8), element k%8;  B[k][n]: lane = n + 32*(k/8),
// element k%8;  D[m][n]: lane = n + 32*((m/4)%2), register (m%4) + 4*(m/8).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA.  A[m][k]: lane = m + 16*(k/8), element k%8; B alike with
// n; D[m][n]: lane = n + 16*(m/4), register m%4.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Hardware 2^x (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Round-to-nearest-even fp32 -> bf16 of 8 values.
__device__ __forceinline__ bf16x8 cvt_bf16x8(f32x8 f) { return __builtin_convertvector(f, bf16x8); }

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

} // namespace blasst
