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

// max(x, x of lane i ^ 32) with the gfx950 v_permlane32_swap, which swaps the
// upper half-wave of one copy of x with the lower half of another: each lane
// ends up holding its own value and its partner's, in either order, with no
// LDS round trip.
__device__ __forceinline__ float max_xor32(float x)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// max(x, x of lane i ^ 16) with v_permlane16_swap (odd 16-lane rows of one
// copy swapped with the even rows of another), likewise without LDS.
__device__ __forceinline__ float max_xor16(float x)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

} // namespace blasst

namespace blasst {

// s_waitcnt that waits until at most N vector-memory operations (including
// global->LDS copies) of this wave are outstanding; other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS byte address of a pointer into __shared__ memory: the value the copies
// below put in m0.  Taken once per buffer, outside the loops: converting a
// generic pointer costs a null test, and per copy those tests and the 64-bit
// pointers they need crowd the scalar registers.
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_void *)p; }

// 16-byte global -> LDS copy (global_load_lds_dwordx4); the wave's 64 lanes
// fill 1024 consecutive LDS bytes starting at LDS byte address lds
// (wave-uniform).  It is
// issued from inline asm so that the compiler does not add its own
// conservative vmcnt(0) waits before every later LDS read: the kernels wait
// for these copies explicitly (wait_vmcnt) before the barrier that publishes
// the data.  The instruction writes no register.
// (m0 is set right before the copy; the compiler uses it nowhere else in
// these kernels, so the clobber is honoured in practice.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// NT = true adds the non-temporal hint, for data that is streamed once (a
// decode step reads each cache row once).
template <bool NT = false>
__device__ __forceinline__ void copy16_to_lds(const void *src, uint32_t lds)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    if (NT)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(m0), "v"(src) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory", "m0");
}

// Same copy with a wave-uniform 64-bit base (SGPR pair) and a per-lane 32-bit
// byte offset: the per-block address arithmetic becomes one scalar add.
template <bool NT = false>
__device__ __forceinline__ void copy16_to_lds_s(const void *sbase, uint32_t voff, uint32_t lds)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    // readfirstlane returns int: zero-extend each half (a sign-extended low
    // half would turn the base into an invalid address).
    const uint64_t bs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
    if (NT)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0), "v"(voff), "s"(bs)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(bs)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// Compiler-level memory barrier (no instruction): keeps LDS reads below an
// explicit wait_vmcnt for copies the compiler does not track.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier that orders LDS accesses only: global memory is not
// fenced, so outstanding global->LDS copies and global stores are not drained
// (the kernels wait for their copies explicitly before the barrier).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// gfx950 LDS transpose read of 16-bit data.  Within each group of 16 lanes,
// lane s supplies an 8-byte address; lane i receives element (i % 4) of the
// data addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12, in that order.
__device__ __forceinline__ i16x4 lds_read_tr16(const void *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
}

} // namespace blasst
