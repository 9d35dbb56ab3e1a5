// acc.h -- MFMA accumulators pinned in physical AGPRs, and MFMAs with VGPR
// accumulators, for kernels whose per-wave state fills both register files
// (one wave per SIMD).
//
// Left to itself the compiler gives every builtin MFMA an AGPR accumulator
// and, when the accumulators plus their VALU users exceed one file, shuffles
// them between VGPRs and AGPRs and spills.  The kernels that include this
// header therefore keep their output accumulator in physical AGPRs (tile at
// a[base, base+16)) that no compiler-managed value touches: every access --
// zeroing, the MFMAs, rescaling, read-out -- is inline asm on the physical
// registers, and the compiler, which sees no AGPR values, keeps its own values
// in VGPRs (a CPU test checks the generated code for AGPR use outside these
// blocks).  Their other MFMAs are asm too, with VGPR accumulators.  The
// compiler does not see through asm, so hazard padding is explicit: three
// wait states before each MFMA cover a VALU or accvgpr write of its sources,
// and 24 wait states follow the last MFMA of a chain before any other
// instruction reads its result.
#pragma once

#include "device.h"

namespace blasst {

#define BLASST_ALL_AGPRS \
    "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", \
    "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", \
    "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", \
    "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", \
    "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79", \
    "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95", \
    "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", \
    "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127", \
    "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143", \
    "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159", \
    "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175", \
    "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191", \
    "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207", \
    "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223", \
    "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239", \
    "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255"

// Zeroes a0..a255 (and declares all of them used by the kernel).
__device__ __forceinline__ void acc_zero()
{
    asm volatile(".set .Lac, 0\n\t.rept 256\n\tv_accvgpr_write_b32 a[.Lac], 0\n\t"
                 ".set .Lac, .Lac+1\n\t.endr" ::: BLASST_ALL_AGPRS);
}

// a[base, base+16) += A * B (32x32x16 bf16); base is a compile-time constant
// after unrolling.
__device__ __forceinline__ void acc_mfma(int base, const u32x4 &a, const bf16x8 &b)
{
    asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[%2:%3], %0, %1, a[%2:%3]"
                 ::"v"(a), "v"(b), "i"(base), "i"(base + 15));
}

// 24 wait states: an MFMA result may be read by any instruction afterwards.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// a0..a255 *= alpha, four registers at a time.
__device__ __forceinline__ void acc_scale(float alpha)
{
    float t0, t1, t2, t3;
    asm volatile(".set .Lac, 0\n\t.rept 64\n\t"
                 "v_accvgpr_read_b32 %0, a[.Lac]\n\tv_accvgpr_read_b32 %1, a[.Lac+1]\n\t"
                 "v_accvgpr_read_b32 %2, a[.Lac+2]\n\tv_accvgpr_read_b32 %3, a[.Lac+3]\n\t"
                 "v_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\t"
                 "v_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\t"
                 "v_accvgpr_write_b32 a[.Lac], %0\n\tv_accvgpr_write_b32 a[.Lac+1], %1\n\t"
                 "v_accvgpr_write_b32 a[.Lac+2], %2\n\tv_accvgpr_write_b32 a[.Lac+3], %3\n\t"
                 ".set .Lac, .Lac+4\n\t.endr"
                 : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
                 : "v"(alpha)
                 : BLASST_ALL_AGPRS);
}

// Reads the 16 registers a[base, base+16).
__device__ __forceinline__ f32x16 acc_read(int base)
{
    float e[16];
    asm volatile("v_accvgpr_read_b32 %0, a[%16]\n\tv_accvgpr_read_b32 %1, a[%16+1]\n\t"
                 "v_accvgpr_read_b32 %2, a[%16+2]\n\tv_accvgpr_read_b32 %3, a[%16+3]\n\t"
                 "v_accvgpr_read_b32 %4, a[%16+4]\n\tv_accvgpr_read_b32 %5, a[%16+5]\n\t"
                 "v_accvgpr_read_b32 %6, a[%16+6]\n\tv_accvgpr_read_b32 %7, a[%16+7]\n\t"
                 "v_accvgpr_read_b32 %8, a[%16+8]\n\tv_accvgpr_read_b32 %9, a[%16+9]\n\t"
                 "v_accvgpr_read_b32 %10, a[%16+10]\n\tv_accvgpr_read_b32 %11, a[%16+11]\n\t"
                 "v_accvgpr_read_b32 %12, a[%16+12]\n\tv_accvgpr_read_b32 %13, a[%16+13]\n\t"
                 "v_accvgpr_read_b32 %14, a[%16+14]\n\tv_accvgpr_read_b32 %15, a[%16+15]"
                 : "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]),
                   "=v"(e[6]), "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]),
                   "=v"(e[12]), "=v"(e[13]), "=v"(e[14]), "=v"(e[15])
                 : "i"(base));
    f32x16 r;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        r[i] = e[i];
    return r;
}

// MFMAs with VGPR accumulators.  The first k-step of several accumulators is
// one statement so that the early-clobber outputs cannot overlap an A or B
// operand that an earlier MFMA of the step may still be reading.
__device__ __forceinline__ void mfma_v_first2(f32x16 &c0, f32x16 &c1, const u32x4 &a0, const u32x4 &a1,
                                              const bf16x8 &b)
{
    asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %2, %4, 0\n\t"
                 "v_mfma_f32_32x32x16_bf16 %1, %3, %4, 0"
                 : "=&v"(c0), "=&v"(c1)
                 : "v"(a0), "v"(a1), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16 &c, const u32x4 &a, const bf16x8 &b)
{
    asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_drain2(f32x16 &c0, f32x16 &c1)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
}
} // namespace blasst
