// kcommon.h -- device-side vocabulary shared by the gfx950 attention kernels:
// vector types, bf16 packing, MFMA wrappers and cross-lane helpers.
//
// MFMA register layouts used throughout (wave64, gfx950):
//  * v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//      A: lane l holds 8 bf16 of row (l % 32); B: lane l holds 8 bf16 of
//      column (l % 32); lanes 0-31 and 32-63 hold the two halves of the K
//      dimension.  The kernels only rely on A and B using the same K
//      assignment, so the order of K inside an operand is irrelevant.
//      D: lane l holds column (l % 32), element i is row
//      8*(i/4) + 4*(l/32) + (i%4), i = 0..15.
//  * v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//      A: lane l holds 8 bf16 of row (l % 16); B: 8 bf16 of column (l % 16);
//      the four lane groups (l / 16) hold the four quarters of K.
//      D: lane l holds column (l % 16), element i is row 4*(l/16) + i.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Eight fp32 -> bf16x8 (RNE).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
    u32x4 u = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5),
               pack_bf16x2(a6, a7)};
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (l ^ mask), through ds_bpermute (any mask < 64).
__device__ __forceinline__ float shfl_xor(float x, int mask) {
    int lane = __lane_id();
    int src = lane ^ mask;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)p;
}

// Global 16-byte load/store helpers (plain vector accesses).
__device__ __forceinline__ u32x4 ldg16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace mi355
