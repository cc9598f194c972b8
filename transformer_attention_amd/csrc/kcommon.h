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

// Score-product MFMAs as inline asm with a VGPR accumulator, for kernels
// whose output accumulators fill the AGPRs (the compiler would otherwise
// place every MFMA accumulator there and spill).  The hazards the compiler
// cannot see through asm are covered here: the first MFMA of a chain waits
// 5 cycles (VALU writes of its operands just before), consecutive MFMAs of
// one chain accumulate into the same registers with the same opcode
// (forwarded by the hardware), and mfma_s_last is followed by 19 wait states
// before any VALU instruction may read the 16-pass result.  Operands coming
// from LDS or global loads are covered by the waitcnts the compiler inserts
// for every asm register operand.  Callers put a sched_barrier after the
// last MFMA of a group of chains so that no read of any of them is scheduled
// before the trailing wait states.
__device__ __forceinline__ f32x16 mfma_s_first(bf16x8 a, bf16x8 b) {
    f32x16 d;
    asm("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ f32x16 mfma_s_acc(bf16x8 a, bf16x8 b, f32x16 c) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    return c;
}
__device__ __forceinline__ f32x16 mfma_s_last(bf16x8 a, bf16x8 b, f32x16 c) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
        : "+v"(c) : "v"(a), "v"(b));
    return c;
}
// Output-product MFMA as inline asm with the accumulator pinned in AGPRs.
// Its B operand must have been written by VALU at least 5 wait states
// earlier (the callers' operands are older than the preceding mfma_s_last).
__device__ __forceinline__ void mfma_o_acc(bf16x8 a, bf16x8 b, f32x16 &acc) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// 19 wait states after the last MFMA that wrote `acc` (AGPRs), before VALU
// reads of it; ties the accumulator so that no read is scheduled earlier.
__device__ __forceinline__ void settle_acc(f32x16 &acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(acc));
}
// acc *= f on an accumulator held in AGPRs, as asm so that a (rare)
// conditional rescale does not make the compiler move the output registers
// through VGPRs around the branch.  The leading wait states cover an MFMA
// that may have written the accumulator just before; the trailing ones cover
// the AGPR writes before the next MFMA reads them as its accumulator.
__device__ __forceinline__ void scale_acc(f32x16 &acc, float f) {
    float t;
    asm volatile(
        "s_nop 7\n\ts_nop 7\n\ts_nop 4\n\t"
        "v_accvgpr_read_b32 %[t], %[a0]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a0], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a1]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a1], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a2]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a2], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a3]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a3], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a4]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a4], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a5]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a5], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a6]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a6], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a7]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a7], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a8]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a8], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a9]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a9], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a10]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a10], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a11]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a11], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a12]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a12], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a13]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a13], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a14]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a14], %[t]\n\t"
        "v_accvgpr_read_b32 %[t], %[a15]\n\tv_mul_f32 %[t], %[t], %[f]\n\tv_accvgpr_write_b32 %[a15], %[t]\n\t"
        "s_nop 4"
        : [a0] "+a"(acc[0]), [a1] "+a"(acc[1]), [a2] "+a"(acc[2]), [a3] "+a"(acc[3]),
          [a4] "+a"(acc[4]), [a5] "+a"(acc[5]), [a6] "+a"(acc[6]), [a7] "+a"(acc[7]),
          [a8] "+a"(acc[8]), [a9] "+a"(acc[9]), [a10] "+a"(acc[10]), [a11] "+a"(acc[11]),
          [a12] "+a"(acc[12]), [a13] "+a"(acc[13]), [a14] "+a"(acc[14]), [a15] "+a"(acc[15]),
          [t] "=&v"(t)
        : [f] "v"(f));
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

// End of a row with a sink logit s2 (log2 units): the row's online-softmax
// state is the reference max m (log2 units, -inf if no key was visible), the
// sum l of 2^(x - m) over its keys and the output accumulated against m.  The
// sink adds 2^s2 to the denominator and has no value row.  Returns the factor
// that turns the accumulated output into O, and writes the natural-log
// log-sum-exp of keys and sink.
__device__ __forceinline__ float finish_row_with_sink(float m, float l, float s2, float &lse_nat) {
    const float M = fmaxf(m, s2);
    if (M == -INFINITY) { lse_nat = -INFINITY; return 0.f; }
    const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
    const float z = l * f + (s2 == -INFINITY ? 0.f : fast_exp2(s2 - M));
    lse_nat = z > 0.f ? M * kLn2 + __logf(z) : -INFINITY;
    return z > 0.f ? f / z : 0.f;
}

// One split's normalised partial outputs of the MLA decode, stored as bf16
// rows through LDS.  The wave's 32 heads x 32*NDB values sit in O^T
// accumulators (element i of d-block db is value 32db + 8(i/4) + 4hh + (i%4)
// of head column l32); they go to the wave's own region of `lds` (rows
// 2*DV + 16 bytes apart), then each store writes one head's whole row.
// row0 is the partial-row index of the wave's first head, rows of
// consecutive heads are n_split apart, and only the first n_valid heads
// are stored.  The caller makes sure no wave still reads the region.
template <int NDB>
__device__ __forceinline__ void store_partial_rows(char *lds, int wave, int lane, const f32x16 (&oacc)[NDB],
                                                   float inv, __bf16 *ws_o, size_t row0, int n_split,
                                                   int n_valid) {
    constexpr int DV = 32 * NDB;
    constexpr int PITCH = 2 * DV + 16;
    static_assert(2 * DV == 64 * 16, "one 16-byte piece per lane covers a row");
    char *reg = lds + wave * 32 * PITCH;
    const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                             pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
            *reinterpret_cast<u32x2 *>(reg + l32 * PITCH + 2 * (32 * db + 8 * g + 4 * hh)) = w;
        }
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
        if (r >= n_valid) break;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(reg + r * PITCH + 16 * lane);
        *reinterpret_cast<u32x4 *>(ws_o + (row0 + (size_t)r * n_split) * DV + 8 * lane) = v;
    }
}

// Value of lane (l ^ mask), through ds_bpermute (any mask < 64).
__device__ __forceinline__ float shfl_xor(float x, int mask) {
    int lane = __lane_id();
    int src = lane ^ mask;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// Value of x in lane `l` (wave-uniform index) for every lane.
__device__ __forceinline__ float readlane_f32(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Max / sum of x over the lane pair (l, l ^ 32) through v_permlane32_swap
// (a VALU exchange of the two wave halves; lane l receives x[l % 32] and
// x[l % 32 + 32]).  Both lanes of a pair get bitwise the same result.
__device__ __forceinline__ float pair32_max(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N & 0x30) << 10) | (0x7 << 4) | (0xF << 8));
}
// wait_vmcnt with a wave-uniform runtime count in [0, 63] (larger counts wait
// for everything, which is always safe).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    switch (n) {
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 13: wait_vmcnt<13>(); break;
        case 14: wait_vmcnt<14>(); break;
        case 15: wait_vmcnt<15>(); break;
        case 16: wait_vmcnt<16>(); break;
        case 17: wait_vmcnt<17>(); break;
        case 18: wait_vmcnt<18>(); break;
        case 19: wait_vmcnt<19>(); break;
        case 20: wait_vmcnt<20>(); break;
        case 21: wait_vmcnt<21>(); break;
        case 22: wait_vmcnt<22>(); break;
        case 23: wait_vmcnt<23>(); break;
        case 24: wait_vmcnt<24>(); break;
        case 25: wait_vmcnt<25>(); break;
        case 26: wait_vmcnt<26>(); break;
        case 27: wait_vmcnt<27>(); break;
        case 28: wait_vmcnt<28>(); break;
        case 29: wait_vmcnt<29>(); break;
        case 30: wait_vmcnt<30>(); break;
        case 31: wait_vmcnt<31>(); break;
        case 32: wait_vmcnt<32>(); break;
        case 33: wait_vmcnt<33>(); break;
        case 34: wait_vmcnt<34>(); break;
        case 35: wait_vmcnt<35>(); break;
        case 36: wait_vmcnt<36>(); break;
        case 37: wait_vmcnt<37>(); break;
        case 38: wait_vmcnt<38>(); break;
        case 39: wait_vmcnt<39>(); break;
        case 40: wait_vmcnt<40>(); break;
        case 41: wait_vmcnt<41>(); break;
        case 42: wait_vmcnt<42>(); break;
        case 43: wait_vmcnt<43>(); break;
        case 44: wait_vmcnt<44>(); break;
        case 45: wait_vmcnt<45>(); break;
        case 46: wait_vmcnt<46>(); break;
        case 47: wait_vmcnt<47>(); break;
        case 48: wait_vmcnt<48>(); break;
        case 49: wait_vmcnt<49>(); break;
        case 50: wait_vmcnt<50>(); break;
        case 51: wait_vmcnt<51>(); break;
        case 52: wait_vmcnt<52>(); break;
        case 53: wait_vmcnt<53>(); break;
        case 54: wait_vmcnt<54>(); break;
        case 55: wait_vmcnt<55>(); break;
        case 56: wait_vmcnt<56>(); break;
        case 57: wait_vmcnt<57>(); break;
        case 58: wait_vmcnt<58>(); break;
        case 59: wait_vmcnt<59>(); break;
        case 60: wait_vmcnt<60>(); break;
        case 61: wait_vmcnt<61>(); break;
        case 62: wait_vmcnt<62>(); break;
        case 63: wait_vmcnt<63>(); break;
        default: wait_vmcnt<0>(); break;
    }
}
// s_waitcnt lgkmcnt(0): every LDS read this wave issued has returned.
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}
// Workgroup barrier without the memory fence of __syncthreads (which would
// drain every outstanding global->LDS load).  The wave's own LDS reads are
// complete before it arrives (so a stage may be refilled by any wave after
// the barrier), and the asm statements keep the compiler from moving memory
// accesses across it.  Global->LDS copies are ordered with wait_vmcnt.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Read-only load with a wave-uniform index through the constant address
// space: the compiler emits a scalar load (tracked by lgkmcnt, so it does not
// wait for outstanding vector-memory copies).  The data must not change
// while the kernel runs.
__device__ __forceinline__ int ld_uniform(const int32_t *p, int i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

// LDS byte offset of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char *)p);
}
// 16-byte global -> LDS copy (global_load_lds_dwordx4): lane L of the wave
// writes bytes [16L, 16L+16) after the wave-uniform LDS address `lds_base`.
// Issued through asm so the compiler does not treat every later LDS read as
// possibly aliasing the copy (it would wait for all outstanding copies, i.e.
// drain the prefetch ring); callers order the copies themselves with
// wait_vmcnt and a barrier.  The instruction has no register results (its
// address registers are read at issue), and nothing else in these kernels
// uses m0.
__device__ __forceinline__ void dma16(const void *gsrc, const void *lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gsrc), "s"(m0v) : "memory");
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the saddr form: one VGPR per address instead of two).  NT
// marks data that is streamed once (decode caches): the copy carries the
// non-temporal cache policy, so it does not displace reusable lines in L2 and
// the memory-attached last-level cache.  Data that other workgroups re-read
// (prefill K/V tiles) keeps the default policy.
template <bool NT = false>
__device__ __forceinline__ void dma16_off(const void *gbase, uint32_t off, const void *lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     :: "v"(off), "s"(gbase), "s"(m0v) : "memory");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(gbase), "s"(m0v) : "memory");
}
// The same with the LDS destination given as a wave-uniform LDS byte address.
template <bool NT = false>
__device__ __forceinline__ void dma16_off_at(const void *gbase, uint32_t off, uint32_t lds_addr_u) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr_u);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     :: "v"(off), "s"(gbase), "s"(m0v) : "memory");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(gbase), "s"(m0v) : "memory");
}

// 16-byte / 4-byte global stores issued through asm, for kernels that count
// their own vector-memory instructions (the compiler neither counts nor waits
// for them).  A store reads its data registers when it is issued; the
// trailing wait state covers a VALU write of them right after.
__device__ __forceinline__ void store16(void *p, f32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store4(void *p, float v) {
    asm volatile("global_store_dword %0, %1, off\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
// ds_read_b64_tr_b16: within each 16-lane group, result lane i element r is
// the (i%4)-th bf16 of the 8 bytes addressed by lane 4r + i/4 of that group.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void *lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t *)((__attribute__((address_space(3))) char *)lds_ptr));
}

typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
// ds_read_b64_tr_b8: within each 16-lane group, result lane i byte r is byte
// i % 8 of the 8 bytes addressed by lane 2r + i / 8 of that group (so if lanes
// 2r and 2r+1 address the two halves of 16 bytes of row r, lane i receives
// column i of the group's 8 rows).
__device__ __forceinline__ i32x2 lds_read_tr8(const void *lds_ptr) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2_t *)((__attribute__((address_space(3))) char *)lds_ptr));
}
// Eight OCP FP8 E4M3 codes (byte r of the pair of words = element r) to bf16.
// Every E4M3 value is exact in bf16 (3 mantissa bits, exponents in range).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 w) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ float ld_uniform_f(const float *p, long long i) {
    return ((const __attribute__((address_space(4))) float *)p)[i];
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)p;
}

// Global 16-byte load/store helpers (plain vector accesses).
__device__ __forceinline__ u32x4 ldg16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace mi355
