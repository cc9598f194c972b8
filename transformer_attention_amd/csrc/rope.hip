// rope.hip -- rotary position embedding of the queries and keys, in place,
// in one launch.
//
// The pages rotate each pair (x_{2j}, x_{2j+1}) of a head as a complex number
// by the angle m theta_j at token position m, theta_j = base^(-2j/d), so
// that a rotated query and key interact through their distance only
// ("Attention Engineering: From MHA to GQA, MLA & FlashAttention", section
// 1); MLA rotates only the decoupled 64-d part of the query and the shared
// key ("Attention Engineering ...", section 3, "Complete MLA Attention
// Score").  Here the rotated dimensions are [rope_offset, rope_offset +
// rope_dim) of every row, which covers both.
//
// One thread per (batch, position, pair): it computes the angle and its
// cosine and sine once, in double precision (positions reach 10^5 and more,
// where an fp32 angle would be off by ~1e-2 rad), and applies them to that
// pair of every query head and every key head (fp32 arithmetic, rounded to
// the storage type).  Consecutive threads take consecutive pairs of a row,
// so each wave reads and writes contiguous row segments.  HBM-bound: every
// rotated value is read and written once.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

template <typename T> struct Pair;
template <> struct Pair<float> {
    static __device__ __forceinline__ void load(const float *p, float &a, float &b) {
        const f32x2 v = *reinterpret_cast<const f32x2 *>(p);
        a = v[0];
        b = v[1];
    }
    static __device__ __forceinline__ void store(float *p, float a, float b) {
        *reinterpret_cast<f32x2 *>(p) = f32x2{a, b};
    }
};
template <> struct Pair<__bf16> {
    static __device__ __forceinline__ void load(const __bf16 *p, float &a, float &b) {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
        a = __builtin_bit_cast(float, v << 16);
        b = __builtin_bit_cast(float, v & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(__bf16 *p, float a, float b) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
    }
};

template <typename T>
__global__ __launch_bounds__(256) void rope_qk_kernel(T *q, T *k, const int32_t *positions, int B,
                                                      int Tn, int hq, int hk, int row_q, int row_k,
                                                      int off, int half, double log2_base) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long n = (long long)B * Tn * half;
    if (i >= n) return;
    const int j = (int)(i % half);
    const long long bt = i / half;
    const int t = (int)(bt % Tn);
    const int b = (int)(bt / Tn);
    const double m = positions ? (double)positions[bt] : (double)t;
    const double theta = exp2(-(double)j / (double)half * log2_base);     // base^(-2j/d)
    double sd, cd;
    sincos(m * theta, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    for (int h = 0; h < hq; ++h) {
        T *p = q + (((size_t)b * hq + h) * Tn + t) * row_q + off + 2 * j;
        float x0, x1;
        Pair<T>::load(p, x0, x1);
        Pair<T>::store(p, x0 * c - x1 * s, x0 * s + x1 * c);
    }
    for (int h = 0; h < hk; ++h) {
        T *p = k + (((size_t)b * hk + h) * Tn + t) * row_k + off + 2 * j;
        float x0, x1;
        Pair<T>::load(p, x0, x1);
        Pair<T>::store(p, x0 * c - x1 * s, x0 * s + x1 * c);
    }
}

}  // namespace

hipError_t launch_rope_qk(const RopeArgs &a, hipStream_t stream) {
    const long long n = (long long)a.B * a.T * (a.rope_dim / 2);
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    const double l2b = log2((double)a.base);
    if (a.bf16)
        hipLaunchKernelGGL(rope_qk_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<__bf16 *>(a.q), static_cast<__bf16 *>(a.k), a.positions, a.B,
                           a.T, a.hq, a.hk, a.row_q, a.row_k, a.rope_offset, a.rope_dim / 2, l2b);
    else
        hipLaunchKernelGGL(rope_qk_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<float *>(a.q), static_cast<float *>(a.k), a.positions, a.B,
                           a.T, a.hq, a.hk, a.row_q, a.row_k, a.rope_offset, a.rope_dim / 2, l2b);
    return hipGetLastError();
}

}  // namespace mi355
