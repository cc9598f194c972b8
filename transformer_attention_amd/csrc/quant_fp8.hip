// quant_fp8.hip -- per-tile FP8 (OCP E4M3) quantisation of a bf16 KV cache.
//
// The pages quantise each tile with the scale amax / 448, 448 being the
// largest E4M3 value, and cast x / scale to E4M3 ("Flash Attention 3 and
// Multi-Headed Latent Attention", the FP8 attention section); a quantised
// KV cache halves the cache bytes ("Attention deep dive (MHA -> MQA -> GQA ->
// FlashAttention)", section 5, production-engine notes).  Here a tile is 32
// consecutive positions of one K/V head (all d values), the tile the decode
// kernel streams, so each streamed tile carries one scale.  An all-zero tile
// gets scale 1.  The division is IEEE fp32 and the cast rounds to nearest
// even (v_cvt_pk_fp8_f32), with magnitudes clamped to 448 first.
// E4M3 has no infinities: a NaN or +-inf input is stored as the NaN code
// (0x7f, or 0xff with the sign bit set), and the tile's amax runs over its
// finite values only, so such an entry changes no other code of its tile.
//
// One wave per tile.  For d_h <= 128 a tile (at most 4096 values) is held in
// registers (eight 16-byte loads per lane), so the cache is read once: the
// absolute maximum, then the codes.  Wider rows take a second pass over the
// tile (mostly from L2).  Bound by HBM: 2 bytes read and 1 written per value
// (the 70B workload's K cache, 2.1 G values: 1.32 ms, 4.9 TB/s).
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int TILE = 32;

// |x| of a finite value, 0 for NaN and +-inf (the amax statistic)
__device__ __forceinline__ float finite_abs(float x) {
    const float a = fabsf(x);
    return a < __builtin_inff() ? a : 0.f;
}

__device__ __forceinline__ i32x2 encode8(const bf16x8 v, float sc) {
    float y[8];
    unsigned nan_bytes[2] = {0u, 0u}, nan_mask[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = (float)v[e];
        const bool fin = fabsf(x) < __builtin_inff();
        y[e] = fin ? fminf(fmaxf(x / sc, -448.0f), 448.0f) : 0.f;
        if (!fin) {
            const unsigned sh = 8u * (e & 3);
            nan_mask[e >> 2] |= 0xffu << sh;
            nan_bytes[e >> 2] |= (__builtin_bit_cast(unsigned, x) >> 31 ? 0xffu : 0x7fu) << sh;
        }
    }
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    w0 = (int)(((unsigned)w0 & ~nan_mask[0]) | nan_bytes[0]);
    w1 = (int)(((unsigned)w1 & ~nan_mask[1]) | nan_bytes[1]);
    return i32x2{w0, w1};
}

template <bool IN_REGS>
__global__ __launch_bounds__(256) void quantize_kv_fp8_kernel(const __bf16 *x, uint8_t *codes,
                                                              float *scales, long long n_tiles,
                                                              int nt, int S, int d) {
    const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;
    const int lane = threadIdx.x & 63;
    const long long head = tile / nt;
    const int t = (int)(tile - head * nt);
    const int r0 = t * TILE;
    const int r1 = min(r0 + TILE, S);
    const size_t base = ((size_t)head * S + r0) * d;
    const int n = (r1 - r0) * d;                      // a multiple of 8
    float amax = 0.f;
    if constexpr (IN_REGS) {                          // n <= 4096: 8 chunks of 8 per lane
        bf16x8 buf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 8 * lane + 512 * i;
            buf[i] = c < n ? __builtin_bit_cast(bf16x8, ldg16(x + base + c)) : bf16x8{};
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, finite_abs((float)buf[i][e]));
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
        if (lane == 0) scales[tile] = sc;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 8 * lane + 512 * i;
            if (c < n) *reinterpret_cast<i32x2 *>(codes + base + c) = encode8(buf[i], sc);
        }
    } else {
        for (int c = 8 * lane; c < n; c += 512) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, ldg16(x + base + c));
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, finite_abs((float)v[e]));
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
        if (lane == 0) scales[tile] = sc;
        for (int c = 8 * lane; c < n; c += 512)
            *reinterpret_cast<i32x2 *>(codes + base + c) =
                encode8(__builtin_bit_cast(bf16x8, ldg16(x + base + c)), sc);
    }
}

}  // namespace

hipError_t launch_quantize_kv_fp8(const void *x, void *codes, float *scales, long long n_heads,
                                  int S, int d, hipStream_t stream) {
    const int nt = (S + TILE - 1) / TILE;
    const long long n_tiles = n_heads * nt;
    const long long blocks = (n_tiles + 3) / 4;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (d <= 128)
        hipLaunchKernelGGL(quantize_kv_fp8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const __bf16 *>(x), static_cast<uint8_t *>(codes), scales,
                           n_tiles, nt, S, d);
    else
        hipLaunchKernelGGL(quantize_kv_fp8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const __bf16 *>(x), static_cast<uint8_t *>(codes), scales,
                           n_tiles, nt, S, d);
    return hipGetLastError();
}

}  // namespace mi355
