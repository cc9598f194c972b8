// decode_bf16.hip -- single-token GQA decode against a bf16 KV cache (d_h = 128),
// split over the cache ("flash-decoding"), plus the log-sum-exp merge of the
// split partials shared with the MLA decode.
//
// Method: the one new query of each sequence attends to every cached key of
// that sequence ("Attention deep dive (MHA -> MQA -> GQA -> FlashAttention)",
// section 5); the cache keeps only the h_kv heads and every query head of a
// group reads its group's K/V ("2.4 Multi-Head Attention, MQA, GQA & MLA",
// "Implementing the MHA -> GQA conversion").  Decode is bound by the bytes of
// the cache: arithmetic intensity about h_q / h_kv FLOP per byte ("Attention
// Engineering: From MHA to GQA, MLA & FlashAttention", section 0, equation
// "Decoding Attention Arithmetic Intensity"), so the design goal is to read
// each cached K/V byte exactly once, coalesced, with many bytes in flight.
//
// The cache of each (sequence, K/V head) is cut into chunks of `split` keys;
// one workgroup handles one chunk for up to 16 query heads of the group, so
// every K/V byte of the chunk is read from HBM once:
//  * 64-key tiles of K and V stream HBM -> LDS through a 4-stage ring filled
//    by global_load_lds_dwordx4 (three tiles in flight per CU, no staging
//    registers); rows are stored with a 304-byte stride (19 = 3 mod 16 bank
//    slots), so 16-byte reads down a column and transposing reads of 4 rows
//    are bank-conflict free and all addresses are base + immediate;
//  * each of the 4 waves computes the whole score tile S^T = K q^T
//    (v_mfma_f32_16x16x32_bf16, the group's heads as the 16 columns) and the
//    softmax -- MFMA time is small next to the tile's HBM time, and doing it
//    redundantly gives every wave the same (m, l) with no exchange -- then
//    the P.V product for its own quarter of d: O^T = V^T P^T, with V^T read
//    by ds_read_b64_tr_b16 and the rounded probabilities as the B operand;
//  * the chunk's normalised partial output and log-sum-exp go to the
//    workspace; a second kernel merges the chunks of each (sequence, head):
//    L = log sum_s exp(L_s), O = sum_s exp(L_s - L) O_s, the FlashAttention-2
//    state merge ("Attention Engineering ...", section 4).
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int D = 128;
constexpr int BN = 64;                    // keys per tile
constexpr int NW = 4;                     // waves per workgroup
constexpr int LROW = D * 2 + 48;          // LDS row stride, bytes (304)
constexpr int REGION = BN * LROW;         // 19456 B: K rows, then V rows
constexpr int TILE_BYTES = 2 * REGION;    // 38912 B = 38 one-KB DMA blocks
constexpr int NSTAGE = 4;
constexpr int LDS_BYTES = NSTAGE * TILE_BYTES;   // 155648
constexpr float TAU = 8.0f;

struct Params {
    const __bf16 *q, *k, *v;
    const int32_t *seq_lens;
    float *ws_o, *ws_lse;
    int S_max, hq, hkv, G, n_hchunk;
    int split, n_split_max, window;
    float scale_log2;
};

__device__ __forceinline__ int tile_off(int r, int chunk) { return r * LROW + (chunk << 4); }

__global__ __launch_bounds__(64 * NW, 1) void decode_bf16_d128_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int j16 = lane & 15;
    const int q16 = lane >> 4;

    const int s = blockIdx.x;
    const int g = blockIdx.y / p.n_hchunk;
    const int hc = blockIdx.y % p.n_hchunk;
    const int b = blockIdx.z;
    int len = p.seq_lens[b];
    len = len < 0 ? 0 : (len > p.S_max ? p.S_max : len);
    if (s * p.split >= len) return;                      // beyond the sequence: unused split
    const int kvis = p.window > 0 ? max(0, len - p.window) : 0;
    const int lo = max(s * p.split, kvis);
    const int hi = min((s + 1) * p.split, len);
    const int n_tiles = lo < hi ? (hi - lo + BN - 1) / BN : 0;

    const int hidx = hc * 16 + j16;                       // head within the group (column)
    const bool head_ok = hidx < p.G;
    const int h = g * p.G + hidx;
    const size_t kv_base = ((size_t)b * p.hkv + g) * (size_t)p.S_max * D;
    const char *kg = reinterpret_cast<const char *>(p.k + kv_base);
    const char *vg = reinterpret_cast<const char *>(p.v + kv_base);

    // DMA of tile t: blocks 0-18 fill the K rows, 19-37 the V rows; waves 0-1
    // issue 10 blocks, waves 2-3 issue 9.  LDS byte o of a region holds row
    // o / 304, chunk (o % 304) / 16; pad slots receive an arbitrary valid
    // chunk, rows past the chunk end re-read the last valid key (masked).
    const int my_blk0 = wave < 2 ? 10 * wave : 20 + 9 * (wave - 2);
    const int my_nblk = wave < 2 ? 10 : 9;
    auto issue_tile = [&](int t) {
        char *stage = smem + (t % NSTAGE) * TILE_BYTES;
        const int t0 = lo + t * BN;
#pragma unroll
        for (int i = 0; i < 10; ++i) {
            if (i >= my_nblk) break;
            const int blk = my_blk0 + i;
            const int o = blk * 1024 + lane * 16;
            const bool is_v = o >= REGION;
            const int ro = is_v ? o - REGION : o;
            const int r = ro / LROW;
            const int ch = min((ro - r * LROW) >> 4, D / 8 - 1);
            const int key = min(t0 + r, hi - 1);
            const char *src = (is_v ? vg : kg) + (size_t)key * (D * 2) + ch * 16;
            dma16(src, stage + blk * 1024);
        }
    };
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t)
        if (t < n_tiles) issue_tile(t);

    // q^T as B operand: column = head j16, d = 32ks + 8 q16 .. +7.
    bf16x8 qop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (head_ok) val = ldg16(p.q + ((size_t)b * p.hq + h) * D + 32 * ks + 8 * q16);
        qop[ks] = __builtin_bit_cast(bf16x8, val);
    }

    f32x4 oacc[2];                                        // d = 32 wave + 16 dbl + 4 q16 + i
    oacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    oacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const int v_row_lane = 4 * q16 + (j16 >> 2);
    const int v_chunk_lane = 4 * wave + ((j16 & 3) >> 1);  // chunk of d = 32 wave + 16 dbl + 4(j%4)
    const int v_byte_lane = 8 * (j16 & 1);

    for (int t = 0; t < n_tiles; ++t) {
        const int newer = t == 0 ? 0 : min(NSTAGE - 2, n_tiles - 1 - t);
        if (newer == 0) wait_vmcnt<0>();
        else if (newer == 1) { if (my_nblk == 10) wait_vmcnt<10>(); else wait_vmcnt<9>(); }
        else { if (my_nblk == 10) wait_vmcnt<20>(); else wait_vmcnt<18>(); }
        raw_barrier();
        if (t + NSTAGE - 1 < n_tiles) issue_tile(t + NSTAGE - 1);

        const char *kt = smem + (t % NSTAGE) * TILE_BYTES;
        const char *vt = kt + REGION;
        const int t0 = lo + t * BN;
        // S^T blocks mb = 0..3: key 16mb + j16 (A row), element (mb, i) of this
        // lane = key t0 + 16mb + 4 q16 + i of head column j16.
        f32x4 sacc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kt + tile_off(16 * mb + j16, 4 * ks + q16));
                sacc[mb] = mfma16x16x32(a, qop[ks], sacc[mb]);
            }
        }
        const bool tail = t0 + BN > hi;
        float x[16];
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = sacc[mb][i] * p.scale_log2;
                if (tail) v = (t0 + 16 * mb + 4 * q16 + i < hi) ? v : -INFINITY;
                x[4 * mb + i] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const bool upd = mx > m_run + TAU;
        const float m_new = upd ? mx : m_run;
        const float alpha = upd ? fast_exp2(m_run - m_new) : 1.0f;
        m_run = m_new;
        oacc[0] *= alpha;
        oacc[1] *= alpha;
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        float pv[16];
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            pv[e] = fast_exp2(x[e] - m_use);
            lsum += pv[e];
        }
        l_run = l_run * alpha + lsum;
        // K-step kk covers keys 32kk .. 32kk+31: elements (mb = 2kk, i) then (2kk+1, i)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 pop = to_bf16x8(pv[8 * kk + 0], pv[8 * kk + 1], pv[8 * kk + 2], pv[8 * kk + 3],
                                         pv[8 * kk + 4], pv[8 * kk + 5], pv[8 * kk + 6], pv[8 * kk + 7]);
#pragma unroll
            for (int dbl = 0; dbl < 2; ++dbl) {
                const int r = 32 * kk + v_row_lane;
                const int ch = v_chunk_lane + 2 * dbl;
                const bf16x4 lo4 = lds_read_tr16(vt + tile_off(r, ch) + v_byte_lane);
                const bf16x4 hi4 = lds_read_tr16(vt + tile_off(r + 16, ch) + v_byte_lane);
                const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[dbl] = mfma16x16x32(a, pop, oacc[dbl]);
            }
        }
    }
    float lt = l_run + shfl_xor(l_run, 16);
    lt += shfl_xor(lt, 32);
    if (!head_ok) return;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const size_t ws = ((size_t)b * p.hq + h) * p.n_split_max + s;
    float *wo = p.ws_o + ws * D;
#pragma unroll
    for (int dbl = 0; dbl < 2; ++dbl)
        *reinterpret_cast<f32x4 *>(wo + 32 * wave + 16 * dbl + 4 * q16) = oacc[dbl] * inv;
    if (wave == 0 && q16 == 0) p.ws_lse[ws] = lt > 0.f ? m_run + __log2f(lt) : -INFINITY;
}

// One wave per (head, sequence): merge the partials of the sequence's splits.
template <int DV>
__global__ __launch_bounds__(64) void split_combine_kernel(const float *ws_o, const float *ws_lse,
                                                           const int32_t *seq_lens, __bf16 *o, float *lse,
                                                           int H, int S_max, int split, int n_split_max) {
    constexpr int PER = DV / 64;
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    int len = seq_lens[b];
    len = len < 0 ? 0 : (len > S_max ? S_max : len);
    const int ns = (len + split - 1) / split;
    const size_t base = ((size_t)b * H + h) * n_split_max;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ws_lse[base + s]);
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    float Z = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < ns; ++s) {
            const float ls = ws_lse[base + s];
            if (ls == -INFINITY) continue;
            const float w = fast_exp2(ls - M);
            Z += w;
            const float *src = ws_o + (base + s) * DV;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] += w * src[lane + 64 * i];
        }
    }
    const float inv = Z > 0.f ? 1.0f / Z : 0.f;
    __bf16 *dst = o + ((size_t)b * H + h) * DV;
#pragma unroll
    for (int i = 0; i < PER; ++i) dst[lane + 64 * i] = (__bf16)(acc[i] * inv);
    if (lse && lane == 0) lse[(size_t)b * H + h] = Z > 0.f ? (M + __log2f(Z)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_decode_bf16_d128(const DecodeArgs &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.k = static_cast<const __bf16 *>(a.k_cache);
    p.v = static_cast<const __bf16 *>(a.v_cache);
    p.seq_lens = a.seq_lens;
    p.ws_o = a.ws_o;
    p.ws_lse = a.ws_lse;
    p.S_max = a.S_max;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.n_hchunk = (p.G + 15) / 16;
    p.split = a.split;
    p.n_split_max = a.n_split_max;
    p.window = a.window;
    p.scale_log2 = a.scale * kLog2e;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_bf16_d128_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid(a.n_split_max, a.hkv * p.n_hchunk, a.B);
    hipLaunchKernelGGL(decode_bf16_d128_kernel, grid, dim3(64 * NW), LDS_BYTES, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_combine(a.ws_o, a.ws_lse, a.seq_lens, a.o, a.lse, a.B, a.hq, D, a.S_max,
                                a.split, a.n_split_max, stream);
}

hipError_t launch_split_combine(const float *ws_o, const float *ws_lse, const int32_t *seq_lens,
                                void *o, float *lse, int B, int H, int dv, int S_max, int split,
                                int n_split_max, hipStream_t stream) {
    dim3 grid(H, B);
    __bf16 *ob = static_cast<__bf16 *>(o);
    switch (dv) {
        case 128:
            hipLaunchKernelGGL(split_combine_kernel<128>, grid, dim3(64), 0, stream, ws_o, ws_lse,
                               seq_lens, ob, lse, H, S_max, split, n_split_max);
            break;
        case 512:
            hipLaunchKernelGGL(split_combine_kernel<512>, grid, dim3(64), 0, stream, ws_o, ws_lse,
                               seq_lens, ob, lse, H, S_max, split, n_split_max);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mi355
