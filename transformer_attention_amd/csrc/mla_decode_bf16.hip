// mla_decode_bf16.hip -- Multi-head Latent Attention decode with absorbed
// up-projections (d_c = 512 latent + d_r = 64 decoupled RoPE key), bf16 on gfx950.
//
// Method ("Attention Engineering: From MHA to GQA, MLA & FlashAttention",
// section 3): with W_UK folded into the query and W_UV into the output
// projection, every head scores its 576-wide query [q~ ; q_R] against the
// shared per-token cache row [c_KV ; k_R] (equation "Complete MLA Attention
// Score", scale 1/sqrt(d_h + d_R)) and mixes the latent rows c_KV themselves,
// i.e. the value of token j is the first 512 entries of the same cache row.
// All heads read the same cache, so one workgroup processes all (up to 128)
// heads of a sequence against one chunk of the cache and every cache byte is
// read from HBM once per chunk; the chunks are merged by the log-sum-exp
// combine shared with the GQA decode.
//
// gfx950 mapping:
//  * a 32-token tile [32 x 576] is staged in LDS twice: row-major for the
//    score product (key rows permuted, see below) and transposed (c^T, the
//    first 512 columns) for the P.V product; global loads of the next tile
//    are in flight while the current one is consumed;
//  * each wave owns 16 heads: S^T = K Q^T with v_mfma_f32_16x16x32_bf16
//    (the wave's 16 queries, 576 wide, stay in registers as B operands),
//    then O^T[512 x 16] += C^T P^T, with the rounded probabilities used
//    directly as the B operand (keys assigned so each lane's eight values
//    are eight consecutive tokens);
//  * the online-softmax state is per head (one column of the wave) and the
//    reference max only moves when a tile exceeds it by 2^8.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int DC = 512, DR = 64, DK = DC + DR;
constexpr int TB = 32;              // tokens per tile
constexpr int KST = DK + 8;         // LDS row stride (bf16) of a K row: 1168 B
constexpr int VTS = TB + 8;         // LDS row stride (bf16) of a c^T row: 80 B
constexpr int K_ELEMS = TB * KST;
constexpr int V_ELEMS = DC * VTS;
constexpr int LDS_BYTES = (K_ELEMS + V_ELEMS) * 2;
constexpr float TAU = 8.0f;
constexpr int MAX_WAVES = 8;

struct Params {
    const __bf16 *q, *c;
    const int32_t *seq_lens;
    float *ws_o, *ws_lse;
    int S_max, H, n_hchunk;
    int split, n_split_max;
    float scale_log2;
};

// token index within a tile -> LDS row, for the 16x16 D-layout key assignment:
// MFMA row m of block mb holds token 8*(m>>2) + 4*mb + (m&3).
__device__ __forceinline__ int tok_to_row(int j) {
    return 16 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3);
}

__global__ __launch_bounds__(64 * MAX_WAVES, 1) void mla_decode_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    __bf16 *ks_l = smem;
    __bf16 *vt_l = smem + K_ELEMS;
    const int tid = threadIdx.x;
    constexpr int nthreads = 64 * MAX_WAVES;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c16 = lane & 15;
    const int grp = lane >> 4;

    const int s = blockIdx.x;
    const int hc = blockIdx.y;
    const int b = blockIdx.z;
    int len = p.seq_lens[b];
    len = len < 0 ? 0 : (len > p.S_max ? p.S_max : len);
    if (s * p.split >= len) return;
    const int lo = s * p.split;
    const int hi = min(lo + p.split, len);

    // A chunk is 128 heads; waves past the last head only help stage tiles.
    const int h = hc * 16 * MAX_WAVES + wave * 16 + c16;
    const bool wave_active = hc * 16 * MAX_WAVES + wave * 16 < p.H;   // H % 16 == 0
    bf16x8 qop[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (wave_active) val = ldg16(p.q + ((size_t)b * p.H + h) * DK + 32 * ks + 8 * grp);
        qop[ks] = __builtin_bit_cast(bf16x8, val);
    }

    const __bf16 *cg = p.c + (size_t)b * p.S_max * DK;

    f32x4 oacc[DC / 16];
#pragma unroll
    for (int db = 0; db < DC / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // Tile staging: units u = tid + nthreads*i over 16 token pairs x 72 chunks.
    constexpr int UNITS = (TB / 2) * (DK / 8);   // 1152
    constexpr int MAXU = (UNITS + nthreads - 1) / nthreads;
    u32x4 reg[MAXU][2];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            const int u = tid + nthreads * i;
            const int pr = u / (DK / 8), ch = u % (DK / 8);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int tok = t0 + 2 * pr + e;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (u < UNITS && tok < hi) val = ldg16(cg + (size_t)tok * DK + 8 * ch);
                reg[i][e] = val;
            }
        }
    };
    auto store_tile = [&]() {
        uint32_t *vt32 = reinterpret_cast<uint32_t *>(vt_l);
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            const int u = tid + nthreads * i;
            if (u >= UNITS) continue;
            const int pr = u / (DK / 8), ch = u % (DK / 8);
#pragma unroll
            for (int e = 0; e < 2; ++e)
                *reinterpret_cast<u32x4 *>(ks_l + tok_to_row(2 * pr + e) * KST + 8 * ch) = reg[i][e];
            if (ch < DC / 8) {
                const u32x4 a = reg[i][0], bq = reg[i][1];
#pragma unroll
                for (int st = 0; st < 8; ++st) {
                    const int e = (st + ch) & 7;
                    const uint32_t wa = a[e >> 1], wb = bq[e >> 1];
                    const uint32_t packed = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u))
                                                    : ((wa & 0xffffu) | (wb << 16));
                    vt32[((8 * ch + e) * VTS) / 2 + pr] = packed;
                }
            }
        }
    };

    load_tile(lo);
    for (int t0 = lo; t0 < hi; t0 += TB) {
        __syncthreads();                 // previous tile fully consumed
        store_tile();
        __syncthreads();
        if (t0 + TB < hi) load_tile(t0 + TB);
        if (!wave_active) continue;

        f32x4 sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks_l + (16 * mb + c16) * KST + 32 * ks + 8 * grp);
                sacc[mb] = mfma16x16x32(a, qop[ks], sacc[mb]);
            }
        }
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = t0 + 8 * grp + 4 * mb + i;
                float v = sacc[mb][i] * p.scale_log2;
                v = tok < hi ? v : -INFINITY;
                x[4 * mb + i] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const bool upd = mx > m_run + TAU;
        const float m_new = upd ? mx : m_run;
        const float alpha = upd ? fast_exp2(m_run - m_new) : 1.0f;
        m_run = m_new;
        if (__any(upd)) {
#pragma unroll
            for (int db = 0; db < DC / 16; ++db) oacc[db] *= alpha;
        }
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        float pv[8];
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pv[e] = fast_exp2(x[e] - m_use);
            lsum += pv[e];
        }
        l_run = l_run * alpha + lsum;
        const bf16x8 pop = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
#pragma unroll
        for (int db = 0; db < DC / 16; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vt_l + (16 * db + c16) * VTS + 8 * grp);
            oacc[db] = mfma16x16x32(a, pop, oacc[db]);
        }
    }
    if (!wave_active) return;
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    const size_t ws = ((size_t)b * p.H + h) * p.n_split_max + s;
    float *wo = p.ws_o + ws * DC;
#pragma unroll
    for (int db = 0; db < DC / 16; ++db) {
        const int d = 16 * db + 4 * grp;
        f32x4 v = oacc[db] * inv;
        *reinterpret_cast<f32x4 *>(wo + d) = v;
    }
    if (grp == 0) p.ws_lse[ws] = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;
}

}  // namespace

hipError_t launch_mla_decode_bf16(const MlaArgs &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.c = static_cast<const __bf16 *>(a.cache);
    p.seq_lens = a.seq_lens;
    p.ws_o = a.ws_o;
    p.ws_lse = a.ws_lse;
    p.S_max = a.S_max;
    p.H = a.H;
    p.n_hchunk = (a.H + 16 * MAX_WAVES - 1) / (16 * MAX_WAVES);
    p.split = a.split;
    p.n_split_max = a.n_split_max;
    p.scale_log2 = a.scale * kLog2e;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)mla_decode_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int threads = 64 * MAX_WAVES;
    dim3 grid(a.n_split_max, p.n_hchunk, a.B);
    hipLaunchKernelGGL(mla_decode_kernel, grid, dim3(threads), LDS_BYTES, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_combine(a.ws_o, a.ws_lse, a.seq_lens, a.o, a.lse, a.B, a.H, DC, a.S_max,
                                a.split, a.n_split_max, stream);
}

}  // namespace mi355
