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
// one workgroup handles one chunk for all query heads of the group (up to 16
// per workgroup), so every K/V byte is read once.  Inside a workgroup each of
// the 4 waves streams 32-key blocks:
//  * S^T = K q^T with v_mfma_f32_16x16x32_bf16: K rows go straight from global
//    memory into the A operand (16-byte loads), q is held in registers as the
//    B operand (the group's heads are the 16 columns);
//  * the 16x16 D layout gives each lane four keys of one head; the two
//    16-key blocks are assigned keys so that each lane's eight probabilities
//    are eight consecutive keys, which makes P^T directly the B operand of
//    O^T = V^T P^T;
//  * V is written transposed into a wave-private LDS area (coalesced 16-byte
//    global loads of key pairs, 32-bit LDS writes) and read back as 16-byte
//    A operands;
//  * the next block's K/V loads are issued before the current block is
//    consumed.
// The running (m, l, O) of the four waves are merged through LDS and the
// chunk's normalised partial output and log-sum-exp are written to the
// workspace; a second kernel merges the chunks of each (sequence, head):
// L = log sum_s exp(L_s), O = sum_s exp(L_s - L) O_s, which is the
// FlashAttention-2 state merge ("Attention Engineering ...", section 4).
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int D = 128;
constexpr int KB = 32;          // keys per wave step
constexpr int NW = 4;           // waves per workgroup
constexpr int VTS = KB + 8;     // LDS row stride of V^T, bf16 elements (80 B)
constexpr int VT_WAVE = D * VTS;  // bf16 elements per wave
constexpr float TAU = 8.0f;

struct Params {
    const __bf16 *q, *k, *v;
    const int32_t *seq_lens;
    float *ws_o, *ws_lse;
    int S_max, hq, hkv, G, n_hchunk;
    int split, n_split_max, window;
    float scale_log2;
};

__global__ __launch_bounds__(256) void decode_bf16_d128_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) __bf16 smem[NW * VT_WAVE];   // 40 KB
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c16 = lane & 15;
    const int grp = lane >> 4;

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

    const int hidx = hc * 16 + c16;                       // head within the group
    const bool head_ok = hidx < p.G;
    const int h = g * p.G + hidx;

    // q^T as B operand: column = head, K = d (four quarters of 32).
    bf16x8 qop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (head_ok) val = ldg16(p.q + ((size_t)b * p.hq + h) * D + 32 * ks + 8 * grp);
        qop[ks] = __builtin_bit_cast(bf16x8, val);
    }

    const size_t kv_base = ((size_t)b * p.hkv + g) * (size_t)p.S_max * D;
    const __bf16 *kg = p.k + kv_base;
    const __bf16 *vg = p.v + kv_base;
    __bf16 *vt = smem + wave * VT_WAVE;
    uint32_t *vt32 = reinterpret_cast<uint32_t *>(vt);

    f32x4 oacc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // Register staging of one 32-key block starting at kb0.
    // K: A operand for block mb, quarter ks: lane row r = c16 holds key
    //    kb0 + 8*(r>>2) + 4*mb + (r&3), d = 32ks + 8grp.
    // V: key pairs (2pr, 2pr+1), pr = grp + 4j, chunk c16.
    u32x4 kreg[2][4], vreg[4][2];
    auto load_block = [&](int kb0) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int key = kb0 + 8 * (c16 >> 2) + 4 * mb + (c16 & 3);
            const bool ok = key >= lo && key < hi;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4 val = {0u, 0u, 0u, 0u};
                if (ok) val = ldg16(kg + (size_t)key * D + 32 * ks + 8 * grp);
                kreg[mb][ks] = val;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = kb0 + 2 * (grp + 4 * j) + e;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (key >= lo && key < hi) val = ldg16(vg + (size_t)key * D + 8 * c16);
                vreg[j][e] = val;
            }
    };

    // blocks handled by this wave: kb0 = lo + KB * (wave + NW * n)
    int kb0 = lo + KB * wave;
    if (kb0 < hi) load_block(kb0);
    for (; kb0 < hi; kb0 += KB * NW) {
        // V^T into the wave's LDS area (rotated element order spreads banks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pr = grp + 4 * j;
            const u32x4 a = vreg[j][0], bq = vreg[j][1];
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const int e = (st + c16) & 7;
                const uint32_t wa = a[e >> 1], wb = bq[e >> 1];
                const uint32_t packed = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u))
                                                : ((wa & 0xffffu) | (wb << 16));
                vt32[((8 * c16 + e) * VTS) / 2 + pr] = packed;
            }
        }
        bf16x8 kop[2][4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kop[mb][ks] = __builtin_bit_cast(bf16x8, kreg[mb][ks]);
        const int cur = kb0;
        if (kb0 + KB * NW < hi) load_block(kb0 + KB * NW);

        f32x4 sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sacc[mb] = mfma16x16x32(kop[mb][ks], qop[ks], sacc[mb]);
        }
        // element (mb, i) of this lane is key cur + 8*grp + 4*mb + i
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = cur + 8 * grp + 4 * mb + i;
                float v = sacc[mb][i] * p.scale_log2;
                v = (key >= lo && key < hi) ? v : -INFINITY;
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
            for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
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
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vt + (16 * db + c16) * VTS + 8 * grp);
            oacc[db] = mfma16x16x32(a, pop, oacc[db]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // Per-wave state: m_run (same in all lanes of a column), l partial per lane.
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);

    // Merge the four waves through LDS (reusing the V^T area).
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);        // [NW][16 heads][D] + m, l
    float *red_m = red + NW * 16 * D;
    float *red_l = red_m + NW * 16;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 16 * db + 4 * grp + i;
            red[(wave * 16 + c16) * D + d] = oacc[db][i];
        }
    if (grp == 0) {
        red_m[wave * 16 + c16] = m_run;
        red_l[wave * 16 + c16] = l_run;
    }
    __syncthreads();
    // 256 threads: head = tid >> 4 (16 heads), d-range (tid & 15) * 8 .. +7
    {
        const int hh = tid >> 4;
        const int d0 = (tid & 15) * 8;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w * 16 + hh]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, wgt[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            wgt[w] = fast_exp2(red_m[w * 16 + hh] - Mu);
            L += wgt[w] * red_l[w * 16 + hh];
        }
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const int hidx2 = hc * 16 + hh;
        if (hidx2 < p.G) {
            const int h2 = g * p.G + hidx2;
            const size_t ws = (((size_t)b * p.hq + h2) * p.n_split_max + s);
            float *wo = p.ws_o + ws * D;
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) acc += wgt[w] * red[(w * 16 + hh) * D + d0 + dd];
                wo[d0 + dd] = acc * inv;
            }
            if ((tid & 15) == 0) p.ws_lse[ws] = L > 0.f ? Mu + __log2f(L) : -INFINITY;
        }
    }
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
    dim3 grid(a.n_split_max, a.hkv * p.n_hchunk, a.B);
    hipLaunchKernelGGL(decode_bf16_d128_kernel, grid, dim3(256), 0, stream, p);
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
