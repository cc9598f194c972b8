// prefill_bf16.hip -- causal / sliding-window / full attention forward for
// bf16 inputs with d_h = 128 on gfx950, using bf16 MFMA for both products.
//
// Method: the FlashAttention-2 tiling and online-softmax recurrence
// ("Attention Engineering: From MHA to GQA, MLA & FlashAttention", section 4,
// equation "FlashAttention-2 Exact Tiled Rescaling Recurrence" and Figure 3):
// a block of query rows stays resident while K/V tiles stream past; the
// running max m, running sum l and unnormalised output are kept in fp32
// registers and the division by l happens once in the epilogue, which also
// stores L = m + ln l.  Causal tiles strictly above the diagonal are never
// visited ("Attention, Worked Out by Hand (Part 2)", section 2).  Query heads
// of one K/V group share the K/V tile staged in LDS ("Attention Engineering",
// section 2, the zero-copy grouped broadcast instead of repeat_interleave).
//
// gfx950 mapping (the pages' kernels target A100/H100 and are prior art only):
//  * workgroup = 4 waves (one per SIMD); each wave owns 64 query rows of one
//    query head; the workgroup covers 1, 2 or 4 heads of the same K/V group;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (A = K rows from LDS, B = the wave's Q rows held in registers).  In the
//    D layout each lane then owns ONE query row (its column), so a row's
//    max/sum is a per-lane reduction plus one exchange with lane l^32;
//  * the P.V product is computed as O^T = V^T P^T: the S^T accumulator,
//    rounded to bf16, is directly the B operand (no LDS round trip for P).
//    For that, key rows are stored in LDS permuted (bits 2 and 3 of the key
//    index swapped) so each lane's eight P values are eight consecutive keys,
//    and V is stored transposed (V^T[d][key]) so the A operand is one 16-byte
//    LDS read;
//  * K/V tiles of 64 keys are double-buffered in LDS, with the next tile's
//    global loads in flight while the current one is consumed (one barrier
//    per tile);
//  * the reference max is only moved when a tile's row max exceeds it by
//    more than 2^8 (exact: every exponent is taken against the same
//    reference max that l and O carry), so the O rescale is rare;
//  * workgroups are ordered heaviest row-block first (causal), and the
//    head-group index is the fastest-varying part of the workgroup id, so
//    with 8 (or a multiple of 8) head groups every workgroup of one K/V head
//    lands on the same XCD (dispatch is round-robin over the 8 XCDs) and
//    shares that XCD's L2.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int D = 128;          // head size
constexpr int BN = 64;          // keys per tile
constexpr int NW = 4;           // waves per workgroup
constexpr int RW = 64;          // query rows per wave (two 32-row MFMA blocks)
constexpr int KS = D + 8;       // LDS row stride of a K row, bf16 elements (272 B)
constexpr int VS = BN + 8;      // LDS row stride of a V^T row, bf16 elements (144 B)
constexpr int K_ELEMS = BN * KS;
constexpr int V_ELEMS = D * VS;
constexpr int STAGE = K_ELEMS + V_ELEMS;   // bf16 elements per buffer stage
constexpr int LDS_BYTES = 2 * STAGE * 2;   // two stages
constexpr float TAU = 8.0f;     // lazy-rescale threshold, log2 units

struct Params {
    const __bf16 *q, *k, *v;
    __bf16 *o;
    float *lse;
    int T, hq, hkv, G;
    int hpw;              // query heads per workgroup (1, 2 or 4)
    int rows_per_wg;      // RW * NW / hpw
    int n_row_blocks;
    int n_head_groups;    // B * hkv * (G / hpw)
    int causal, window;
    float scale_log2;     // scale * log2(e)
};

// Key index <-> LDS row: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int perm_key(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__global__ __launch_bounds__(256, 1) void prefill_bf16_d128_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int id = blockIdx.x;
    const int rb = p.n_row_blocks - 1 - id / p.n_head_groups;
    const int hg = id % p.n_head_groups;
    const int subs = p.G / p.hpw;
    const int sub = hg % subs;
    const int g = (hg / subs) % p.hkv;
    const int b = hg / (subs * p.hkv);
    const int wph = NW / p.hpw;                       // waves per head
    const int h = g * p.G + sub * p.hpw + wave / wph;
    const int r0 = rb * p.rows_per_wg;
    const int rw0 = r0 + (wave % wph) * RW;
    const int T = p.T;

    // Key range of the workgroup and of this wave.
    const int kend = p.causal ? min(T, r0 + p.rows_per_wg) : T;
    const int kbeg = p.window > 0 ? max(0, r0 - p.window + 1) : 0;
    const int t_begin = kbeg / BN;
    const int t_end = (kend + BN - 1) / BN;
    const bool wave_active = rw0 < T;
    const int kend_w = p.causal ? min(T, rw0 + RW) : T;
    const int kbeg_w = p.window > 0 ? max(0, rw0 - p.window + 1) : 0;

    const size_t kv_base = ((size_t)b * p.hkv + g) * (size_t)T * D;
    const __bf16 *kg = p.k + kv_base;
    const __bf16 *vg = p.v + kv_base;
    const size_t q_base = ((size_t)b * p.hq + h) * (size_t)T * D;

    // Q rows of this wave as MFMA B operands: qop[nb][ks], row = rw0 + 32nb + l32,
    // d = 16ks + 8hi .. +7.
    bf16x8 qop[2][8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int row = rw0 + 32 * nb + l32;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4 val = {0u, 0u, 0u, 0u};
            if (row < T) val = ldg16(p.q + q_base + (size_t)row * D + 16 * ks + 8 * hi);
            qop[nb][ks] = __builtin_bit_cast(bf16x8, val);
        }
    }

    f32x16 oacc[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][nb][i] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    // Global -> register staging of one tile.
    // K: 64 rows x 16 chunks of 16 B; thread handles chunks tid + 256 i.
    // V: 32 key pairs x 16 chunks; thread handles pair (tid>>4) + 16 i, chunk tid&15.
    u32x4 kreg[4], vreg[2][2];
    auto load_tile = [&](int t) {
        const int ts = t * BN;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int r = c >> 4, ch = c & 15;
            const int key = ts + r;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (key < T) val = ldg16(kg + (size_t)key * D + 8 * ch);
            kreg[i] = val;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pr = (tid >> 4) + 16 * i, ch = tid & 15;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = ts + 2 * pr + e;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (key < T) val = ldg16(vg + (size_t)key * D + 8 * ch);
                vreg[i][e] = val;
            }
        }
    };
    auto store_tile = [&](int buf) {
        __bf16 *ks_l = smem + buf * STAGE;
        __bf16 *vt_l = ks_l + K_ELEMS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int r = c >> 4, ch = c & 15;
            *reinterpret_cast<u32x4 *>(ks_l + perm_key(r) * KS + 8 * ch) = kreg[i];
        }
        uint32_t *vt32 = reinterpret_cast<uint32_t *>(vt_l);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pr = (tid >> 4) + 16 * i, ch = tid & 15;
            const u32x4 a = vreg[i][0], bq = vreg[i][1];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int e = (s + ch) & 7;            // rotation spreads LDS banks
                const uint32_t wa = a[e >> 1], wb = bq[e >> 1];
                // low halves (even e) or high halves (odd e) of the two keys
                const uint32_t packed = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u))
                                                : ((wa & 0xffffu) | (wb << 16));
                vt32[((8 * ch + e) * VS) / 2 + pr] = packed;
            }
        }
    };

    if (t_begin < t_end) load_tile(t_begin);

    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        store_tile(buf);
        __syncthreads();
        if (t + 1 < t_end) load_tile(t + 1);

        const int ts = t * BN;
        const bool do_tile = wave_active && ts < kend_w && ts + BN > kbeg_w;
        if (do_tile) {
            const __bf16 *ks_l = smem + buf * STAGE;
            const __bf16 *vt_l = ks_l + K_ELEMS;
            // S^T = K Q^T : sacc[kb][nb], 32 keys x 32 rows each.
            f32x16 sacc[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[kb][nb][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        ks_l + (32 * kb + l32) * KS + 16 * ks + 8 * hi);
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        sacc[kb][nb] = mfma32x32x16(a, qop[nb][ks], sacc[kb][nb]);
                }
            }

            const bool need_mask =
                (ts + BN > T) ||
                (p.causal && ts + BN - 1 > rw0) ||
                (p.window > 0 && (rw0 + RW - 1) - ts >= p.window);
            bf16x8 pop[2][2][2];   // [kb][nb][half]
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int row = rw0 + 32 * nb + l32;
                float x[2][16];
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float v = sacc[kb][nb][i] * p.scale_log2;
                        if (need_mask) {
                            const int mrow = 8 * (i >> 2) + 4 * hi + (i & 3);
                            const int key = ts + 32 * kb + perm_key(mrow);
                            bool vis = key < T;
                            if (p.causal) vis = vis && key <= row;
                            if (p.window > 0) vis = vis && (row - key) < p.window;
                            v = vis ? v : -INFINITY;
                        }
                        x[kb][i] = v;
                        mx = fmaxf(mx, v);
                    }
                mx = fmaxf(mx, shfl_xor(mx, 32));
                const float m_old = m_run[nb];
                const bool upd = mx > m_old + TAU;
                const float m_new = upd ? mx : m_old;
                const float alpha = upd ? fast_exp2(m_old - m_new) : 1.0f;
                m_run[nb] = m_new;
                if (__any(upd)) {
#pragma unroll
                    for (int db = 0; db < 4; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[db][nb][i] *= alpha;
                }
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    float pv[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        pv[i] = fast_exp2(x[kb][i] - m_use);
                        lsum += pv[i];
                    }
                    pop[kb][nb][0] = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
                    pop[kb][nb][1] = to_bf16x8(pv[8], pv[9], pv[10], pv[11], pv[12], pv[13], pv[14], pv[15]);
                }
                l_run[nb] = l_run[nb] * alpha + lsum;
            }

            // O^T += V^T P^T
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                            vt_l + (32 * db + l32) * VS + 32 * kb + 16 * half + 8 * hi);
#pragma unroll
                        for (int nb = 0; nb < 2; ++nb)
                            oacc[db][nb] = mfma32x32x16(a, pop[kb][nb][half], oacc[db][nb]);
                    }
        }
    }

    if (!wave_active) return;
    // Epilogue: O = O~ / l, L = m ln2 + ln l.
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int row = rw0 + 32 * nb + l32;
        const float lt = l_run[nb] + shfl_xor(l_run[nb], 32);
        if (row >= T) continue;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        __bf16 *orow = p.o + q_base + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * db + 8 * q4 + 4 * hi;
                u32x2 w = {pack_bf16x2(oacc[db][nb][4 * q4 + 0] * inv, oacc[db][nb][4 * q4 + 1] * inv),
                           pack_bf16x2(oacc[db][nb][4 * q4 + 2] * inv, oacc[db][nb][4 * q4 + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + d) = w;
            }
        if (p.lse && hi == 0) {
            const size_t li = ((size_t)b * p.hq + h) * (size_t)T + row;
            p.lse[li] = lt > 0.f ? m_run[nb] * kLn2 + __logf(lt) : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16_d128(const PrefillArgs &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.k = static_cast<const __bf16 *>(a.k);
    p.v = static_cast<const __bf16 *>(a.v);
    p.o = static_cast<__bf16 *>(a.o);
    p.lse = a.lse;
    p.T = a.T;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.hpw = (p.G % 4 == 0) ? 4 : (p.G % 2 == 0 ? 2 : 1);
    p.rows_per_wg = RW * NW / p.hpw;
    p.n_row_blocks = (a.T + p.rows_per_wg - 1) / p.rows_per_wg;
    p.n_head_groups = a.B * a.hkv * (p.G / p.hpw);
    p.causal = a.causal;
    p.window = a.window;
    p.scale_log2 = a.scale * kLog2e;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_bf16_d128_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const long long nblocks = (long long)p.n_row_blocks * p.n_head_groups;
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_bf16_d128_kernel, dim3((unsigned)nblocks), dim3(256), LDS_BYTES,
                       stream, p);
    return hipGetLastError();
}

}  // namespace mi355
