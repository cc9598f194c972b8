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
//  * workgroup = 8 waves, two per SIMD, so one wave's softmax (VALU, exp)
//    overlaps the other's MFMAs; each wave owns 32 query rows of one query
//    head; the workgroup covers 1, 2, 4 or 8 heads of the same K/V group;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (A = K rows from LDS, B = the wave's Q rows held in registers).  In the
//    D layout each lane owns ONE query row (its column), so a row's max/sum
//    is a per-lane reduction plus one exchange with lane l^32;
//  * the P.V product is computed as O^T = V^T P^T: the S^T accumulator,
//    rounded to bf16, is directly the B operand (no LDS round trip for P);
//    the V^T A operand is read from the row-major V tile with the
//    transposing LDS load ds_read_b64_tr_b16 (two per operand), whose four
//    source rows are exactly the four keys each lane's P values belong to;
//  * K and V tiles (64 keys) are stored row-major in LDS with a 304-byte row
//    stride (19 16-byte slots, 19 = 3 mod 16): 16 consecutive rows of one
//    column land in 16 distinct bank slots (conflict-free 16-byte K reads)
//    and 4 consecutive rows x 32 bytes in 8 distinct slots (conflict-free
//    transposing V reads), while every LDS address stays base + immediate;
//  * tiles are double-buffered in LDS and staged through two register sets,
//    so the global loads of tile t+2 are in flight while tile t is consumed
//    (one barrier per tile);
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
constexpr int NW = 8;           // waves per workgroup
constexpr int RW = 32;          // query rows per wave
constexpr int ROWB = D * 2 + 48;   // LDS row stride of a K/V row (304 B)
constexpr int TILE_BYTES = BN * ROWB;          // 19456 B
constexpr int LDS_BYTES = 4 * TILE_BYTES;      // K[2], V[2]
constexpr float TAU = 8.0f;     // lazy-rescale threshold, log2 units

struct Params {
    const __bf16 *q, *k, *v;
    __bf16 *o;
    float *lse;
    int T, hq, hkv, G;
    int hpw;              // query heads per workgroup (1, 2, 4 or 8)
    int rows_per_wg;      // RW * NW / hpw
    int n_row_blocks;
    int n_head_groups;    // B * hkv * (G / hpw)
    int causal, window;
    float scale_log2;     // scale * log2(e)
};

// byte offset of (row, 16-byte chunk) inside a tile
__device__ __forceinline__ int tile_off(int r, int chunk) { return r * ROWB + (chunk << 4); }

__device__ __forceinline__ bf16x4 lds_tr16(const char *base, int byte_off) {
    return lds_read_tr16(base + byte_off);
}

__global__ __launch_bounds__(512, 1) void prefill_bf16_d128_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int q16 = lane >> 4;      // 16-lane group (for the transposing reads)
    const int j16 = lane & 15;

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
    const int row = rw0 + l32;                        // this lane's query row

    // Q^T B operands: row = rw0 + l32, d = 16ks + 8hi .. +7
    bf16x8 qop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row < T) val = ldg16(p.q + q_base + (size_t)row * D + 16 * ks + 8 * hi);
        qop[ks] = __builtin_bit_cast(bf16x8, val);
    }

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    // Global -> register staging: K and V tiles are 64 rows x 16 chunks
    // (1024 chunks each); thread handles chunks tid and tid + 512 of both.
    // Two register sets: set (t & 1) holds tile t from its load until its store.
    u32x4 kreg[2][2], vreg[2][2];
    auto load_tile = [&](int t, int set) {
        const int ts = t * BN;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 512 * i;
            const int r = c >> 4, ch = c & 15;
            const int key = ts + r;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (key < T) {
                kv = ldg16(kg + (size_t)key * D + 8 * ch);
                vv = ldg16(vg + (size_t)key * D + 8 * ch);
            }
            kreg[set][i] = kv;
            vreg[set][i] = vv;
        }
    };
    auto store_tile = [&](int buf, int set) {
        char *kt = smem + buf * TILE_BYTES;
        char *vt = smem + (2 + buf) * TILE_BYTES;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 512 * i;
            const int r = c >> 4, ch = c & 15;
            *reinterpret_cast<u32x4 *>(kt + tile_off(r, ch)) = kreg[set][i];
            *reinterpret_cast<u32x4 *>(vt + tile_off(r, ch)) = vreg[set][i];
        }
    };

    // Per-lane constant parts of the LDS addresses.
    // K operand (kb, ks): row 32kb + l32, chunk 2ks + hi.
    // V operand (db, kb, half, e4): rows 32kb + 16half + 8e4 + 4hi + (j16>>2),
    //   chunk 4db + 2(q16&1) + ((j16&3)>>1), byte 8*(j16&1).
    const int v_row_lane = 4 * hi + (j16 >> 2);
    const int v_chunk_lane = 2 * (q16 & 1) + ((j16 & 3) >> 1);
    const int v_byte_lane = 8 * (j16 & 1);

    if (t_begin < t_end) load_tile(t_begin, 0);
    if (t_begin + 1 < t_end) load_tile(t_begin + 1, 1);

    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        // register set `buf` holds tile t; after the store it takes tile t+2
        if (buf == 0) store_tile(0, 0); else store_tile(1, 1);
        __syncthreads();
        if (t + 2 < t_end) { if (buf == 0) load_tile(t + 2, 0); else load_tile(t + 2, 1); }

        const int ts = t * BN;
        const bool do_tile = wave_active && ts < kend_w && ts + BN > kbeg_w;
        if (!do_tile) continue;
        const char *kt = smem + buf * TILE_BYTES;
        const char *vt = smem + (2 + buf) * TILE_BYTES;

        // S^T = K Q^T : sacc[kb], 32 keys x 32 rows each.
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int r = 32 * kb + l32;
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kt + tile_off(r, 2 * ks + hi));
                sacc[kb] = mfma32x32x16(a, qop[ks], sacc[kb]);
            }
        }

        const bool need_mask =
            (ts + BN > T) ||
            (p.causal && ts + BN - 1 > rw0) ||
            (p.window > 0 && (rw0 + RW - 1) - ts >= p.window);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float v = sacc[kb][i] * p.scale_log2;
                if (need_mask) {
                    const int key = ts + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
                    bool vis = key < T;
                    if (p.causal) vis = vis && key <= row;
                    if (p.window > 0) vis = vis && (row - key) < p.window;
                    v = vis ? v : -INFINITY;
                }
                sacc[kb][i] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const bool upd = mx > m_run + TAU;
        const float m_new = upd ? mx : m_run;
        const float alpha = upd ? fast_exp2(m_run - m_new) : 1.0f;
        m_run = m_new;
        if (__any(upd)) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        float lsum = 0.f;
        bf16x8 pop[2][2];   // [kb][half]
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float pv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                pv[i] = fast_exp2(sacc[kb][i] - m_use);
                lsum += pv[i];
            }
            pop[kb][0] = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
            pop[kb][1] = to_bf16x8(pv[8], pv[9], pv[10], pv[11], pv[12], pv[13], pv[14], pv[15]);
        }
        l_run = l_run * alpha + lsum;

        // O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int rA = 32 * kb + 16 * half + v_row_lane;
                    const int ch = 4 * db + v_chunk_lane;
                    const bf16x4 lo4 = lds_tr16(vt, tile_off(rA, ch) + v_byte_lane);
                    const bf16x4 hi4 = lds_tr16(vt, tile_off(rA + 8, ch) + v_byte_lane);
                    const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                    oacc[db] = mfma32x32x16(a, pop[kb][half], oacc[db]);
                }
    }

    if (!wave_active) return;
    // Epilogue: O = O~ / l, L = m ln2 + ln l.
    const float lt = l_run + shfl_xor(l_run, 32);
    if (row >= T) return;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    __bf16 *orow = p.o + q_base + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * db + 8 * q4 + 4 * hi;
            u32x2 w = {pack_bf16x2(oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv),
                       pack_bf16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv)};
            *reinterpret_cast<u32x2 *>(orow + d) = w;
        }
    if (p.lse && hi == 0) {
        const size_t li = ((size_t)b * p.hq + h) * (size_t)T + row;
        p.lse[li] = lt > 0.f ? m_run * kLn2 + __logf(lt) : -INFINITY;
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
    p.hpw = (p.G % 8 == 0) ? 8 : (p.G % 4 == 0) ? 4 : (p.G % 2 == 0 ? 2 : 1);
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
    hipLaunchKernelGGL(prefill_bf16_d128_kernel, dim3((unsigned)nblocks), dim3(64 * NW), LDS_BYTES,
                       stream, p);
    return hipGetLastError();
}

}  // namespace mi355
