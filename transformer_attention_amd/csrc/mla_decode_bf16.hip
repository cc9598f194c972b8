// mla_decode_bf16.hip -- Multi-head Latent Attention decode with absorbed
// up-projections (d_c = 512 latent + d_r = 64 decoupled RoPE key), bf16 on gfx950.
//
// Method ("Attention Engineering: From MHA to GQA, MLA & FlashAttention",
// section 3): with W_UK folded into the query and W_UV into the output
// projection, every head scores its 576-wide query [q~ ; q_R] against the
// shared per-token cache row [c_KV ; k_R] (equation "Complete MLA Attention
// Score", scale 1/sqrt(d_h + d_R)) and mixes the latent rows c_KV themselves:
// the value of token j is the first 512 entries of the same cache row.  All
// heads read the same cache, so one workgroup processes all (up to 128) heads
// of a sequence against one chunk of the cache, and every cache byte is read
// from HBM once; the chunks are merged by the log-sum-exp combine shared with
// the GQA decode (the FlashAttention-2 state merge, section 4).
//
// gfx950 mapping:
//  * 32-token tiles [32 x 576 bf16 = 36 KB] stream HBM -> LDS through a
//    4-stage ring filled by global_load_lds_dwordx4 (no staging registers),
//    three tiles in flight per CU while the fourth is consumed;
//  * each tile is stored once, row-major with its 16-byte chunks XOR-swizzled
//    per row; the score product reads it with 16-byte loads, the P.V product
//    reads the first 512 columns transposed with ds_read_b64_tr_b16, so the
//    latent is never copied;
//  * 8 waves (two per SIMD), each owning 16 heads: S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16 (the wave's 16 queries, 576 wide, stay in
//    registers as B operands), then O^T[512 x 16] += C^T P^T with the rounded
//    probabilities as the B operand (the two 16-token halves of the tile
//    form the 32-token K dimension);
//  * the online-softmax state is per head (one lane column), and the
//    reference max only moves when a tile exceeds it by 2^8.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int DC = 512, DR = 64, DK = DC + DR;
constexpr int TB = 32;                    // tokens per tile
constexpr int ROWB = DK * 2;              // 1152 bytes per cache row in HBM
constexpr int LROW = ROWB + 16;           // LDS row stride: 73 16-byte slots
constexpr int TILE_BYTES = 37 * 1024;     // 32 padded rows (37376 B) rounded up to whole DMA blocks
constexpr int NSTAGE = 4;
constexpr int LDS_BYTES = NSTAGE * TILE_BYTES;   // 151552
constexpr int NW = 8;                     // waves per workgroup
constexpr int HPW = 16;                   // heads per wave
constexpr int HPC = NW * HPW;             // heads per workgroup (chunk)
constexpr int NBLK = TILE_BYTES / 1024;   // 37 one-KB DMA blocks per tile:
                                          // waves 0-4 issue 5, waves 5-7 issue 4
constexpr float TAU = 8.0f;

struct Params {
    const __bf16 *q, *c;
    const int32_t *seq_lens;
    float *ws_o, *ws_lse;
    int S_max, H;
    int split, n_split_max;
    float scale_log2;
};

// Row r of a tile starts at 1168 r: 1168 = 73 * 16 and 73 = 9 (mod 16), so
// 16 consecutive rows fall in 16 distinct 16-byte bank slots (conflict-free
// 16-byte reads down a column) and 4 consecutive rows x 32 bytes fall in 8
// distinct slots (conflict-free transposing reads); addresses stay affine.
__device__ __forceinline__ int tile_off(int r, int chunk) { return r * LROW + (chunk << 4); }

__global__ __launch_bounds__(64 * NW, 1) void mla_decode_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int q16 = lane >> 4;
    const int j16 = lane & 15;

    const int s = blockIdx.x;
    const int hc = blockIdx.y;
    const int b = blockIdx.z;
    int len = p.seq_lens[b];
    len = len < 0 ? 0 : (len > p.S_max ? p.S_max : len);
    if (s * p.split >= len) return;
    const int lo = s * p.split;
    const int hi_tok = min(lo + p.split, len);
    const int n_tiles = (hi_tok - lo + TB - 1) / TB;

    const char *cg = reinterpret_cast<const char *>(p.c + (size_t)b * p.S_max * DK);

    // Issue the DMA of tile `t` (relative) into its ring stage: this wave's
    // 1-KB blocks.  LDS byte o = 1024*blk + 16*lane of the stage holds
    // (row o / 1168, chunk (o % 1168) / 16); the pad slot (chunk 72) and the
    // bytes past row 31 receive an arbitrary valid chunk.  Rows past the
    // chunk end re-read the last valid row (their scores are masked).
    const int my_blk0 = wave < 5 ? 5 * wave : 25 + 4 * (wave - 5);
    const int my_nblk = wave < 5 ? 5 : 4;
    auto issue_tile = [&](int t) {
        char *stage = smem + (t % NSTAGE) * TILE_BYTES;
        const int t0 = lo + t * TB;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            if (i >= my_nblk) break;
            const int blk = my_blk0 + i;
            const int o = blk * 1024 + lane * 16;
            const int r = min(o / LROW, TB - 1);
            const int ch = min((o - (o / LROW) * LROW) >> 4, DK / 8 - 1);
            const int tok = min(t0 + r, hi_tok - 1);
            dma16(cg + (size_t)tok * ROWB + ch * 16, stage + blk * 1024);
        }
    };

    // Prologue: tiles 0..NSTAGE-2 in flight.
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t)
        if (t < n_tiles) issue_tile(t);

    // The wave's 16 queries as B operands: head = hc*128 + 16*wave + j16,
    // d = 32ks + 8*q16 .. +7.
    const int h = hc * HPC + wave * HPW + j16;
    const bool head_ok = h < p.H;
    bf16x8 qop[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (head_ok) val = ldg16(p.q + ((size_t)b * p.H + h) * DK + 32 * ks + 8 * q16);
        qop[ks] = __builtin_bit_cast(bf16x8, val);
    }

    f32x4 oacc[DC / 16];
#pragma unroll
    for (int db = 0; db < DC / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // C^T operand (16 d x 32 tokens) through the transposing read: lane j of
    // 16-lane group q16 addresses token row 4*q16 + j/4 (second read: +16),
    // d = 16db + 4(j%4) .. +3, i.e. chunk 2db + (j%4)/2, byte 8(j%2).
    const int v_row_lane = 4 * q16 + (j16 >> 2);
    const int v_chunk_lane = (j16 & 3) >> 1;
    const int v_byte_lane = 8 * (j16 & 1);

    for (int t = 0; t < n_tiles; ++t) {
        // Tile t landed once at most (NSTAGE-2) newer tiles are pending.  The
        // q loads above were issued after the prologue DMAs, so the first
        // iteration waits for everything.
        const int newer = t == 0 ? 0 : min(NSTAGE - 2, n_tiles - 1 - t);
        if (newer == 0) wait_vmcnt<0>();
        else if (newer == 1) { if (my_nblk == 5) wait_vmcnt<5>(); else wait_vmcnt<4>(); }
        else { if (my_nblk == 5) wait_vmcnt<10>(); else wait_vmcnt<8>(); }
        raw_barrier();                          // every wave's part of tile t is in LDS,
                                                // and stage (t-1) is no longer read
        if (t + NSTAGE - 1 < n_tiles) issue_tile(t + NSTAGE - 1);

        const char *kt = smem + (t % NSTAGE) * TILE_BYTES;
        const int t0 = lo + t * TB;
        // S^T (two 16-token blocks x 16 heads): token 16mb + j16, d chunk 4ks + q16
        f32x4 sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kt + tile_off(16 * mb + j16, 4 * ks + q16));
                sacc[mb] = mfma16x16x32(a, qop[ks], sacc[mb]);
                if ((ks & 5) == 5) __builtin_amdgcn_sched_barrier(0);   // bound the load look-ahead
            }
        }
        // element (mb, i) of this lane is token t0 + 16mb + 4*q16 + i of head column j16
        const bool tail = t0 + TB > hi_tok;
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = sacc[mb][i] * p.scale_log2;
                if (tail) {
                    const int tok = t0 + 16 * mb + 4 * q16 + i;
                    v = tok < hi_tok ? v : -INFINITY;
                }
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
            const int ch = 2 * db + v_chunk_lane;
            const bf16x4 lo4 = lds_read_tr16(kt + tile_off(v_row_lane, ch) + v_byte_lane);
            const bf16x4 hi4 = lds_read_tr16(kt + tile_off(v_row_lane + 16, ch) + v_byte_lane);
            const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = mfma16x16x32(a, pop, oacc[db]);
            if ((db & 3) == 3) __builtin_amdgcn_sched_barrier(0);      // bound the load look-ahead
        }
    }

    float lt = l_run + shfl_xor(l_run, 16);
    lt += shfl_xor(lt, 32);
    if (!head_ok) return;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const size_t ws = ((size_t)b * p.H + h) * p.n_split_max + s;
    float *wo = p.ws_o + ws * DC;
    // O^T element i of d-block db is d = 16db + 4*q16 + i of head column j16
#pragma unroll
    for (int db = 0; db < DC / 16; ++db)
        *reinterpret_cast<f32x4 *>(wo + 16 * db + 4 * q16) = oacc[db] * inv;
    if (q16 == 0) p.ws_lse[ws] = lt > 0.f ? m_run + __log2f(lt) : -INFINITY;
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
    const int n_hchunk = (a.H + HPC - 1) / HPC;
    dim3 grid(a.n_split_max, n_hchunk, a.B);
    hipLaunchKernelGGL(mla_decode_kernel, grid, dim3(64 * NW), LDS_BYTES, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_combine(a.ws_o, a.ws_lse, a.seq_lens, a.o, a.lse, a.B, a.H, DC, a.S_max,
                                a.split, a.n_split_max, stream);
}

}  // namespace mi355
