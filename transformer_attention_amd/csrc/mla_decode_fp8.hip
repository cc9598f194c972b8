// mla_decode_fp8.hip -- MLA absorbed decode (d_c = 512 latent + d_r = 64
// RoPE key) with FP8 attention on gfx950: both products on E4M3 MFMAs.
//
// Method: the pages' FP8 attention ("Flash Attention 3 and Multi-Headed
// Latent Attention", the FP8 attention section and its per-tile block
// processor: q, k, v and p quantised to E4M3 with scale amax / 448, both
// matrix products on FP8 operands, results dequantised by the scales) on the
// MLA decode of "Attention Engineering: From MHA to GQA, MLA &
// FlashAttention", section 3 (every head scores its 576-wide absorbed query
// against the shared cache row [c_KV ; k_R] and mixes the latent rows c_KV).
//  * The cache is E4M3 codes with one scale per 32 tokens (the FP8 cache
//    quantiser's tiles with h_kv = 1); the query row of each head is
//    quantised the same way (one scale per row) into the workspace before
//    this kernel runs.  k and v share the codes and the scale.
//  * s_j = scale * sq * sc_j * (q8 . c8_j): the FP8 product, scaled once.
//  * The weight of token j in the value product carries its tile's scale:
//    y_j = s_j log2(e) + log2(sc_j).  Each chunk keeps a reference R: before
//    a 64-token compute tile's weights are taken, if the tile's max of y
//    exceeds R, R moves to that max plus HEADROOM (5, log2 units) and the
//    output accumulated so far is rescaled by 2^(R_old - R_new).  The
//    rescale touches all 256 accumulators of a wave whenever any of its 32
//    heads moves: moving R to every new max did that on most tiles, and with
//    3 units of headroom still on about a third of them; with 5 a head must
//    rise 32x to move it again.  The weights are quantised as e = 448 *
//    2^(y - R) -> E4M3 (the page's p / (amax / 448) with amax bounded by
//    2^R: no weight passes 448), and the product accumulates e * c8.
//    Folding the value scale into the weight lets one 64-token FP8 product
//    span two 32-token scale tiles.
//  * The denominator is the unquantised sum of 2^(s log2 e - R) = e / (448
//    sc) (the page normalises the softmax before quantising p); the chunk's
//    output is acc / (448 l), its log-sum-exp R + log2 l.  Chunks merge in
//    the log-sum-exp combine shared with the bf16 decodes.
//
// gfx950 mapping:
//  * one workgroup = one sequence x one cache chunk x 128 heads, 4 waves of
//    32 heads, one wave per SIMD;
//  * 64-token tiles [64 x 576 B] stream HBM -> LDS through a 4-stage ring of
//    global_load_lds_dwordx4 copies (non-temporal: read once);
//  * S^T [64 tokens x 32 heads] = C Q^T with v_mfma_f32_32x32x64_f8f6f4: A =
//    32 bytes of a cache row from LDS, B = the head's query codes in
//    registers (9 k-steps of 64 per 32-token block);
//  * O^T [512 x 32 heads] += C^T P^T with one 32x32x64 FP8 MFMA per 32 d
//    (K = the tile's 64 tokens): B = the lane's own 32 weights (16 of each
//    32-token block, converted to E4M3 in registers), A = the latent read
//    transposed from the same LDS tile with ds_read_b64_tr_b8, four reads
//    whose token rows are exactly the tokens the lane's weights belong to;
//  * rows sit 36 slots (576 B) apart with a drift of one 16-byte slot every
//    4 rows, so the 16-row score reads of a quarter wave and the 8-row
//    transposing reads of a half wave are bank-conflict free;
//  * MFMA operand pairing: the FP8 MFMA multiplies byte b of lane-half h of
//    A with byte b of lane-half h of B (measured on the hardware), so any
//    token order inside the K dimension works as long as A and B agree.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int DC = 512, DR = 64, DK = DC + DR;
constexpr int TB = 64;                    // tokens per compute tile
constexpr int SCALE_TILE = 32;            // tokens per cache scale
constexpr int ROWS = DK;                  // 576 bytes per cache row (codes)
constexpr int PITCH = DK / 16;            // 36 slots per row in LDS
constexpr int TILE_BYTES = 37 * 1024;     // last row ends at slot 36*63 + 15 + 36 = 2319
constexpr int NBLK = TILE_BYTES / 1024;   // 37 one-KB copies per tile
constexpr int NSTAGE = 4;
constexpr int LDS_BYTES = NSTAGE * TILE_BYTES;   // 151552
constexpr int NW = 4;                     // waves per workgroup
constexpr int HPW = 32;                   // heads per wave
constexpr int HPC = NW * HPW;             // heads per workgroup
constexpr float LOG2_448 = 8.807354922057604f;
constexpr float HEADROOM = 5.0f;          // log2 units above a new max

typedef __attribute__((ext_vector_type(8))) int i32x8;

struct Params {
    const uint8_t *q8;          // [B, H, DK] query codes (workspace)
    const float *qs;            // [B, H] query scales
    const uint8_t *c;           // [B, S_max, DK] cache codes
    const float *cs;            // [B, n_stiles] cache scales
    const int32_t *seq_lens;
    __bf16 *ws_o;
    float *ws_lse;
    int B, S_max, H, n_stiles;
    int split, n_split_max, n_hchunk;
    float scale_log2;           // scale * log2(e)
};

// LDS slot of row r (16-byte units): 36 r plus one slot every 4 rows.
__device__ __forceinline__ int row_slot(int r) { return PITCH * r + (r >> 2); }

// FP8 MFMA wrappers (inline asm; the hazards the compiler cannot see are
// covered as for the bf16 score MFMAs in kcommon.h: the first of a chain
// waits 5 cycles after VALU writes of its operands, the last is followed by
// 21 wait states before VALU reads of its 16-pass result).
__device__ __forceinline__ f32x16 mfma8_first(i32x8 a, i32x8 b) {
    f32x16 d;
    asm("s_nop 4\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ f32x16 mfma8_acc(i32x8 a, i32x8 b, f32x16 c) {
    asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    return c;
}
__device__ __forceinline__ f32x16 mfma8_last(i32x8 a, i32x8 b, f32x16 c) {
    asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
        : "+v"(c) : "v"(a), "v"(b));
    return c;
}
// Output product through the compiler (it tracks the hazards and keeps the
// accumulators in AGPRs): the block-scaled form with both scale exponents
// 127, i.e. x 1.0 -- the plain FP8 product.
__device__ __forceinline__ f32x16 mfma8_o(i32x8 a, i32x8 b, f32x16 acc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 lds32(const char *p) {       // 32 bytes as two 16-byte reads
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// four E4M3 codes of a, b, c, d (bytes 0..3, round to nearest even; the
// callers' values are at most 448 * (1 + 2^-20), which rounds to 448)
// Four E4M3 codes in one word.  The first conversion writes the low half and
// keeps the high half of `old`, which the second then overwrites: passing the
// word's previous contents (rather than 0) spares a register clear per word.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d, int old) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__global__ __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_fp8_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // workgroup id -> (sequence fastest, split, head chunk)
    const int id = blockIdx.x;
    const int b = id % p.B;
    const int rest = id / p.B;
    const int s = rest % p.n_split_max;
    const int hc = rest / p.n_split_max;
    int len = p.seq_lens[b];
    len = len < 0 ? 0 : (len > p.S_max ? p.S_max : len);
    if (s * p.split >= len) return;
    const int lo = s * p.split;
    const int hi_tok = min(lo + p.split, len);
    const int n_tiles = (hi_tok - lo + TB - 1) / TB;
    const uint8_t *cg = p.c + (size_t)b * p.S_max * ROWS;
    const float *csb = p.cs + (size_t)b * p.n_stiles;

    // Copies: LDS slot q = 64 blk + lane of a tile holds row r (the last row
    // with row_slot(r) <= q), chunk q - row_slot(r); pad slots and slots past
    // row 63 receive a valid chunk nobody reads.  Wave 0 issues 10 blocks,
    // waves 1-3 issue 9.
    const int my_blk0 = wave == 0 ? 0 : 10 + 9 * (wave - 1);
    const int my_nblk = wave == 0 ? 10 : 9;
    uint32_t dma_off[10];
    int dma_row[10];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const int q = (my_blk0 + min(i, my_nblk - 1)) * 64 + lane;
        int r = (4 * q) / 145;
        if (r < TB - 1 && row_slot(r + 1) <= q) ++r;
        if (row_slot(r) > q) --r;
        r = min(r, TB - 1);
        const int c = min(q - row_slot(r), PITCH - 1);
        dma_row[i] = r;
        dma_off[i] = (uint32_t)(r * ROWS + c * 16);
    }
    auto issue_tile = [&](int t) {
        char *stage = smem + (t % NSTAGE) * TILE_BYTES;
        const int t0 = lo + t * TB;
        const uint8_t *gbase = cg + (size_t)t0 * ROWS;
        // last valid row of this tile (opaque to the compiler: as an affine
        // function of the tile it was strength-reduced into per-lane counters
        // updated every tile)
        int last = hi_tok - 1 - t0;
        asm volatile("" : "+s"(last));
        if (last >= TB - 1) {
#pragma unroll
            for (int i = 0; i < 10; ++i) {
                if (i >= my_nblk) break;
                dma16_off<true>(gbase, dma_off[i], stage + (my_blk0 + i) * 1024);
            }
        } else {                                    // ragged last tile: rows past the end re-read the last row
#pragma unroll
            for (int i = 0; i < 10; ++i) {
                if (i >= my_nblk) break;
                const uint32_t off = dma_row[i] > last
                    ? dma_off[i] - (uint32_t)((dma_row[i] - last) * ROWS) : dma_off[i];
                dma16_off<true>(gbase, off, stage + (my_blk0 + i) * 1024);
            }
        }
    };

#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t)
        if (t < n_tiles) issue_tile(t);

    // The wave's 32 query heads as B operands: k-step ks holds d = 64 ks + 32 hh .. +31.
    const int h = hc * HPC + wave * HPW + l32;
    const bool head_ok = h < p.H;
    i32x8 qop[DK / 64];
    float a_h = 0.f;                                 // scale * log2(e) * sq
    {
        const size_t qrow = ((size_t)b * p.H + (head_ok ? h : 0));
        const uint8_t *qp = p.q8 + qrow * DK + 32 * hh;
#pragma unroll
        for (int ks = 0; ks < DK / 64; ++ks) {
            const u32x4 x0 = ldg16(qp + 64 * ks);
            const u32x4 x1 = ldg16(qp + 64 * ks + 16);
            qop[ks] = head_ok ? i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                      (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]}
                              : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        a_h = p.scale_log2 * p.qs[qrow];
    }

    f32x16 oacc[DC / 32];
#pragma unroll
    for (int db = 0; db < DC / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float R = -INFINITY, l_run = 0.f;
    i32x8 pop = {0, 0, 0, 0, 0, 0, 0, 0};          // the tile's E4M3 weights (P.V B operand)

    // Score A operand: row 32 blk + l32, bytes 64 ks + 32 hh .. +31.
    const char *srow = smem + 16 * (row_slot(l32) + 2 * hh);
    constexpr int BLK_SLOTS = 32 * PITCH + 8;        // row_slot(r + 32) - row_slot(r)
    // Transposing read j of a d-block: lane L of 16-lane group G (hh = G/2,
    // d-half G%2) addresses token row 16 (j%2) + 32 (j/2) + 8 (r/4) + 4 hh +
    // r%4 with r = L/2, 8 bytes at d = 32 db + 16 (G%2) + 8 (L%2).
    const int g16 = lane >> 4, L16 = lane & 15, rr = L16 >> 1;
    const int v_tok = 8 * (rr >> 2) + 4 * (g16 >> 1) + (rr & 3);
    const int v_lane = 16 * row_slot(v_tok) + 16 * (g16 & 1) + 8 * (L16 & 1);
    auto v_off = [](int j) {                         // row_slot(T + 16 (j%2) + 32 (j/2)) - row_slot(T)
        const int tj = 16 * (j & 1) + 32 * (j >> 1);
        return 16 * (PITCH * tj + tj / 4);
    };

    for (int t = 0; t < n_tiles; ++t) {
        const int newer = t == 0 ? 0 : min(NSTAGE - 2, n_tiles - 1 - t);
        if (newer == 0) wait_vmcnt<0>();
        else if (newer == 1) { if (my_nblk == 10) wait_vmcnt<10>(); else wait_vmcnt<9>(); }
        else { if (my_nblk == 10) wait_vmcnt<20>(); else wait_vmcnt<18>(); }
        raw_barrier();

        const char *kt = smem + (t % NSTAGE) * TILE_BYTES;
        const int t0 = lo + t * TB;
        // scale tiles of the two 32-token blocks (the second only if it exists)
        const int st0 = t0 / SCALE_TILE;
        const float sc0 = ld_uniform_f(csb, st0);
        const float sc1 = t0 + SCALE_TILE < hi_tok ? ld_uniform_f(csb, st0 + 1) : sc0;

        // S^T of the two 32-token blocks as two interleaved chains (step j:
        // block j % 2, k-step j / 2), so consecutive MFMAs are independent;
        // the A operand of step j + PF is read before the MFMA of step j
        constexpr int NKS = DK / 64;
        constexpr int PF = 2;
        const char *ra = kt + (srow - smem);
        auto a_at = [&](int j) { return lds32(ra + 16 * BLK_SLOTS * (j % 2) + 64 * (j / 2)); };
        f32x16 sacc[2];
        i32x8 ka[PF + 1];
#pragma unroll
        for (int i = 0; i < PF; ++i) ka[i] = a_at(i);
#pragma unroll
        for (int j = 0; j < 2 * NKS; ++j) {
            if (j + PF < 2 * NKS) ka[(j + PF) % (PF + 1)] = a_at(j + PF);
            const int blk = j % 2, ks = j / 2;
            const i32x8 a = ka[j % (PF + 1)];
            if (ks == 0) sacc[blk] = mfma8_first(a, qop[0]);
            else if (j == 2 * NKS - 1) sacc[blk] = mfma8_last(a, qop[ks], sacc[blk]);
            else sacc[blk] = mfma8_acc(a, qop[ks], sacc[blk]);
            __builtin_amdgcn_sched_barrier(0);
            if (j == 2 && t + NSTAGE - 1 < n_tiles) {
                issue_tile(t + NSTAGE - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // element i of block blk is token t0 + 32 blk + 8 (i/4) + 4 hh + i%4 of head l32
        if (t0 + TB > hi_tok) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tok = t0 + 32 * blk + 8 * (i >> 2) + 4 * hh + (i & 3);
                    sacc[blk][i] = tok < hi_tok ? sacc[blk][i] : -INFINITY;
                }
        }
        const float A0 = a_h * sc0, A1 = a_h * sc1;
        const float lb0 = __log2f(sc0), lb1 = __log2f(sc1);
        float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mx0 = fmaxf(mx0, sacc[0][i]);
            mx1 = fmaxf(mx1, sacc[1][i]);
        }
        const float ym = fmaxf(__builtin_fmaf(mx0, A0, lb0), __builtin_fmaf(mx1, A1, lb1));
        if (__any(ym > R)) {                         // the reference moves (tile 0 always)
            const float yh = pair32_max(ym);
            if (yh > R) {
                const float Rn = yh + HEADROOM;
                const float f = fast_exp2(R - Rn);   // 0 while R = -inf
                if (t > 0) {
#pragma unroll
                    for (int db = 0; db < DC / 32; ++db) scale_acc(oacc[db], f);
                }
                l_run *= f;
                R = Rn;
            }
        }
        // weights e = 448 * 2^(y - R) as E4M3, and their unquantised sum
        const float R_use = R == -INFINITY ? 0.f : R;
        const float bb0 = lb0 + LOG2_448 - R_use, bb1 = lb1 + LOG2_448 - R_use;
        // (computed in place: sacc[blk][i] becomes the weight of score i)
        float sum0, sum1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sacc[0][i] = fast_exp2(__builtin_fmaf(sacc[0][i], A0, bb0));
            sacc[1][i] = fast_exp2(__builtin_fmaf(sacc[1][i], A1, bb1));
            sum0 = i == 0 ? sacc[0][0] : sum0 + sacc[0][i];
            sum1 = i == 0 ? sacc[1][0] : sum1 + sacc[1][i];
        }
        l_run += sum0 * __builtin_amdgcn_rcpf(448.0f * sc0) + sum1 * __builtin_amdgcn_rcpf(448.0f * sc1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pop[k] = pack_fp8x4(sacc[0][4 * k], sacc[0][4 * k + 1], sacc[0][4 * k + 2], sacc[0][4 * k + 3], pop[k]);
            pop[4 + k] = pack_fp8x4(sacc[1][4 * k], sacc[1][4 * k + 1], sacc[1][4 * k + 2], sacc[1][4 * k + 3],
                                    pop[4 + k]);
        }
        __builtin_amdgcn_sched_barrier(0);

        // O^T += C^T P^T, one FP8 MFMA per 32 d; the A operand of d-block
        // db + VPF is read before the MFMA of db
        const char *vb = kt + v_lane;
        auto v_at = [&](int db) {
            const i32x2 r0 = lds_read_tr8(vb + 32 * db + v_off(0));
            const i32x2 r1 = lds_read_tr8(vb + 32 * db + v_off(1));
            const i32x2 r2 = lds_read_tr8(vb + 32 * db + v_off(2));
            const i32x2 r3 = lds_read_tr8(vb + 32 * db + v_off(3));
            return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
        };
        constexpr int VPF = 2;
        i32x8 va[VPF + 1];
#pragma unroll
        for (int i = 0; i < VPF; ++i) va[i] = v_at(i);
#pragma unroll
        for (int db = 0; db < DC / 32; ++db) {
            if (db + VPF < DC / 32) va[(db + VPF) % (VPF + 1)] = v_at(db + VPF);
            oacc[db] = mfma8_o(va[db % (VPF + 1)], pop, oacc[db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int db = 0; db < DC / 32; ++db) settle_acc(oacc[db]);

    const float lt = pair32_sum(l_run);
    const float inv = lt > 0.f ? 1.0f / (448.0f * lt) : 0.f;
    // bf16 partial rows through LDS, one whole row per store (see the bf16
    // kernel); all tiles have landed and every wave is past the ring.
    raw_barrier();
    store_partial_rows(smem, wave, lane, oacc, inv, p.ws_o, ((size_t)b * p.H + hc * HPC + wave * HPW) * p.n_split_max + s,
                       p.n_split_max, p.H - (hc * HPC + wave * HPW));
    if (head_ok && hh == 0) p.ws_lse[((size_t)b * p.H + h) * p.n_split_max + s] = lt > 0.f ? R + __log2f(lt) : -INFINITY;
}

}  // namespace

hipError_t launch_mla_decode_fp8(const MlaFp8Args &a, hipStream_t stream) {
    // the query rows, one quantisation tile each
    hipError_t e = launch_quantize_kv_fp8(a.q, a.ws_q8, a.ws_qs, (long long)a.B * a.H, 1, DK, stream);
    if (e != hipSuccess) return e;
    Params p;
    p.q8 = static_cast<const uint8_t *>(a.ws_q8);
    p.qs = a.ws_qs;
    p.c = static_cast<const uint8_t *>(a.cache);
    p.cs = a.cache_scales;
    p.seq_lens = a.seq_lens;
    p.ws_o = a.ws_o;
    p.ws_lse = a.ws_lse;
    p.B = a.B;
    p.S_max = a.S_max;
    p.H = a.H;
    p.n_stiles = (a.S_max + SCALE_TILE - 1) / SCALE_TILE;
    p.split = a.split;
    p.n_split_max = a.n_split_max;
    p.scale_log2 = a.scale * kLog2e;
    e = ensure_dynamic_lds((const void *)mla_decode_fp8_kernel, LDS_BYTES);
    if (e != hipSuccess) return e;
    p.n_hchunk = (a.H + HPC - 1) / HPC;
    const long long n_wg = (long long)a.B * a.n_split_max * p.n_hchunk;
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_decode_fp8_kernel, dim3((unsigned)n_wg), dim3(64 * NW), LDS_BYTES, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_combine(a.ws_o, a.ws_lse, a.seq_lens, a.o, a.lse, a.B, a.H, DC, a.S_max,
                                a.split, a.n_split_max, a.sinks, stream, /*partial_bf16=*/true);
}

}  // namespace mi355
