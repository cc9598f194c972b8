// prefill_fp8.hip -- causal / sliding-window / full attention forward with FP8
// attention for d_h = 128 on gfx950: both products on E4M3 MFMAs.
//
// Method: the pages' FP8 attention ("Flash Attention 3 and Multi-Headed
// Latent Attention", the FP8 attention section and its per-tile block
// processor: q, k and v quantised to E4M3 per tile with scale amax / 448,
// both matrix products on FP8 operands, p quantised before the second, the
// results dequantised by the scales) inside the FlashAttention-2 tiling of
// "Attention Engineering: From MHA to GQA, MLA & FlashAttention", section 4.
//  * q, k and v arrive as codes with one scale per 32 positions of a head
//    (the layout attn_quantize_kv_fp8 writes);
//  * s_ij = scale * sq_i * sk_j * (q8_i . k8_j): one FP8 product per 64-key
//    tile, scaled once per 32-key block;
//  * the weight of key j carries its value scale, y_ij = s_ij log2(e) +
//    log2(sv_j), and is quantised as e = 448 * 2^(y - R) -> E4M3 against the
//    row's reference R; R moves to a tile's max plus HEADROOM (5, log2
//    units) when the tile exceeds it, and what was accumulated is rescaled
//    by 2^(R_old - R_new), so no weight passes 448 and rescales are rare;
//  * the numerator accumulates e * v8, the denominator the unquantised
//    2^(s log2(e) - R) = e / (448 sv); o = acc / (448 l), lse = (R + log2 l)
//    ln 2 (with a sink logit merged in the epilogue).
//
// gfx950 mapping:
//  * workgroup = 256 query rows of 1, 2, 4 or 8 heads of one K/V group, 8
//    waves of 32 rows (two waves per SIMD: one wave's softmax overlaps the
//    other's MFMAs), heaviest row block first, head group fastest;
//  * 64-key K and V tiles stream HBM -> LDS through a 4-stage ring of
//    global_load_lds_dwordx4 copies (21 one-KB blocks per tile);
//  * S^T [64 keys x 32 rows] = K Q^T with v_mfma_f32_32x32x64_f8f6f4 (A = 32
//    bytes of a K row from LDS, B = the wave's query codes in registers),
//    two interleaved 32-key chains of 2 k-steps; each lane owns one row;
//  * O^T [128 x 32 rows] += V^T P^T, one FP8 MFMA per 32 d with K = the 64
//    keys: B = the lane's own 32 weights converted to E4M3, A = V read
//    transposed with ds_read_b64_tr_b8 (four reads whose rows are the keys
//    the lane's weights belong to; the FP8 MFMA pairs byte b of lane-half h
//    of A with byte b of lane-half h of B, measured on the hardware);
//  * the tile's max of y is taken only when the weights, taken against the
//    current R, sum past 448 in some lane (or a row has no R yet): positive
//    weights with a sum of at most 448 are each at most 448, so R moves on
//    the same tiles as with the max taken every time;
//  * LDS rows: K at slot 8 r + r/2 (16-row score reads of a quarter wave hit
//    16 distinct slots), V at slot 12 r + (r/4) mod 4 (the 8-row transposing
//    reads of a half wave hit 16 distinct slots);
//  * after the ring, a table of the workgroup's per-key-block constants (k
//    scale, log2 of the v scale, 1 / (448 v scale)), filled once before the
//    tile loop; the output leaves through the ring as whole row halves.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int D = 128;
constexpr int BN = 64;                        // keys per tile
constexpr int NW = 8;                         // waves per workgroup
constexpr int WG_ROWS = 256;                  // query rows x heads per workgroup
constexpr int K_BYTES = 9 * 1024;             // K rows: last slot 8*63 + 31 + 8 = 543
constexpr int V_BYTES = 12 * 1024;            // V rows: last slot 12*63 + 3 + 8 = 767
constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
constexpr int NBLK = STAGE_BYTES / 1024;      // 21 one-KB copies per tile
constexpr int PER_WAVE = (NBLK + NW - 1) / NW; // 3 (the last wave repeats its final block)
constexpr int NSTAGE = 4;
constexpr int RING_BYTES = NSTAGE * STAGE_BYTES;  // 86016
// Per-key-block constants of a workgroup's tiles (k scale, log2 of the v
// scale, 1 / (448 v scale)), computed once before the tile loop: up to
// TAB_CAP blocks of 32 keys; tiles past them take the constants per tile.
constexpr int TAB_CAP = 4096;
constexpr int LDS_BYTES = RING_BYTES + TAB_CAP * 16;   // 151552
static_assert(NW * 32 * 144 <= RING_BYTES, "epilogue staging exceeds the ring");
static_assert(LDS_BYTES <= 160 * 1024, "LDS ring and block table exceed the LDS");
constexpr float LOG2_448 = 8.807354922057604f;
constexpr float HEADROOM = 5.0f;

typedef __attribute__((ext_vector_type(8))) int i32x8;

struct Params {
    const uint8_t *q, *k, *v;          // codes
    const float *qs, *ks, *vs;         // one scale per 32 positions of a head
    __bf16 *o;
    float *lse;
    int T, hq, hkv, G, nt;             // nt = ceil(T / 32)
    int hpw, rows_per_wg, n_row_blocks, n_head_groups;
    int causal, window;
    float scale_log2;
    const float *sinks;
};

__host__ __device__ constexpr int kslot(int r) { return 8 * r + (r >> 1); }
__host__ __device__ constexpr int vslot(int r) { return 12 * r + ((r >> 2) & 3); }

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
// The output product through the compiler (block-scaled form, both scale
// exponents 127: x 1.0), its accumulators in VGPRs like everything else: an
// accumulator pinned in AGPRs made the compiler split the 256 registers
// 128 / 128 and spill the rest of the loop's values through AGPRs on every
// tile.
__device__ __forceinline__ void mfma8_o(i32x8 a, i32x8 b, f32x16 &acc) {
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ i32x8 lds32(const char *p) {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
// Four E4M3 codes in one word.  The first conversion writes the low half and
// keeps the high half of `old`, which the second then overwrites: passing the
// word's previous contents (rather than 0) spares a register clear per word.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d, int old) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__global__ __launch_bounds__(64 * NW, 1) void prefill_fp8_d128_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int id = blockIdx.x;
    const int rb = p.n_row_blocks - 1 - id / p.n_head_groups;
    const int hg = id % p.n_head_groups;
    const int subs = p.G / p.hpw;
    const int sub = hg % subs;
    const int g = (hg / subs) % p.hkv;
    const int b = hg / (subs * p.hkv);
    const int wph = NW / p.hpw;
    const int h = g * p.G + sub * p.hpw + wave / wph;
    const int r0 = rb * p.rows_per_wg;
    const int rw0 = r0 + (wave % wph) * 32;
    const int T = p.T;

    const int kend = p.causal ? min(T, r0 + p.rows_per_wg) : T;
    const int kbeg = p.window > 0 ? max(0, r0 - p.window + 1) : 0;
    const int t_begin = kbeg / BN;
    const int t_end = (kend + BN - 1) / BN;
    const bool wave_active = rw0 < T;
    const int kend_w = p.causal ? min(T, rw0 + 32) : T;
    const int kbeg_w = p.window > 0 ? max(0, rw0 - p.window + 1) : 0;
    auto tile_active = [&](int t) {
        const int ts = t * BN;
        return wave_active && ts < kend_w && ts + BN > kbeg_w;
    };
    auto tile_needs_mask = [&](int t) {
        const int ts = t * BN;
        return (ts + BN > T) || (p.causal && ts + BN - 1 > rw0) ||
               (p.window > 0 && (rw0 + 31) - ts >= p.window);
    };

    const size_t kv_base = ((size_t)b * p.hkv + g) * (size_t)T * D;
    const uint8_t *kg = p.k + kv_base;
    const uint8_t *vg = p.v + kv_base;
    const float *ksg = p.ks + ((size_t)b * p.hkv + g) * p.nt;
    const float *vsg = p.vs + ((size_t)b * p.hkv + g) * p.nt;
    const size_t q_base = ((size_t)b * p.hq + h) * (size_t)T * D;
    const int row = rw0 + l32;                       // this lane's query row

    // copies: LDS slot q of a stage holds (K or V) row r, 16-byte chunk c;
    // pad slots receive a valid chunk nobody reads; rows past T re-read row T-1
    uint32_t dma_off[PER_WAVE];
    int dma_row[PER_WAVE];
    bool dma_v[PER_WAVE];
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int blk = min(PER_WAVE * wave + i, NBLK - 1);
        const bool isv = blk * 1024 >= K_BYTES;
        const int q = (blk * 1024 - (isv ? K_BYTES : 0)) / 16 + lane;
        int r;
        if (!isv) {
            r = min((2 * q) / 17, BN - 1);
            if (r < BN - 1 && kslot(r + 1) <= q) ++r;
            if (kslot(r) > q) --r;
        } else {
            r = min(q / 12, BN - 1);
            if (vslot(r) > q) --r;
        }
        const int c = min(q - (isv ? vslot(r) : kslot(r)), D / 16 - 1);
        dma_row[i] = r;
        dma_v[i] = isv;
        dma_off[i] = (uint32_t)(r * D + c * 16);
    }
    const uint32_t smem_lds = lds_offset(smem);
    auto issue_tile = [&](int t) {
        const uint32_t stage = smem_lds + ((t - t_begin) % NSTAGE) * STAGE_BYTES;
        const int ts = t * BN;
        const uint8_t *kb0 = kg + (size_t)ts * D;
        const uint8_t *vb0 = vg + (size_t)ts * D;
        if (ts + BN <= T) {                          // whole tile: precomputed offsets
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i)
                dma16_off_at(dma_v[i] ? vb0 : kb0, dma_off[i], stage + min(PER_WAVE * wave + i, NBLK - 1) * 1024);
        } else {                                     // ragged last tile: rows past T re-read row T-1
            // (opaque to the compiler: as an affine function of the tile it
            // was strength-reduced into per-lane counters updated every tile)
            int last = T - 1 - ts;
            asm volatile("" : "+s"(last));
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) {
                const uint32_t off = dma_row[i] > last
                    ? dma_off[i] - (uint32_t)((dma_row[i] - last) * D) : dma_off[i];
                dma16_off_at(dma_v[i] ? vb0 : kb0, off, stage + min(PER_WAVE * wave + i, NBLK - 1) * 1024);
            }
        }
    };
    auto wait_tiles = [&](int newer) {               // all but the `newer` most recent tiles landed
        if (newer >= 2) wait_vmcnt<2 * PER_WAVE>();
        else if (newer == 1) wait_vmcnt<PER_WAVE>();
        else wait_vmcnt<0>();
    };

    // the wave's query codes as B operands: k-step ks holds d = 64 ks + 32 hh .. +31
    i32x8 qop[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
        if (row < T) {
            const uint8_t *qp = p.q + q_base + (size_t)row * D + 64 * ks + 32 * hh;
            x0 = ldg16(qp);
            x1 = ldg16(qp + 16);
        }
        qop[ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                        (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
    const float a_row = wave_active ? p.scale_log2 * p.qs[((size_t)b * p.hq + h) * p.nt + rw0 / 32] : 0.f;

    // The key-block constants of this workgroup's tiles, block j = key block
    // 2 t_begin + j; a block past the head's end repeats its last block (its
    // keys are masked, and it is then the tile's first block).
    float4 *stab = reinterpret_cast<float4 *>(smem + RING_BYTES);
    const int n_tab = min(2 * (t_end - t_begin), TAB_CAP);
    for (int j = tid; j < n_tab; j += 64 * NW) {
        const int kb = min(2 * t_begin + j, p.nt - 1);
        const float skj = ksg[kb], svj = vsg[kb];
        stab[j] = float4{skj, __log2f(svj), __builtin_amdgcn_rcpf(448.0f * svj), 0.f};
    }

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float R = -INFINITY, l_run = 0.f;
    i32x8 pop = {0, 0, 0, 0, 0, 0, 0, 0};          // the tile's E4M3 weights (P.V B operand)

    // score A operand: K row 32 blk + l32, bytes 64 ks + 32 hh
    const int k_lane = 16 * (kslot(l32) + 2 * hh);
    constexpr int KBLK = 16 * (kslot(32) - kslot(0));  // bytes from row r to row r + 32
    // transposing read j: lane L of group G (hh = G/2, d-half G%2) addresses
    // V row 16 (j%2) + 32 (j/2) + 8 (r/4) + 4 hh + r%4, r = L/2
    const int g16 = lane >> 4, L16 = lane & 15, rr = L16 >> 1;
    const int v_tok = 8 * (rr >> 2) + 4 * (g16 >> 1) + (rr & 3);
    const int v_lane = K_BYTES + 16 * vslot(v_tok) + 16 * (g16 & 1) + 8 * (L16 & 1);
    auto v_off = [](int j) { return 16 * 12 * (16 * (j & 1) + 32 * (j >> 1)); };

    // prologue: tiles t_begin .. t_begin + NSTAGE - 2 in flight
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i)
        if (t_begin + i < t_end) issue_tile(t_begin + i);
    // Every load so far (the wave's resident operands and the prologue
    // copies) has landed: the compiler then puts no wait for the resident
    // operands inside the loop, whose only outstanding loads are the ring's
    // copies (which it does not track).
    wait_vmcnt<0>();

    for (int t = t_begin; t < t_end; ++t) {
        const int rel = t - t_begin;
        wait_tiles(min(NSTAGE - 2, t_end - 1 - t));
        raw_barrier();                               // tile t landed everywhere; stage t-1 free
        if (t + NSTAGE - 1 < t_end) issue_tile(t + NSTAGE - 1);
        if (!tile_active(t)) continue;               // wave-uniform
        const char *st = smem + (rel % NSTAGE) * STAGE_BYTES;
        const int ts = t * BN;

        // S^T of the two 32-key blocks, interleaved chains
        f32x16 sacc[2];
        {
            const char *ka = st + k_lane;
            i32x8 a0 = lds32(ka), a1 = lds32(ka + KBLK);
            i32x8 a2 = lds32(ka + 64), a3 = lds32(ka + KBLK + 64);
            sacc[0] = mfma8_first(a0, qop[0]);
            sacc[1] = mfma8_first(a1, qop[0]);
            sacc[0] = mfma8_acc(a2, qop[1], sacc[0]);
            sacc[1] = mfma8_last(a3, qop[1], sacc[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // element i of block blk is key ts + 4 hh + e of row `row`, e = 32 blk
        // + 8 (i/4) + i%4.  The visible keys of the row (below T, at or before
        // the row when causal, within the window) are one range [lo, lo +
        // width) of e, so one unsigned compare per element tests it.
        if (tile_needs_mask(t)) {
            int tsm = ts;                            // opaque, as for the ragged copy offsets
            asm volatile("" : "+s"(tsm));
            const int base = tsm + 4 * hh;
            const int diff = row - base;
            int e_hi = min(T - base, BN);
            if (p.causal) e_hi = min(e_hi, diff + 1);
            const int lo = p.window > 0 ? min(max(diff - p.window + 1, 0), BN) : 0;
            const uint32_t width = (uint32_t)max(e_hi - lo, 0);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * blk + 8 * (i >> 2) + (i & 3);
                    sacc[blk][i] = (uint32_t)(e - lo) < width ? sacc[blk][i] : -INFINITY;
                }
        }
        float A0, A1, lb0, lb1, r0, r1;
        if (2 * rel + 1 < TAB_CAP) {                 // wave-uniform
            const float4 e0 = stab[2 * rel], e1 = stab[2 * rel + 1];
            A0 = a_row * e0.x;
            A1 = a_row * e1.x;
            lb0 = e0.y;
            lb1 = e1.y;
            r0 = e0.z;
            r1 = e1.z;
        } else {
            const int st0 = ts / 32;
            const float sk0 = ld_uniform_f(ksg, st0), sv0 = ld_uniform_f(vsg, st0);
            const bool two = ts + 32 < T;
            const float sk1 = two ? ld_uniform_f(ksg, st0 + 1) : sk0;
            const float sv1 = two ? ld_uniform_f(vsg, st0 + 1) : sv0;
            A0 = a_row * sk0;
            A1 = a_row * sk1;
            lb0 = __log2f(sv0);
            lb1 = __log2f(sv1);
            r0 = __builtin_amdgcn_rcpf(448.0f * sv0);
            r1 = __builtin_amdgcn_rcpf(448.0f * sv1);
        }
        // The weights against the current reference.  They are positive, so
        // a lane whose weights sum to at most 448 has none above 448, i.e. no
        // y above R: only when some lane's sum passes 448 (or a row's R is
        // still -inf) is the tile's max of y taken, R moved for the rows whose
        // max exceeds it, and the weights taken again -- R moves on exactly
        // the tiles it would with the max taken every time.
        float wt[2][16];
        float sum0, sum1;
        auto take_weights = [&]() {
            const float R_use = R == -INFINITY ? 0.f : R;
            const float bb0 = lb0 + LOG2_448 - R_use, bb1 = lb1 + LOG2_448 - R_use;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                wt[0][i] = fast_exp2(__builtin_fmaf(sacc[0][i], A0, bb0));
                wt[1][i] = fast_exp2(__builtin_fmaf(sacc[1][i], A1, bb1));
                sum0 = i == 0 ? wt[0][0] : sum0 + wt[0][i];
                sum1 = i == 0 ? wt[1][0] : sum1 + wt[1][i];
            }
        };
        take_weights();
        if (__any(R == -INFINITY || !(sum0 + sum1 <= 448.0f))) {
            float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                mx0 = fmaxf(mx0, sacc[0][i]);
                mx1 = fmaxf(mx1, sacc[1][i]);
            }
            const float yh = pair32_max(fmaxf(__builtin_fmaf(mx0, A0, lb0), __builtin_fmaf(mx1, A1, lb1)));
            if (yh > R) {                            // this row's reference moves
                const float Rn = yh + HEADROOM;
                const float f = fast_exp2(R - Rn);   // 0 while R = -inf
                if (R != -INFINITY) {
#pragma unroll
                    for (int db = 0; db < 4; ++db) oacc[db] *= f;
                }
                l_run *= f;
                R = Rn;
            }
            take_weights();
        }
        l_run += sum0 * r0 + sum1 * r1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pop[k] = pack_fp8x4(wt[0][4 * k], wt[0][4 * k + 1], wt[0][4 * k + 2], wt[0][4 * k + 3], pop[k]);
            pop[4 + k] = pack_fp8x4(wt[1][4 * k], wt[1][4 * k + 1], wt[1][4 * k + 2], wt[1][4 * k + 3], pop[4 + k]);
        }
        __builtin_amdgcn_sched_barrier(0);

        // O^T += V^T P^T, one FP8 MFMA per 32 d
        const char *vb = st + v_lane;
        auto v_at = [&](int db) {
            const i32x2 x0 = lds_read_tr8(vb + 32 * db + v_off(0));
            const i32x2 x1 = lds_read_tr8(vb + 32 * db + v_off(1));
            const i32x2 x2 = lds_read_tr8(vb + 32 * db + v_off(2));
            const i32x2 x3 = lds_read_tr8(vb + 32 * db + v_off(3));
            return i32x8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
        };
        i32x8 va[2];
        va[0] = v_at(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            if (db + 1 < 4) va[(db + 1) & 1] = v_at(db + 1);
            mfma8_o(va[db & 1], pop, oacc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Every wave is past the tile loop and no copy is in flight: the output
    // goes out through the ring, so that each store writes a whole 128-byte
    // row half.  Each lane holds four-value pieces of its row; the wave's 32
    // rows x 64 values of one half go to its own region (rows 144 bytes
    // apart: the 8-byte writes of a quarter wave hit distinct banks) and come
    // back as 16 bytes of 8 consecutive values per lane, 8 lanes per row half.
    raw_barrier();
    if (!wave_active) return;
    const float lt = pair32_sum(l_run);
    float inv = lt > 0.f ? 1.0f / (448.0f * lt) : 0.f;
    float lse_nat = lt > 0.f ? (R + __log2f(lt)) * kLn2 : -INFINITY;
    if (p.sinks) {
        float ls;
        inv = finish_row_with_sink(lt > 0.f ? R : -INFINITY, lt, p.sinks[h] * kLog2e, ls) * (1.0f / 448.0f);
        lse_nat = ls;
    }
    char *reg = smem + wave * (32 * 144);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int db = 2 * half; db < 2 * half + 2; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * db + 8 * q4 + 4 * hh - 64 * half;
                u32x2 w = {pack_bf16x2(oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv),
                           pack_bf16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv)};
                *reinterpret_cast<u32x2 *>(reg + l32 * 144 + 2 * d) = w;
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = 8 * r + (lane >> 3), ch = lane & 7;
            const u32x4 v4 = *reinterpret_cast<const u32x4 *>(reg + rr * 144 + 16 * ch);
            if (rw0 + rr < T)
                *reinterpret_cast<u32x4 *>(p.o + q_base + (size_t)(rw0 + rr) * D + 64 * half + 8 * ch) = v4;
        }
    }
    if (p.lse && hh == 0 && row < T) p.lse[((size_t)b * p.hq + h) * (size_t)T + row] = lse_nat;
}

}  // namespace

hipError_t launch_prefill_fp8_d128(const PrefillFp8Args &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const uint8_t *>(a.q);
    p.k = static_cast<const uint8_t *>(a.k);
    p.v = static_cast<const uint8_t *>(a.v);
    p.qs = a.q_scales;
    p.ks = a.k_scales;
    p.vs = a.v_scales;
    p.o = static_cast<__bf16 *>(a.o);
    p.lse = a.lse;
    p.T = a.T;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.nt = (a.T + 31) / 32;
    p.hpw = (p.G % 8 == 0) ? 8 : (p.G % 4 == 0) ? 4 : (p.G % 2 == 0 ? 2 : 1);
    p.rows_per_wg = WG_ROWS / p.hpw;
    p.n_row_blocks = (a.T + p.rows_per_wg - 1) / p.rows_per_wg;
    p.n_head_groups = a.B * a.hkv * (p.G / p.hpw);
    p.causal = a.causal;
    p.window = a.window;
    p.scale_log2 = a.scale * kLog2e;
    p.sinks = a.sinks;
    hipError_t e = ensure_dynamic_lds((const void *)prefill_fp8_d128_kernel, LDS_BYTES);
    if (e != hipSuccess) return e;
    const long long nblocks = (long long)p.n_row_blocks * p.n_head_groups;
    if (nblocks <= 0) return hipSuccess;
    if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_fp8_d128_kernel, dim3((unsigned)nblocks), dim3(64 * NW), LDS_BYTES,
                       stream, p);
    return hipGetLastError();
}

}  // namespace mi355
