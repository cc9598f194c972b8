// prefill_bwd_bf16.hip -- backward of the bf16, d_h = 128 prefill on gfx950:
// dQ, dK, dV of O = softmax(scale Q K^T + mask) V for grouped K/V heads.
//
// Method: the forward keeps only the per-row log-sum-exp L for this pass and
// the scores are recomputed ("Attention Engineering: From MHA to GQA, MLA &
// FlashAttention", section 4, the text after the FlashAttention-2
// recurrence; "Attention, Worked Out by Hand (Part 2)", section 2).  On
// visible keys P_ij = 2^(c s_ij - L_i log2 e) with c = scale log2 e, and
// with dP_ij = dO_i.v_j and D_i = dO_i.O_i
//     dS_ij = P_ij (dP_ij - D_i),  dQ_i = scale sum_j dS_ij k_j,
//     dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i,
// where for K and V the sum over i runs over every query head of the group.
//
// gfx950 mapping, three launches:
//  * bwd_rows_kernel: per query row, the pair (L log2 e, D = dO.O) in fp32,
//    written to a workspace whose rows are padded to a multiple of 64 (pad
//    rows get L = +inf and D = 0, so their probabilities are exactly 0);
//  * bwd_dkdv_kernel: one workgroup per (batch, K/V head, 128 keys), 4 waves
//    (one per SIMD) of 32 keys each.  A wave keeps its keys' K and V rows in
//    registers as MFMA B operands and streams 64-row Q / dO tiles of every
//    query head of the group through a 3-stage LDS ring (global->LDS
//    copies).  Per 32 query rows: S = Q K^T and dP = dO V^T on
//    v_mfma_f32_32x32x16_bf16 (lane = key column), P and dS in registers,
//    then dV^T += dO^T P and dK^T += Q^T dS with P, dS (rounded to bf16) as
//    B operands straight from the accumulators and dO^T, Q^T read from the
//    row-major tiles with the transposing LDS load.  dK and dV accumulate
//    over all query heads of the group in registers: no atomics;
//  * bwd_dq_kernel: the forward's decomposition (256 query rows x heads per
//    workgroup, 8 waves of 32 rows); a wave keeps its rows' Q and dO as B
//    operands and streams 64-key K / V tiles: S^T = K Q^T and dP^T = V dO^T
//    (lane = query row, so L and D are per-lane scalars), dS^T in
//    registers, dQ^T += K^T dS^T with K^T from the transposing load.
//  Tiles are stored with rows 320 bytes apart and row r shifted by
//  (r / 4) mod 4 16-byte slots: both the 16-byte row reads of a quarter wave
//  (16 consecutive rows, one chunk) and the transposing reads of a half wave
//  (4 rows x 64 bytes) then hit 16 distinct slots, i.e. no bank conflicts.
#include <type_traits>

#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int D = 128;
constexpr int TROWS = 64;                    // rows per streamed tile
constexpr int TSLOTS = 20;                   // 16-byte slots per LDS row (16 data + 4 pad)
constexpr int TBYTES = TROWS * TSLOTS * 16;  // 20480 bytes per tile
constexpr int TBLK = TBYTES / 1024;          // 20 one-KB copy blocks per tile

__device__ __forceinline__ int rot(int r) { return (r >> 2) & 3; }
// byte offset of (row r, 16-byte chunk ch) inside a tile
__device__ __forceinline__ int toff(int r, int ch) { return 16 * (TSLOTS * r + rot(r) + ch); }
// Source of LDS slot blk * 64 + lane of a tile: its row and the byte offset
// of its chunk inside the 64 tile rows in global memory (pad slots copy a
// valid chunk of their row).
__device__ __forceinline__ void tile_src(int blk, int lane, int &row, uint32_t &off) {
    const int qs = blk * 64 + lane;
    const int r = qs / TSLOTS;
    int ch = qs - TSLOTS * r - rot(r);
    ch = ch < 0 ? 0 : (ch > 15 ? 15 : ch);
    row = r;
    off = (uint32_t)(r * D * 2 + ch * 16);
}

struct Params {
    const __bf16 *q, *k, *v, *o, *dout;
    const float *lse;
    __bf16 *dq, *dk, *dv;
    const float *stats;                      // [B * hq, Tpad, 2]: L log2 e, D
    float *stats_w;
    int B, T, Tpad, hq, hkv, G;
    int causal, window;
    float scale, c;                          // c = scale * log2(e)
    // dq kernel decomposition (as the forward)
    int hpw, rows_per_wg, n_row_blocks, n_head_groups;
    const float *sinks;
    float *dsinks;
};

// ---------------------------------------------------------------------------
// Gradient of a sink logit s_h (an extra softmax-denominator term without a
// value row): dL/ds_h = -sum over the head's rows (every batch entry) of
// exp(s_h - L_i) D_i, from the row statistics.  One workgroup per query
// head; fixed summation order, so the result is reproducible.
__global__ __launch_bounds__(256) void bwd_sink_grad_kernel(Params p) {
    const int h = blockIdx.x;
    const float s2 = p.sinks[h] * kLog2e;
    float acc = 0.f;
    for (int b = 0; b < p.B; ++b) {
        const float *st = p.stats + 2 * ((size_t)b * p.hq + h) * p.Tpad;
        for (int r = threadIdx.x; r < p.T; r += 256) {
            const f32x2 v = *reinterpret_cast<const f32x2 *>(st + 2 * r);
            acc = __builtin_fmaf(fast_exp2(s2 - v[0]), v[1], acc);
        }
    }
    __shared__ float part[4];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) p.dsinks[h] = -((part[0] + part[1]) + (part[2] + part[3]));
}

// ---------------------------------------------------------------------------
// Row statistics: D_i = dO_i . O_i and L_i log2(e); 16 lanes per row.
__global__ __launch_bounds__(256) void bwd_rows_kernel(Params p) {
    const int bh = blockIdx.y;
    const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int part = threadIdx.x & 15;
    if (r >= p.Tpad) return;
    float acc = 0.f;
    if (r < p.T) {
        const size_t base = ((size_t)bh * p.T + r) * D + 8 * part;
        const u32x4 ov = ldg16(p.o + base);
        const u32x4 gv = ldg16(p.dout + base);
        const bf16x8 ob = __builtin_bit_cast(bf16x8, ov);
        const bf16x8 gb = __builtin_bit_cast(bf16x8, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ob[e], (float)gb[e], acc);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (part == 0) {
        f32x2 st = {INFINITY, 0.f};
        if (r < p.T) {
            const float L = p.lse[(size_t)bh * p.T + r];
            st[0] = L == -INFINITY ? INFINITY : L * kLog2e;
            st[1] = acc;
        }
        *reinterpret_cast<f32x2 *>(p.stats_w + 2 * ((size_t)bh * p.Tpad + r)) = st;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = (batch b, K/V head g, 128 keys); wave = 32 keys.
constexpr int KA_WAVES = 4;
constexpr int KA_KEYS = 32 * KA_WAVES;
constexpr int KA_NSTAGE = 3;
constexpr int KA_STAGE = 2 * TBYTES + 1024;  // Q tile, dO tile, row statistics
constexpr int KA_NBLK = 2 * TBLK + 1;        // 41 one-KB copies per step
constexpr int KA_PER_WAVE = (KA_NBLK + KA_WAVES - 1) / KA_WAVES;   // 11
constexpr int KA_LDS = KA_NSTAGE * KA_STAGE;

__global__ __launch_bounds__(64 * KA_WAVES, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int q16 = lane >> 4;
    const int j16 = lane & 15;
    const int T = p.T;

    // key blocks ascending (the causal heaviest first); (b, g) fastest, so
    // the key blocks of one K/V head share an XCD when B*hkv is a multiple of 8
    const int nbg = p.B * p.hkv;
    const int kblk = blockIdx.x / nbg;
    const int bg = blockIdx.x % nbg;
    const int b = bg / p.hkv;
    const int g = bg % p.hkv;
    const int kb0 = kblk * KA_KEYS;
    const int kw0 = kb0 + 32 * wave;             // this wave's first key
    const int key = kw0 + l32;                   // this lane's key (B-operand column)

    // query tiles that can see a key of this workgroup
    const int nqt = (T + TROWS - 1) / TROWS;
    const int qt_beg = p.causal ? kb0 / TROWS : 0;
    int qt_end = nqt;
    if (p.window > 0) qt_end = min(nqt, (kb0 + KA_KEYS - 1 + p.window - 1) / TROWS + 1);
    const int nq = max(qt_end - qt_beg, 0);
    const int n_steps = p.G * nq;

    // the wave's K and V rows as B operands: key `key`, d = 16 ks + 8 hi .. +7
    const size_t kv_base = ((size_t)b * p.hkv + g) * (size_t)T * D;
    bf16x8 kop[8], vop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        u32x4 kv4 = {0u, 0u, 0u, 0u}, vv4 = {0u, 0u, 0u, 0u};
        if (key < T) {
            kv4 = ldg16(p.k + kv_base + (size_t)key * D + 16 * ks + 8 * hi);
            vv4 = ldg16(p.v + kv_base + (size_t)key * D + 16 * ks + 8 * hi);
        }
        kop[ks] = __builtin_bit_cast(bf16x8, kv4);
        vop[ks] = __builtin_bit_cast(bf16x8, vv4);
    }
    f32x16 dkacc[4], dvacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) { dkacc[db][i] = 0.f; dvacc[db][i] = 0.f; }

    // copies of one step: blocks 0-19 Q tile, 20-39 dO tile, 40 row statistics
    uint32_t dma_off[KA_PER_WAVE];
    int dma_row[KA_PER_WAVE];
    int dma_kind[KA_PER_WAVE];                   // 0 Q, 1 dO, 2 statistics
#pragma unroll
    for (int i = 0; i < KA_PER_WAVE; ++i) {
        const int blk = min(KA_PER_WAVE * wave + i, KA_NBLK - 1);
        if (blk < 2 * TBLK) {
            dma_kind[i] = blk / TBLK;
            tile_src(blk % TBLK, lane, dma_row[i], dma_off[i]);
        } else {                                 // lane l < 32: (L, D) of rows 2l, 2l+1
            dma_kind[i] = 2;                     // (lanes 32-63 repeat them)
            dma_row[i] = 0;
            dma_off[i] = (uint32_t)(16 * (lane & 31));
        }
    }
    const uint32_t smem_lds = lds_offset(smem);
    // Steps run over (query tile, head) with the head fastest and the tiles
    // from the last one down: every key block of a K/V head then reads the
    // same Q / dO tile at the same time (they only differ in where they
    // stop), so the tiles are shared through the XCD's L2.
    int is_h = 0, is_qt = qt_end - 1;           // next step to copy
    auto issue_step = [&](int s) {
        const int h = g * p.G + is_h;
        const int qt = is_qt;
        if (++is_h == p.G) { is_h = 0; --is_qt; }
        const int r0 = qt * TROWS;
        const size_t bh = (size_t)b * p.hq + h;
        const __bf16 *qb = p.q + (bh * T + r0) * D;
        const __bf16 *gb = p.dout + (bh * T + r0) * D;
        const float *sb_ = p.stats + 2 * (bh * p.Tpad + r0);
        const int last = T - 1 - r0;             // rows past T re-read row T-1
        const uint32_t stage = smem_lds + (s % KA_NSTAGE) * KA_STAGE;
#pragma unroll
        for (int i = 0; i < KA_PER_WAVE; ++i) {
            const int blk = min(KA_PER_WAVE * wave + i, KA_NBLK - 1);
            const uint32_t dst = stage + blk * 1024;
            if (dma_kind[i] == 2) {
                dma16_off_at(sb_, dma_off[i], dst);
            } else {
                const uint32_t off = dma_row[i] > last
                    ? dma_off[i] - (uint32_t)((dma_row[i] - last) * D * 2) : dma_off[i];
                dma16_off_at(dma_kind[i] ? (const void *)gb : (const void *)qb, off, dst);
            }
        }
    };
    auto wait_steps = [&](int newer) {           // all but the `newer` most recent steps landed
        if (newer >= 1) wait_vmcnt<KA_PER_WAVE>();
        else wait_vmcnt<0>();
    };

    // transposing-read lane constants (rows 4hi + (j16 >> 2) (+8) of a
    // 16-row half, d = 32 db + 16 (q16 & 1) + 4 (j16 & 3) .. +3)
    const int tr_row = 4 * hi + (j16 >> 2);
    const int tr_ch = 2 * (q16 & 1) + ((j16 & 3) >> 1);
    const int tr_byte = 8 * (j16 & 1);
    auto tr_operand = [&](const char *tile, int rbase, int db) {
        const int r = rbase + tr_row;
        const bf16x4 lo4 = lds_read_tr16(tile + toff(r, 4 * db + tr_ch) + tr_byte);
        const bf16x4 hi4 = lds_read_tr16(tile + toff(r + 8, 4 * db + tr_ch) + tr_byte);
        return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    const float c = p.c;
    // One 64-row Q / dO tile against this wave's 32 keys (MASKED: some pair
    // of the tile is not visible, or rows pass T), one 32-row block at a
    // time.  S, dP accumulate in VGPRs and dK^T, dV^T stay pinned in AGPRs
    // (asm MFMAs that carry their own wait states: mfma_s_first /
    // mfma_s_last / mfma_o_acc), so the compiler never moves the output
    // accumulators through VGPRs.
    // The rows of a tile that see this lane's key form one range of the row
    // offset e within the tile: at or after the key (causal), before T, less
    // than the window past the key; [m_lo, m_lo + m_width) when need_mask.
    auto step_rows = [&](bool need_mask, const char *qtile, const char *gtile, const char *stat,
                         int r0) {
        int m_lo = 0;
        uint32_t m_width = 0;
        if (need_mask) {
            int e_hi = T - r0;
            if (p.window > 0) e_hi = min(e_hi, key + p.window - r0);
            m_lo = p.causal ? max(key - r0, 0) : 0;
            m_width = (uint32_t)max(min(e_hi, TROWS) - m_lo, 0);
        }
        // (not unrolled: one block at a time keeps the live registers of a
        // single block)
#pragma unroll 1
        for (int mb = 0; mb < 2; ++mb) {
            // S = Q K^T and dP = dO V^T for tile rows 32 mb .. 32 mb + 31
            // (operands are loaded SPF k-steps ahead of their MFMAs)
            constexpr int SPF = 2;
            f32x16 sacc, pacc;
            bf16x8 aqs[SPF + 1], ags[SPF + 1];
            // element i: tile row 32 mb + 8 (i / 4) + 4 hi + (i % 4), key `key`;
            // st[i/2] holds (L, D) of rows 2(i/2) and 2(i/2)+1 of that pattern
            // (read under the last score MFMAs)
            f32x4 st[8];
            const char *qrow = qtile + toff(32 * mb + l32, hi);
            const char *grow = gtile + toff(32 * mb + l32, hi);
#pragma unroll
            for (int i = 0; i < SPF; ++i) {
                aqs[i] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * i);
                ags[i] = *reinterpret_cast<const bf16x8 *>(grow + 32 * i);
            }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks + SPF < 8) {
                    aqs[(ks + SPF) % (SPF + 1)] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * (ks + SPF));
                    ags[(ks + SPF) % (SPF + 1)] = *reinterpret_cast<const bf16x8 *>(grow + 32 * (ks + SPF));
                }
                const bf16x8 aq = aqs[ks % (SPF + 1)];
                const bf16x8 ag = ags[ks % (SPF + 1)];
                if (ks == 0) {
                    sacc = mfma_s_first(aq, kop[0]);
                    pacc = mfma_s_first(ag, vop[0]);
                } else if (ks < 7) {
                    sacc = mfma_s_acc(aq, kop[ks], sacc);
                    pacc = mfma_s_acc(ag, vop[ks], pacc);
                } else {
                    sacc = mfma_s_acc(aq, kop[7], sacc);
                    pacc = mfma_s_last(ag, vop[7], pacc);
                }
                if (ks == 5) {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int row = 32 * mb + 8 * gq + 4 * hi;
                        st[2 * gq] = *reinterpret_cast<const f32x4 *>(stat + 8 * row);
                        st[2 * gq + 1] = *reinterpret_cast<const f32x4 *>(stat + 8 * row + 16);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            float pv[16], dsv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float l2e = st[i >> 1][2 * (i & 1)];
                const float dde = st[i >> 1][2 * (i & 1) + 1];
                pv[i] = fast_exp2(__builtin_fmaf(sacc[i], c, -l2e));
                dsv[i] = pv[i] * (pacc[i] - dde);
            }
            if (need_mask) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
                    const bool vis = (uint32_t)(e - m_lo) < m_width;
                    pv[i] = vis ? pv[i] : 0.f;
                    dsv[i] = vis ? dsv[i] : 0.f;
                }
            }
            bf16x8 pb[2], sb[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                pb[hf] = to_bf16x8(pv[8 * hf], pv[8 * hf + 1], pv[8 * hf + 2], pv[8 * hf + 3],
                                   pv[8 * hf + 4], pv[8 * hf + 5], pv[8 * hf + 6], pv[8 * hf + 7]);
                sb[hf] = to_bf16x8(dsv[8 * hf], dsv[8 * hf + 1], dsv[8 * hf + 2], dsv[8 * hf + 3],
                                   dsv[8 * hf + 4], dsv[8 * hf + 5], dsv[8 * hf + 6], dsv[8 * hf + 7]);
            }
            // the B operands were just written by VALU: 5 wait states before
            // the first asm MFMA reads them
            asm volatile("s_nop 4" : "+v"(pb[0]), "+v"(pb[1]), "+v"(sb[0]), "+v"(sb[1]));
            // dV^T += dO^T P and dK^T += Q^T dS over these 32 rows (two 16-row
            // halves); step j = (hf, db), operands loaded TPF steps ahead
            constexpr int TPF = 2;
            bf16x8 tg[TPF + 1], tq[TPF + 1];
#pragma unroll
            for (int i = 0; i < TPF; ++i) {
                tg[i] = tr_operand(gtile, 32 * mb + 16 * (i >> 2), i & 3);
                tq[i] = tr_operand(qtile, 32 * mb + 16 * (i >> 2), i & 3);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j + TPF < 8) {
                    const int jn = j + TPF;
                    tg[jn % (TPF + 1)] = tr_operand(gtile, 32 * mb + 16 * (jn >> 2), jn & 3);
                    tq[jn % (TPF + 1)] = tr_operand(qtile, 32 * mb + 16 * (jn >> 2), jn & 3);
                }
                const int hf = j >> 2, db = j & 3;
                mfma_o_acc(tg[j % (TPF + 1)], pb[hf], dvacc[db]);
                mfma_o_acc(tq[j % (TPF + 1)], sb[hf], dkacc[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // ---- ring: steps 0 .. NSTAGE-2 in flight ----
#pragma unroll
    for (int i = 0; i < KA_NSTAGE - 1; ++i)
        if (i < n_steps) issue_step(i);
    // Every load so far (the wave's resident operands and the prologue
    // copies) has landed: the compiler then puts no wait for the resident
    // operands inside the loop, whose only outstanding loads are the ring's
    // copies (which it does not track).
    wait_vmcnt<0>();

    int cs_h = 0, cs_qt = qt_end - 1;           // step being computed
    for (int s = 0; s < n_steps; ++s) {
        wait_steps(min(KA_NSTAGE - 2, n_steps - 1 - s));
        raw_barrier();                           // step s landed everywhere; step s-1 done
        if (s + KA_NSTAGE - 1 < n_steps) issue_step(s + KA_NSTAGE - 1);

        const int r0 = cs_qt * TROWS;
        if (++cs_h == p.G) { cs_h = 0; --cs_qt; }
        // does any row of the tile see any key of this wave?
        const bool active = kw0 < T && (!p.causal || r0 + TROWS - 1 >= kw0) &&
                            (p.window <= 0 || r0 <= kw0 + 31 + p.window - 1);
        if (!active) continue;
        const bool need_mask = (p.causal && r0 < kw0 + 31) ||
                               (p.window > 0 && r0 + TROWS - 1 - kw0 >= p.window) ||
                               (r0 + TROWS > T);
        const char *qtile = smem + (s % KA_NSTAGE) * KA_STAGE;
        const char *gtile = qtile + TBYTES;
        const char *stat = gtile + TBYTES;
        step_rows(need_mask, qtile, gtile, stat, r0);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        settle_acc(dkacc[db]);
        settle_acc(dvacc[db]);
    }

    // dK^T / dV^T element i of d-block db: d = 32 db + 8 (i / 4) + 4 hi + (i % 4), key `key`
    if (key >= T) return;
    __bf16 *dkrow = p.dk + kv_base + (size_t)key * D;
    __bf16 *dvrow = p.dv + kv_base + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * db + 8 * q4 + 4 * hi;
            u32x2 wk = {pack_bf16x2(dkacc[db][4 * q4] * p.scale, dkacc[db][4 * q4 + 1] * p.scale),
                        pack_bf16x2(dkacc[db][4 * q4 + 2] * p.scale, dkacc[db][4 * q4 + 3] * p.scale)};
            u32x2 wv = {pack_bf16x2(dvacc[db][4 * q4], dvacc[db][4 * q4 + 1]),
                        pack_bf16x2(dvacc[db][4 * q4 + 2], dvacc[db][4 * q4 + 3])};
            *reinterpret_cast<u32x2 *>(dkrow + d) = wk;
            *reinterpret_cast<u32x2 *>(dvrow + d) = wv;
        }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 256 query rows x heads of one K/V group (as the forward);
// wave = 32 query rows of one head; 64-key K / V tiles stream through LDS.
constexpr int KB_WAVES = 8;
constexpr int KB_NSTAGE = 3;
constexpr int KB_STAGE = 2 * TBYTES;         // K tile, V tile
constexpr int KB_NBLK = 2 * TBLK;            // 40
constexpr int KB_PER_WAVE = KB_NBLK / KB_WAVES;   // 5
constexpr int KB_LDS = KB_NSTAGE * KB_STAGE;
constexpr int WG_ROWS = 256;

__global__ __launch_bounds__(64 * KB_WAVES, 1) void bwd_dq_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int q16 = lane >> 4;
    const int j16 = lane & 15;
    const int T = p.T;

    const int id = blockIdx.x;
    const int rb = p.n_row_blocks - 1 - id / p.n_head_groups;
    const int hg = id % p.n_head_groups;
    const int subs = p.G / p.hpw;
    const int sub = hg % subs;
    const int g = (hg / subs) % p.hkv;
    const int b = hg / (subs * p.hkv);
    const int wph = KB_WAVES / p.hpw;
    const int h = g * p.G + sub * p.hpw + wave / wph;
    const int r0 = rb * p.rows_per_wg;
    const int rw0 = r0 + (wave % wph) * 32;
    const int row0 = rw0 + l32;

    const int kend = p.causal ? min(T, r0 + p.rows_per_wg) : T;
    const int kbeg = p.window > 0 ? max(0, r0 - p.window + 1) : 0;
    const int t_begin = kbeg / TROWS;
    const int t_end = (kend + TROWS - 1) / TROWS;
    const int n_tiles = max(t_end - t_begin, 0);
    const bool wave_active = rw0 < T;
    const int kend_w = p.causal ? min(T, rw0 + 32) : T;
    const int kbeg_w = p.window > 0 ? max(0, rw0 - p.window + 1) : 0;

    const size_t bh = (size_t)b * p.hq + h;
    const size_t q_base = bh * (size_t)T * D;
    const size_t kv_base = ((size_t)b * p.hkv + g) * (size_t)T * D;
    // Q^T and dO^T B operands of row row0: d = 16 ks + 8 hi .. +7
    bf16x8 qop[8], gop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        u32x4 a4 = {0u, 0u, 0u, 0u}, g4 = {0u, 0u, 0u, 0u};
        if (row0 < T) {
            a4 = ldg16(p.q + q_base + (size_t)row0 * D + 16 * ks + 8 * hi);
            g4 = ldg16(p.dout + q_base + (size_t)row0 * D + 16 * ks + 8 * hi);
        }
        qop[ks] = __builtin_bit_cast(bf16x8, a4);
        gop[ks] = __builtin_bit_cast(bf16x8, g4);
    }
    f32x2 strow = {INFINITY, 0.f};
    if (row0 < p.Tpad) strow = *reinterpret_cast<const f32x2 *>(p.stats + 2 * (bh * p.Tpad + row0));
    const float l2row = strow[0], ddrow = strow[1];
    f32x16 dqacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

    uint32_t dma_off[KB_PER_WAVE];
    int dma_row[KB_PER_WAVE];
#pragma unroll
    for (int i = 0; i < KB_PER_WAVE; ++i)
        tile_src((KB_PER_WAVE * wave + i) % TBLK, lane, dma_row[i], dma_off[i]);
    const bool dma_v = KB_PER_WAVE * wave >= TBLK;   // waves 0-3 copy K, 4-7 copy V
    const uint32_t smem_lds = lds_offset(smem);
    auto issue_tile = [&](int t) {
        const int ts = t * TROWS;
        const __bf16 *src = (dma_v ? p.v : p.k) + kv_base + (size_t)ts * D;
        const int last = T - 1 - ts;
        const uint32_t stage = smem_lds + ((t - t_begin) % KB_NSTAGE) * KB_STAGE + (dma_v ? TBYTES : 0);
#pragma unroll
        for (int i = 0; i < KB_PER_WAVE; ++i) {
            const uint32_t off = dma_row[i] > last
                ? dma_off[i] - (uint32_t)((dma_row[i] - last) * D * 2) : dma_off[i];
            dma16_off_at(src, off, stage + ((KB_PER_WAVE * wave + i) % TBLK) * 1024);
        }
    };

    const int tr_row = 4 * hi + (j16 >> 2);
    const int tr_ch = 2 * (q16 & 1) + ((j16 & 3) >> 1);
    const int tr_byte = 8 * (j16 & 1);
    const float c = p.c;

#pragma unroll
    for (int i = 0; i < KB_NSTAGE - 1; ++i)
        if (i < n_tiles) issue_tile(t_begin + i);
    // Every load so far (the wave's resident operands and the prologue
    // copies) has landed: the compiler then puts no wait for the resident
    // operands inside the loop, whose only outstanding loads are the ring's
    // copies (which it does not track).
    wait_vmcnt<0>();

    for (int t = t_begin; t < t_end; ++t) {
        const int rel = t - t_begin;
        if (n_tiles - 1 - rel >= 1) wait_vmcnt<KB_PER_WAVE>();
        else wait_vmcnt<0>();
        raw_barrier();
        if (t + KB_NSTAGE - 1 < t_end) issue_tile(t + KB_NSTAGE - 1);

        const int ts = t * TROWS;
        const bool active = wave_active && ts < kend_w && ts + TROWS > kbeg_w;
        if (!active) continue;
        const bool need_mask = (ts + TROWS > T) || (p.causal && ts + TROWS - 1 > rw0) ||
                               (p.window > 0 && (rw0 + 31) - ts >= p.window);
        const char *ktile = smem + (rel % KB_NSTAGE) * KB_STAGE;
        const char *vtile = ktile + TBYTES;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // S^T = K Q^T and dP^T = V dO^T for keys 32 kb .. 32 kb + 31 of the tile
            f32x16 sacc, pacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; pacc[i] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(ktile + toff(32 * kb + l32, 2 * ks + hi));
                const bf16x8 av = *reinterpret_cast<const bf16x8 *>(vtile + toff(32 * kb + l32, 2 * ks + hi));
                sacc = mfma32x32x16(ak, qop[ks], sacc);
                pacc = mfma32x32x16(av, gop[ks], pacc);
            }
            // element i: key ts + 32 kb + 8 (i / 4) + 4 hi + (i % 4) of row row0
            float dsv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pe = fast_exp2(__builtin_fmaf(sacc[i], c, -l2row));
                dsv[i] = pe * (pacc[i] - ddrow);
            }
            // the keys this row sees form one range of the offset e within
            // the tile: below T, at or before the row, within the window
            if (need_mask) {
                int e_hi = min(T - ts, TROWS);
                if (p.causal) e_hi = min(e_hi, row0 - ts + 1);
                const int lo = p.window > 0 ? min(max(row0 - ts - p.window + 1, 0), TROWS) : 0;
                const uint32_t width = (uint32_t)max(e_hi - lo, 0);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
                    dsv[i] = (uint32_t)(e - lo) < width ? dsv[i] : 0.f;
                }
            }
            bf16x8 sb[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                sb[hf] = to_bf16x8(dsv[8 * hf], dsv[8 * hf + 1], dsv[8 * hf + 2], dsv[8 * hf + 3],
                                   dsv[8 * hf + 4], dsv[8 * hf + 5], dsv[8 * hf + 6], dsv[8 * hf + 7]);
            // dQ^T += K^T dS^T over these 32 keys
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int r = 32 * kb + 16 * hf + tr_row;
                    const bf16x4 lo4 = lds_read_tr16(ktile + toff(r, 4 * db + tr_ch) + tr_byte);
                    const bf16x4 hi4 = lds_read_tr16(ktile + toff(r + 8, 4 * db + tr_ch) + tr_byte);
                    const bf16x8 ak = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                    dqacc[db] = mfma32x32x16(ak, sb[hf], dqacc[db]);
                }
        }
    }

    if (!wave_active || row0 >= T) return;
    __bf16 *qrow = p.dq + q_base + (size_t)row0 * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * db + 8 * q4 + 4 * hi;
            u32x2 w = {pack_bf16x2(dqacc[db][4 * q4] * p.scale, dqacc[db][4 * q4 + 1] * p.scale),
                       pack_bf16x2(dqacc[db][4 * q4 + 2] * p.scale, dqacc[db][4 * q4 + 3] * p.scale)};
            *reinterpret_cast<u32x2 *>(qrow + d) = w;
        }
}

}  // namespace

hipError_t launch_prefill_bwd_bf16_d128(const PrefillBwdArgs &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.k = static_cast<const __bf16 *>(a.k);
    p.v = static_cast<const __bf16 *>(a.v);
    p.o = static_cast<const __bf16 *>(a.o);
    p.dout = static_cast<const __bf16 *>(a.dout);
    p.lse = a.lse;
    p.dq = static_cast<__bf16 *>(a.dq);
    p.dk = static_cast<__bf16 *>(a.dk);
    p.dv = static_cast<__bf16 *>(a.dv);
    p.stats = a.ws_stats;
    p.stats_w = a.ws_stats;
    p.B = a.B;
    p.T = a.T;
    p.Tpad = a.Tpad;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.causal = a.causal;
    p.window = a.window;
    p.scale = a.scale;
    p.c = a.scale * kLog2e;
    p.sinks = a.sinks;
    p.dsinks = a.dsinks;
    p.hpw = (p.G % 8 == 0) ? 8 : (p.G % 4 == 0) ? 4 : (p.G % 2 == 0 ? 2 : 1);
    p.rows_per_wg = WG_ROWS / p.hpw;
    p.n_row_blocks = (a.T + p.rows_per_wg - 1) / p.rows_per_wg;
    p.n_head_groups = a.B * a.hkv * (p.G / p.hpw);

    hipError_t e = ensure_dynamic_lds((const void *)bwd_dkdv_kernel, KA_LDS);
    if (e != hipSuccess) return e;
    e = ensure_dynamic_lds((const void *)bwd_dq_kernel, KB_LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)(a.Tpad / 16), (unsigned)(a.B * a.hq)), dim3(256),
                       0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long n_kb = ((long long)a.T + KA_KEYS - 1) / KA_KEYS;
    const long long n_a = n_kb * a.B * a.hkv;
    const long long n_b = (long long)p.n_row_blocks * p.n_head_groups;
    if (n_a > 0x7fffffffLL || n_b > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)n_a), dim3(64 * KA_WAVES), KA_LDS, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)n_b), dim3(64 * KB_WAVES), KB_LDS, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess || !a.dsinks) return e;
    hipLaunchKernelGGL(bwd_sink_grad_kernel, dim3((unsigned)a.hq), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mi355
