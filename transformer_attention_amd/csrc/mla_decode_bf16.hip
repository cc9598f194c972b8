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
//    4-stage ring filled by global_load_lds_dwordx4 (no staging registers,
//    non-temporal: the cache is read once), three tiles in flight per CU
//    while the fourth is consumed;
//  * each tile is stored once, row-major with rows 1216 bytes apart; the
//    score product reads it with 16-byte loads, the P.V product reads the
//    first 512 columns transposed with ds_read_b64_tr_b16, so the latent is
//    never copied;
//  * 4 waves (one per SIMD, up to 512 registers each), each owning 32 heads:
//    S^T[32 tokens x 32 heads] = K Q^T with v_mfma_f32_32x32x16_bf16 (the
//    wave's 32 queries, 576 wide, stay in registers as B operands), then
//    O^T[512 x 32 heads] += C^T P^T with the rounded probabilities as the B
//    operand straight from the score accumulator.  Every 16-byte LDS read
//    feeds a 32x32x16 MFMA, half the LDS bytes per FLOP of a 16-head split;
//  * the online-softmax state is per head (one lane column; the two lane
//    halves hold the two 16-token halves of a tile and share the max), and
//    the reference max only moves when a tile exceeds it by 2^8;
//  * the workgroup id runs over sequences fastest, so with a batch that is a
//    multiple of 8 all chunks of one sequence run on one XCD and share its
//    L2 for the query rows.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int DC = 512, DR = 64, DK = DC + DR;
constexpr int TB = 32;                    // tokens per tile
constexpr int ROWB = DK * 2;              // 1152 bytes per cache row in HBM
constexpr int LROW_SLOTS = 76;            // LDS row pitch in 16-byte slots (72 data + 4 pad)
constexpr int LROW = LROW_SLOTS * 16;     // 1216 bytes
constexpr int TILE_BYTES = 38 * 1024;     // 32 rows (last row ends at slot 2432) = 38 DMA blocks
constexpr int NSTAGE = 4;
constexpr int LDS_BYTES = NSTAGE * TILE_BYTES;   // 155648
constexpr int NW = 4;                     // waves per workgroup
constexpr int HPW = 32;                   // heads per wave
constexpr int HPC = NW * HPW;             // heads per workgroup (chunk)
constexpr int NBLK = TILE_BYTES / 1024;   // 38 one-KB DMA blocks per tile:
                                          // waves 0-1 issue 10, waves 2-3 issue 9
constexpr float TAU = 8.0f;

struct Params {
    const __bf16 *q, *c;
    const int32_t *seq_lens;
    // paged cache: c is [num_pages, page_size, DK]; position t of sequence b
    // is row t % page_size of page block_table[b * max_blocks + t / page_size]
    // (entries clamped to [0, num_pages - 1])
    const int32_t *block_table;
    int max_blocks, page_size, num_pages;
    __bf16 *ws_o;
    float *ws_lse;
    int B, S_max, H;
    int split, n_split_max, n_hchunk;
    float scale_log2;
};

// Row r of a tile starts at slot 76 r + rho(r), rho(r) = (r / 4) mod 4, and
// holds its 72 16-byte chunks contiguously (4 pad slots per row).  With 64
// four-byte banks (16 slots):
//  * 16 consecutive rows at one chunk (the 16-byte score-operand reads of a
//    quarter wave) hit slots 12 r + rho(r) + c = 16 distinct values;
//  * 4 rows 4j..4j+3 x 64 bytes (what a half wave reads through the
//    transposing load) start at slots 12 i + rho + const, i.e. four disjoint
//    4-slot groups;
// so neither read pattern has bank conflicts, and every address stays affine
// in the loop indices.
__device__ __forceinline__ int row_slot(int r) { return LROW_SLOTS * r + ((r >> 2) & 3); }

// PAGED: tiles start at multiples of 32 tokens (chunks start at multiples of
// the split, itself a multiple of 64), so a tile never straddles two pages
// when the page size is a multiple of 32.
template <bool PAGED>
__global__ __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l32 = lane & 31;
    const int hh = lane >> 5;                 // lane half: which 16 tokens of a tile

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

    const char *cg = PAGED ? nullptr : reinterpret_cast<const char *>(p.c + (size_t)b * p.S_max * DK);

    // Issue the DMA of tile `t` (relative) into its ring stage: this wave's
    // 1-KB blocks.  LDS slot q = (1024*blk + 16*lane) / 16 of the stage holds
    // row r = q / 76, chunk q - row_slot(r); the pad slots and the slots past
    // row 31 receive an arbitrary valid chunk.  Rows past the chunk end
    // re-read the last valid row (their scores are masked).
    const int my_blk0 = wave < 2 ? 10 * wave : 20 + 9 * (wave - 2);
    const int my_nblk = wave < 2 ? 10 : 9;
    // Byte offset (within a tile's 32 cache rows) that lane `lane` copies for
    // each of this wave's blocks; pad slots re-read a valid chunk.
    uint32_t dma_off[10];
    int dma_row[10];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const int q = (my_blk0 + min(i, my_nblk - 1)) * 64 + lane;     // slot index in the tile
        const int r = q / LROW_SLOTS;
        const int c = min(max(q - row_slot(r), 0), DK / 8 - 1);
        dma_row[i] = r;
        dma_off[i] = (uint32_t)(r * ROWB + c * 16);
    }
    auto issue_tile = [&](int t) {
        char *stage = smem + (t % NSTAGE) * TILE_BYTES;
        const int t0 = lo + t * TB;
        const char *gbase;
        if constexpr (PAGED) {
            int pg = ld_uniform(p.block_table, b * p.max_blocks + t0 / p.page_size);
            pg = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
            gbase = reinterpret_cast<const char *>(p.c) +
                    ((size_t)pg * p.page_size + (t0 % p.page_size)) * ROWB;
        } else {
            gbase = cg + (size_t)t0 * ROWB;
        }
        const int last = hi_tok - 1 - t0;       // last valid row of this tile
        if (last >= TB - 1) {
#pragma unroll
            for (int i = 0; i < 10; ++i) {
                if (i >= my_nblk) break;
                dma16_off<true>(gbase, dma_off[i], stage + (my_blk0 + i) * 1024);
            }
        } else {                                // ragged last tile: rows past the end re-read the last row
#pragma unroll
            for (int i = 0; i < 10; ++i) {
                if (i >= my_nblk) break;
                const uint32_t off = dma_row[i] > last
                    ? dma_off[i] - (uint32_t)((dma_row[i] - last) * ROWB) : dma_off[i];
                dma16_off<true>(gbase, off, stage + (my_blk0 + i) * 1024);
            }
        }
    };

    // Prologue: tiles 0..NSTAGE-2 in flight.
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t)
        if (t < n_tiles) issue_tile(t);

    // The wave's 32 queries as B operands: head = hc*128 + 32*wave + l32,
    // d = 16ks + 8*hh .. +7.
    const int h = hc * HPC + wave * HPW + l32;
    const bool head_ok = h < p.H;
    bf16x8 qop[DK / 16];
    {
        const __bf16 *qrow = p.q + ((size_t)b * p.H + (head_ok ? h : 0)) * DK + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) {
            u32x4 val = ldg16(qrow + 16 * ks);
            if (!head_ok) val = u32x4{0u, 0u, 0u, 0u};
            qop[ks] = __builtin_bit_cast(bf16x8, val);
        }
    }

    f32x16 oacc[DC / 32];
#pragma unroll
    for (int db = 0; db < DC / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    float thr_raw = -INFINITY;              // raw-score level that moves the reference max

    // C^T operand (32 d x 16 tokens) through the transposing read.  K slot j
    // of lane half hh in token step kk is token 16kk + 8(j/4) + 4hh + (j%4),
    // the order in which the score accumulator holds the probabilities.  Lane
    // L of 16-lane group G addresses token row 16kk + 4(G/2) + L/4 (second
    // read: +8) at d = 32db + 16(G%2) + 4(L%4), so result lane i of group G
    // receives d = 32db + 16(G%2) + i, i.e. A row l % 32.
    const int g16 = lane >> 4;
    const int L16 = lane & 15;
    // token row 16kk + 4(G/2) + L/4 (+8): rho = G/2 (+2), independent of kk
    const int v_byte_lane = LROW * (4 * (g16 >> 1) + (L16 >> 2)) + 16 * (g16 >> 1) +
                            32 * (g16 & 1) + 8 * (L16 & 3);

    constexpr int NKS = DK / 16;              // 36 k-steps of the score product
    constexpr int PF = 3;                     // LDS operand loads issued ahead of their MFMA
    for (int t = 0; t < n_tiles; ++t) {
        // Tile t landed once at most (NSTAGE-2) newer tiles are pending.  The
        // q loads above were issued after the prologue DMAs, so the first
        // iteration waits for everything.
        const int newer = t == 0 ? 0 : min(NSTAGE - 2, n_tiles - 1 - t);
        if (newer == 0) wait_vmcnt<0>();
        else if (newer == 1) { if (my_nblk == 10) wait_vmcnt<10>(); else wait_vmcnt<9>(); }
        else { if (my_nblk == 10) wait_vmcnt<20>(); else wait_vmcnt<18>(); }
        raw_barrier();                          // every wave's part of tile t is in LDS,
                                                // and stage (t-1) is no longer read

        const char *kt = smem + (t % NSTAGE) * TILE_BYTES;
        const int t0 = lo + t * TB;
        // S^T (32 tokens x 32 heads): A = token row l32, d chunk 2ks + hh.
        // The operand of k-step ks + PF is loaded before the MFMA of k-step
        // ks; the next tile's copies are issued after the first few MFMAs.
        const char *krow = kt + 16 * (row_slot(l32) + hh);
        bf16x8 ka[PF + 1];
#pragma unroll
        for (int i = 0; i < PF; ++i) ka[i] = *reinterpret_cast<const bf16x8 *>(krow + 32 * i);
        f32x16 sacc;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (ks + PF < NKS)
                ka[(ks + PF) % (PF + 1)] = *reinterpret_cast<const bf16x8 *>(krow + 32 * (ks + PF));
            const bf16x8 a = ka[ks % (PF + 1)];
            if (ks == 0) sacc = mfma_s_first(a, qop[0]);
            else if (ks == NKS - 1) sacc = mfma_s_last(a, qop[ks], sacc);
            else sacc = mfma_s_acc(a, qop[ks], sacc);
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 2 && t + NSTAGE - 1 < n_tiles) {
                issue_tile(t + NSTAGE - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // element i of this lane is token t0 + 8(i/4) + 4hh + (i%4) of head column l32
        float mx = -INFINITY;
        if (t0 + TB > hi_tok) {                 // ragged last tile: mask the rows past the end
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tok = t0 + 8 * (i >> 2) + 4 * hh + (i & 3);
                sacc[i] = tok < hi_tok ? sacc[i] : -INFINITY;
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
        // The reference max moves only when some lane's raw score exceeds
        // thr_raw = (m_run + TAU) / scale_log2 (tile 0 always: thr_raw starts
        // at -inf).  Only then is the head's max taken over both lane halves.
        float alpha = 1.0f;
        if (__any(mx > thr_raw)) {
            const float mxp = pair32_max(mx) * p.scale_log2;
            const bool upd = mxp > m_run + TAU;
            const float m_new = upd ? mxp : m_run;
            alpha = upd ? fast_exp2(m_run - m_new) : 1.0f;
            if (t > 0) {                        // before tile 0 the output is still zero
#pragma unroll
                for (int db = 0; db < DC / 32; ++db) scale_acc(oacc[db], alpha);
            }
            m_run = m_new;
            thr_raw = (m_run + TAU) / p.scale_log2;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        // p = 2^(s * scale_log2 - m): one FMA and one exp per score
        // (computed in place: sacc[i] becomes the probability of score i)
#pragma unroll
        for (int i = 0; i < 8; ++i) sacc[i] = fast_exp2(__builtin_fmaf(sacc[i], p.scale_log2, -m_use));
        const bf16x8 pop0 = to_bf16x8(sacc[0], sacc[1], sacc[2], sacc[3], sacc[4], sacc[5], sacc[6], sacc[7]);
        __builtin_amdgcn_sched_barrier(0);

        // O^T += C^T P^T: token step kk = 0 for all d-blocks (the second half
        // of the probabilities is computed in the shadow of these MFMAs),
        // then kk = 1.
        const char *vbase = kt + v_byte_lane;
        bf16x4 va[PF + 1][2];
        auto vload = [&](int j, bf16x4 *dst) {     // j = kk * 16 + db
            const char *vb = vbase + (16 * (j >> 4)) * LROW + 64 * (j & 15);
            dst[0] = lds_read_tr16(vb);
            dst[1] = lds_read_tr16(vb + 8 * LROW + 32);
        };
#pragma unroll
        for (int i = 0; i < PF; ++i) vload(i, va[i]);
        bf16x8 pop1;
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < 2 * (DC / 32); ++j) {
            if (j + PF < 2 * (DC / 32)) vload(j + PF, va[(j + PF) % (PF + 1)]);
            const bf16x4 *v = va[j % (PF + 1)];
            const bf16x8 a = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
            const int db = j & 15;
            if (j < 16) {
                oacc[db] = mfma32x32x16(a, pop0, oacc[db]);
                if (j < 8) {                    // second half of the probabilities
                    sacc[8 + j] = fast_exp2(__builtin_fmaf(sacc[8 + j], p.scale_log2, -m_use));
                }
                if (j == 8) {
                    pop1 = to_bf16x8(sacc[8], sacc[9], sacc[10], sacc[11], sacc[12], sacc[13], sacc[14], sacc[15]);
#pragma unroll
                    for (int i = 0; i < 16; ++i) lsum += sacc[i];
                }
            } else {
                oacc[db] = mfma32x32x16(a, pop1, oacc[db]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run = l_run * alpha + lsum;
    }

    const float lt = pair32_sum(l_run);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    // The normalised partial O goes out as bf16 through LDS, so that every
    // store writes one head's whole 1-KB row (straight from the registers
    // each store would touch 32 heads' rows, 32 bytes apiece).  All tiles
    // have landed and every wave is past its last read of the ring.
    raw_barrier();
    store_partial_rows(smem, wave, lane, oacc, inv, p.ws_o, ((size_t)b * p.H + hc * HPC + wave * HPW) * p.n_split_max + s,
                       p.n_split_max, p.H - (hc * HPC + wave * HPW));
    if (head_ok && hh == 0) p.ws_lse[((size_t)b * p.H + h) * p.n_split_max + s] = lt > 0.f ? m_run + __log2f(lt) : -INFINITY;
}

}  // namespace

hipError_t launch_mla_decode_bf16(const MlaArgs &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.c = static_cast<const __bf16 *>(a.cache);
    p.seq_lens = a.seq_lens;
    p.block_table = a.block_table;
    p.max_blocks = a.max_blocks;
    p.page_size = a.page_size;
    p.num_pages = a.num_pages;
    p.ws_o = a.ws_o;
    p.ws_lse = a.ws_lse;
    p.B = a.B;
    p.S_max = a.S_max;
    p.H = a.H;
    p.split = a.split;
    p.n_split_max = a.n_split_max;
    p.scale_log2 = a.scale * kLog2e;
    hipError_t e = a.block_table ? ensure_dynamic_lds((const void *)mla_decode_kernel<true>, LDS_BYTES)
                                 : ensure_dynamic_lds((const void *)mla_decode_kernel<false>, LDS_BYTES);
    if (e != hipSuccess) return e;
    p.n_hchunk = (a.H + HPC - 1) / HPC;
    const long long n_wg = (long long)a.B * a.n_split_max * p.n_hchunk;
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.block_table)
        hipLaunchKernelGGL(mla_decode_kernel<true>, dim3((unsigned)n_wg), dim3(64 * NW), LDS_BYTES,
                           stream, p);
    else
        hipLaunchKernelGGL(mla_decode_kernel<false>, dim3((unsigned)n_wg), dim3(64 * NW), LDS_BYTES,
                           stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_combine(a.ws_o, a.ws_lse, a.seq_lens, a.o, a.lse, a.B, a.H, DC, a.S_max,
                                a.split, a.n_split_max, a.sinks, stream, /*partial_bf16=*/true);
}

}  // namespace mi355
