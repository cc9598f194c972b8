// decode_bf16.hip -- single-token GQA decode against a bf16 or FP8 (E4M3) KV
// cache (d_h = 128), split over the cache ("flash-decoding"), plus the
// log-sum-exp merge of the split partials shared with the MLA decode.
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
// The cache of each (sequence, K/V head) is cut into chunks of `split` keys.
// A unit of work is one chunk of one K/V head for up to 16 of its query
// heads; its K/V bytes are read from HBM once.  A small plan kernel counts
// the units of every sequence (prefix sums in the workspace); the main kernel
// is persistent: every wave walks its own list of units (unit ids w, w + W,
// ... for W waves in the grid) and streams their 32-key tiles continuously:
//  * tiles go HBM -> LDS through a private 2-stage ring per wave, filled by
//    global_load_lds_dwordx4 (no staging registers, no workgroup barrier:
//    a wave waits only for its own copies); the ring keeps streaming across
//    unit boundaries, so there is no per-unit pipeline drain or refill;
//  * K rows are stored 272 bytes apart (17 16-byte slots: 16 consecutive rows
//    of one column hit 16 distinct bank slots) and V rows 288 bytes apart
//    (18 = 2 mod 16: the 8 rows x 32 bytes a half-wave reads through the
//    transposing load hit 16 distinct slots); all addresses are base + imm;
//  * per tile: S^T = K q^T with v_mfma_f32_16x16x32_bf16 (the group's heads
//    are the 16 columns), online softmax per head column, then O^T = V^T P^T
//    with V^T read by ds_read_b64_tr_b16 and the rounded probabilities as the
//    B operand;
//  * at the end of a unit the wave writes the chunk's normalised partial
//    output and log-sum-exp; a second kernel merges the chunks of each
//    (sequence, head): L = log sum_s exp(L_s), O = sum_s exp(L_s - L) O_s,
//    the FlashAttention-2 state merge ("Attention Engineering ...", section 4).
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int D = 128;
constexpr int BN = 32;                    // keys per tile
#ifndef DECODE_NW
#define DECODE_NW 4
#endif
#ifndef DECODE_NSTG
#define DECODE_NSTG 2
#endif
constexpr int NW = DECODE_NW;             // waves per workgroup (independent)
constexpr int NSTG = DECODE_NSTG;         // stages of each wave's private ring
constexpr int KROW = D * 2 + 16;          // 272 B
constexpr int VROW = D * 2 + 32;          // 288 B
constexpr int KREG = 9 * 1024;            // K rows (8704 B) padded to whole one-KB DMA blocks, so
                                          // no block straddles the K and V regions
constexpr int STAGE_BLK = (KREG + BN * VROW + 1023) / 1024;      // 18 one-KB blocks
constexpr int STAGE_BYTES = STAGE_BLK * 1024;                   // 18432 B
constexpr int WAVE_BYTES = NSTG * STAGE_BYTES;                  // private ring
constexpr int QBUF_BYTES = 16 * D * 2;                          // one unit's 16 query rows
constexpr int LDS_BYTES = NW * (WAVE_BYTES + QBUF_BYTES);
static_assert(LDS_BYTES <= 160 * 1024, "decode rings exceed the LDS");
static_assert(NSTG >= 2 && NSTG <= 4, "the wait below handles up to 3 tiles in flight");
constexpr float TAU = 8.0f;
// FP8 cache: K and V rows of 128 one-byte codes stored 144 bytes apart (9
// 16-byte slots): the 8-byte row reads of 16 consecutive rows and the 8-bit
// transposing reads of 16 rows x 16 bytes both hit 64 distinct banks.
constexpr int ROW8 = D + 16;              // 144 B
constexpr int KREG8 = 5 * 1024;           // K rows (4608 B) padded to whole one-KB blocks
constexpr int STAGE_BLK8 = 10;            // K and V regions of an FP8 stage
static_assert(BN * ROW8 <= KREG8 && KREG8 + BN * ROW8 <= STAGE_BLK8 * 1024, "FP8 stage layout");
#ifndef DECODE8_NSTG
#define DECODE8_NSTG 2
#endif
#ifndef DECODE8_NW
#define DECODE8_NW 6
#endif
// An FP8 stage is 10 KB instead of 18, so the FP8 kernel runs six waves per
// workgroup (measured at the 70B workload: 0.418 ms against 0.437 ms with
// four; a third ring stage with four waves gave nothing).
template <bool FP8> struct Layout {
    static constexpr int nstg = FP8 ? DECODE8_NSTG : NSTG;
    static constexpr int nw = FP8 ? DECODE8_NW : NW;
    static constexpr int blk = FP8 ? STAGE_BLK8 : STAGE_BLK;      // one-KB copy blocks per stage
    static constexpr int bytes = blk * 1024;
    static constexpr int wave = nstg * bytes;
    static constexpr int lds = nw * (wave + QBUF_BYTES);
    static constexpr int kreg = FP8 ? KREG8 : KREG;
    static constexpr int krow = FP8 ? ROW8 : KROW;
    static constexpr int vrow = FP8 ? ROW8 : VROW;
    static constexpr int row_bytes = FP8 ? D : 2 * D;              // one cache row in HBM
};

struct Params {
    const __bf16 *q;
    const char *k, *v;                    // bf16 rows or FP8 (E4M3) codes
    // FP8: one scale per 32 positions of a K/V head: contiguous
    // [B, h_kv, n_stiles], paged [num_pages, h_kv, page_size / 32]
    const float *k_scales, *v_scales;
    int n_stiles;
    const int32_t *seq_lens;
    // paged cache: k and v are [num_pages, h_kv, page_size, D]; position t of
    // sequence b is row t % page_size of page block_table[b * max_blocks +
    // t / page_size] (entries clamped to [0, num_pages - 1])
    const int32_t *block_table;
    int max_blocks, page_size, num_pages;
    const int32_t *plan;                  // [B+1] unit prefix sums
    float *ws_o, *ws_lse;
    int B, S_max, hq, hkv, G, n_hchunk;
    int split, n_split_max, window;
    float scale_log2;
};

// pre[b] = number of units of sequences 0..b-1; units of a sequence are
// ceil(len / split) chunks x h_kv x n_hchunk.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t *seq_lens, int B, int S_max,
                                                           int split, int mult, int32_t *pre) {
    __shared__ int sc[1024];
    int carry = 0;
    const int t = threadIdx.x;
    if (t == 0) pre[0] = 0;
    for (int base = 0; base < B; base += 1024) {
        const int b = base + t;
        int cnt = 0;
        if (b < B) {
            int len = seq_lens[b];
            len = len < 0 ? 0 : (len > S_max ? S_max : len);
            cnt = (len + split - 1) / split * mult;
        }
        sc[t] = cnt;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {         // inclusive scan
            const int v = t >= off ? sc[t - off] : 0;
            __syncthreads();
            sc[t] += v;
            __syncthreads();
        }
        if (b < B) pre[b + 1] = carry + sc[t];
        carry += sc[1023];
        __syncthreads();
    }
}

struct Unit {
    int b, g, hc, c;      // sequence, K/V head, head chunk, chunk index
    int lo, hi;           // visible key range of the chunk
    int t_first;          // first key of the first tile (lo, or lo rounded down to 32 when paged)
    int n_tiles;
};

// PAGED: the tiles of a chunk start on 32-key boundaries, so that a tile
// never straddles two pages (page sizes are multiples of 32); keys before
// the visible start of the first tile are masked.
// FP8: the cache holds E4M3 codes with one scale per 32-position tile of a
// head (tiles aligned as for PAGED, so each tile has one K and one V scale).
// A tile is copied to LDS as codes (half the bytes), the codes are widened
// to bf16 in registers (exact) as they are read for the MFMAs, the K scale
// multiplies the tile's scores and the V scale its probabilities in the P.V
// operand (the running sum l takes the unscaled probabilities).
template <bool PAGED, bool FP8>
__global__ __launch_bounds__(64 * Layout<FP8>::nw, 1) void decode_bf16_d128_kernel(Params p) {
    using LY = Layout<FP8>;
    constexpr int NSTG = LY::nstg;
    constexpr int NW = LY::nw;
    static_assert(LY::lds <= 160 * 1024 && NSTG >= 2 && NSTG <= 3, "decode ring");
    constexpr bool ALIGN = PAGED || FP8;
    constexpr int STAGE_BLK = LY::blk;
    constexpr int STAGE_BYTES = LY::bytes;
    constexpr int WAVE_BYTES = LY::wave;
    constexpr int KREG = LY::kreg;
    constexpr int KROW = LY::krow;
    constexpr int VROW = LY::vrow;
    constexpr int RB = LY::row_bytes;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int j16 = lane & 15;
    const int q16 = lane >> 4;
    const int wid = blockIdx.x * NW + wave;
    const int nwaves = gridDim.x * NW;
    const int total = ld_uniform(p.plan, p.B);
    char *ring = smem + wave * WAVE_BYTES;
    char *qbuf = smem + NW * WAVE_BYTES + wave * QBUF_BYTES;
    // Every vector-memory instruction of this kernel is issued through asm
    // (tile copies, query copies, partial stores), and `vmc` counts them, so
    // each wait below lets exactly the instructions issued after the one
    // waited for stay in flight (vmcnt drains in issue order).
    int vmc = 0;
    auto wait_after = [&](int mark) { wait_vmcnt_dyn(min(vmc - mark, 63)); };   // fewer is stricter

    // Unit id -> geometry.  Each cursor visits increasing unit ids, so its
    // sequence index is found by walking forward from its previous one.
    auto describe = [&](int u, int &walk_b) {
        // the three scalar loads of a step are issued together (one latency)
        int pb = ld_uniform(p.plan, walk_b);
        int pb1 = ld_uniform(p.plan, walk_b + 1);
        int len = ld_uniform(p.seq_lens, walk_b);
        while (walk_b + 1 < p.B && pb1 <= u) {
            ++walk_b;
            pb = pb1;
            pb1 = ld_uniform(p.plan, walk_b + 1);
            len = ld_uniform(p.seq_lens, walk_b);
        }
        Unit d;
        d.b = walk_b;
        len = len < 0 ? 0 : (len > p.S_max ? p.S_max : len);
        const int nc = (len + p.split - 1) / p.split;
        const int r = u - pb;
        const int gh = r / nc;
        d.c = r - gh * nc;
        d.g = gh / p.n_hchunk;
        d.hc = gh - d.g * p.n_hchunk;
        const int kvis = p.window > 0 ? max(0, len - p.window) : 0;
        d.lo = max(d.c * p.split, kvis);
        d.hi = min((d.c + 1) * p.split, len);
        d.t_first = ALIGN ? (d.lo & ~(BN - 1)) : d.lo;
        d.n_tiles = d.lo < d.hi ? (d.hi - d.t_first + BN - 1) / BN : 0;
        return d;
    };

    // Per-lane DMA offsets inside a tile: block i of a stage covers stage
    // bytes [1024 i, 1024 i + 1024); lane byte o = 1024 i + 16 lane holds K row
    // o / KROW (o < KREG; rows past 31 and pad slots take a valid chunk of the
    // last row) or V row (o - KREG) / VROW, chunk (remainder) / 16.
    // The byte offset of each block's lane chunk relative to the tile's
    // first K (or V) row is fixed; only the ragged last tile of a unit needs
    // its rows clamped.
    uint32_t blk_off[STAGE_BLK];
    unsigned is_v_mask = 0;
#pragma unroll
    for (int i = 0; i < STAGE_BLK; ++i) {
        const int o = i * 1024 + lane * 16;
        const bool is_v = i * 1024 >= KREG;         // wave-uniform: blocks never straddle K and V
        const int ro = is_v ? o - KREG : o;
        const int r = min(is_v ? ro / VROW : ro / KROW, BN - 1);
        const int col = min((ro - r * (is_v ? VROW : KROW)) >> 4, RB / 16 - 1) * 16;
        blk_off[i] = (uint32_t)(r * RB + col);
        is_v_mask |= (unsigned)is_v << i;
    }
    const uint32_t ring_lds = lds_offset(ring);

    // Fetch cursor: unit id fu (geometry fd), tile ft; fetched-tile counter nf;
    // vm_tile[s] = value of vmc once the tile in ring stage s was issued.
    int fu = wid, ft = 0, nf = 0, f_walk = 0;
    // At most NSTG (2 or 3) fetched tiles are unconsumed: vm_last / vm_prev /
    // vm_prev2 hold vmc after the issue of tile nf-1 / nf-2 / nf-3 (plain
    // scalars: an indexed array would live in scratch memory, whose accesses
    // are vector-memory instructions too).
    int vm_last = 0, vm_prev = 0, vm_prev2 = 0;
    // FP8: scale index of the tile in each ring stage
    long long sidx0 = 0, sidx1 = 0, sidx2 = 0;
    Unit fd;
    if (fu < total) fd = describe(fu, f_walk);
    auto fetch_skip_empty = [&]() {
        while (fu < total && ft >= fd.n_tiles) {
            fu += nwaves;
            ft = 0;
            if (fu < total) fd = describe(fu, f_walk);
        }
    };
    auto issue_next = [&]() {                        // issue the fetch cursor's tile
        fetch_skip_empty();
        if (fu >= total) return false;
        const int t0 = fd.t_first + ft * BN;
        size_t row0;                             // index of the tile's first row
        long long sidx = 0;
        if constexpr (PAGED) {
            int pg = ld_uniform(p.block_table, fd.b * p.max_blocks + t0 / p.page_size);
            pg = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
            row0 = ((size_t)pg * p.hkv + fd.g) * p.page_size + (t0 % p.page_size);
            sidx = ((long long)pg * p.hkv + fd.g) * (p.page_size / BN) + (t0 % p.page_size) / BN;
        } else {
            row0 = ((size_t)fd.b * p.hkv + fd.g) * (size_t)p.S_max + t0;
            sidx = ((long long)fd.b * p.hkv + fd.g) * p.n_stiles + t0 / BN;
        }
        if constexpr (FP8) {                     // branch-free: the stage is wave-uniform
            const int stg = nf % NSTG;
            sidx0 = stg == 0 ? sidx : sidx0;
            sidx1 = stg == 1 ? sidx : sidx1;
            sidx2 = stg == 2 ? sidx : sidx2;
        }
        const char *kg = p.k + row0 * RB;
        const char *vg = p.v + row0 * RB;
        const uint32_t stage = ring_lds + (nf % NSTG) * STAGE_BYTES;
        vmc += STAGE_BLK;
        vm_prev2 = vm_prev;
        vm_prev = vm_last;
        vm_last = vmc;
        if (t0 + BN <= fd.hi) {
#pragma unroll
            for (int i = 0; i < STAGE_BLK; ++i)
                dma16_off_at<true>(((is_v_mask >> i) & 1) ? vg : kg, blk_off[i], stage + i * 1024);
        } else {                                   // ragged tile: rows past the end re-read the last row
            const uint32_t lim = (uint32_t)(fd.hi - 1 - t0) * RB;
#pragma unroll
            for (int i = 0; i < STAGE_BLK; ++i) {
                const uint32_t row_b = blk_off[i] & ~(uint32_t)(RB - 1);
                const uint32_t off = row_b > lim ? lim + (blk_off[i] & (RB - 1)) : blk_off[i];
                dma16_off_at<true>(((is_v_mask >> i) & 1) ? vg : kg, off, stage + i * 1024);
            }
        }
        ++ft;
        ++nf;
        return true;
    };

    // V^T operand: lane j of group q16 addresses V row 4 q16 + j/4 (second
    // read: +16), d = 16 db + 4 (j%4) .. +3: chunk 2 db + (j%4)/2, byte 8 (j%2).
    // FP8: the transposing 8-bit read gives lane j16 column j16 of the 8 rows
    // addressed by its group's lane pairs; pair r addresses key
    // 16 (r / 4) + 4 q16 + r % 4 -- the key order of the probability operand
    // (the score accumulator's element order) -- bytes 8 (j16 % 2) .. +7 of a
    // 16-column block.  K codes: 8 bytes of row j16 (+16) at d = 8 q16 + 32 ks.
    const int v_lane_off = FP8
        ? KREG + (16 * ((j16 >> 1) >> 2) + 4 * q16 + ((j16 >> 1) & 3)) * VROW + 8 * (j16 & 1)
        : KREG + (4 * q16 + (j16 >> 2)) * VROW + ((j16 & 3) >> 1) * 16 + 8 * (j16 & 1);
    const int k_lane_off = FP8 ? j16 * KROW + q16 * 8 : j16 * KROW + q16 * 16;

    // Query rows of a unit: 16 heads x 256 B, contiguous in q, copied into the
    // wave's query buffer (4 one-KB blocks; rows past the group's heads
    // re-read its last head and are masked below).
    const uint32_t qbuf_lds = lds_offset(qbuf);
    int vm_q = 0, q_walk = 0;
    auto issue_q = [&](int u) {
        const Unit e = describe(u, q_walk);
        const int last = p.G - 1 - e.hc * 16;            // last valid row of the chunk
        const char *qg = reinterpret_cast<const char *>(p.q + ((size_t)e.b * p.hq + e.g * p.G + e.hc * 16) * D);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = min(4 * i + (lane >> 4), last);
            dma16_off_at(qg, (uint32_t)(row * D * 2 + (lane & 15) * 16), qbuf_lds + i * 1024);
        }
        vmc += 4;
        vm_q = vmc;
    };
    if (wid < total) issue_q(wid);

    // Prime the ring.
    bool more = true;
#pragma unroll
    for (int i = 0; i < NSTG; ++i)
        if (more) more = issue_next();
    int nc_done = 0;                                  // tiles consumed so far

    int c_walk = 0;
    for (int cu = wid; cu < total; cu += nwaves) {
        const Unit d = describe(cu, c_walk);
        const int hidx = d.hc * 16 + j16;
        const bool head_ok = hidx < p.G;
        const int h = d.g * p.G + hidx;
        // this unit's query rows (copied one unit ahead) -> B operands
        wait_after(vm_q);
        bf16x8 qop[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 val = *reinterpret_cast<const u32x4 *>(qbuf + j16 * D * 2 + (4 * ks + q16) * 16);
            if (!head_ok) val = u32x4{0u, 0u, 0u, 0u};
            qop[ks] = __builtin_bit_cast(bf16x8, val);
        }
        asm volatile("" ::: "memory");
        wait_lgkmcnt0();                              // the buffer may be refilled now
        if (cu + nwaves < total) issue_q(cu + nwaves);
        f32x4 oacc[8];
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.f;

        for (int j = 0; j < d.n_tiles; ++j) {
            // this tile is the nc_done-th fetched; a later one may be in flight
            float k_sc = 1.f, v_sc = 1.f;
            if constexpr (FP8) {                      // scalar loads, in flight during the wait
                const int stg = nc_done % NSTG;
                const long long si = stg == 0 ? sidx0 : (stg == 1 ? sidx1 : sidx2);
                k_sc = ld_uniform_f(p.k_scales, si);
                v_sc = ld_uniform_f(p.v_scales, si);
            }
            // this tile's copies landed (later tiles may still be in flight)
            wait_after(nc_done == nf - 1 ? vm_last : (nc_done == nf - 2 ? vm_prev : vm_prev2));
            const char *st = ring + (nc_done % NSTG) * STAGE_BYTES;
            const int t0 = d.t_first + j * BN;
            bf16x8 ka[2][4];
            bf16x8 vop[8];
            if constexpr (FP8) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        ka[mb][ks] = fp8x8_to_bf16x8(
                            *reinterpret_cast<const i32x2 *>(st + k_lane_off + 16 * mb * KROW + 32 * ks));
#pragma unroll
                for (int db = 0; db < 8; ++db) vop[db] = fp8x8_to_bf16x8(lds_read_tr8(st + v_lane_off + 16 * db));
            } else {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        ka[mb][ks] = *reinterpret_cast<const bf16x8 *>(st + k_lane_off + 16 * mb * KROW + 64 * ks);
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const bf16x4 v0 = lds_read_tr16(st + v_lane_off + 32 * db);
                    const bf16x4 v1 = lds_read_tr16(st + v_lane_off + 16 * VROW + 32 * db);
                    vop[db] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            }
            f32x4 sacc[2];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    if (ks == 0) sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    sacc[mb] = mfma16x16x32(ka[mb][ks], qop[ks], sacc[mb]);
                }
            // element (mb, i) of this lane is key t0 + 16 mb + 4 q16 + i of head column j16
            const bool tail = t0 + BN > d.hi || (ALIGN && t0 < d.lo);
            const float sl = FP8 ? p.scale_log2 * k_sc : p.scale_log2;
            float x[8];
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = sacc[mb][i] * sl;
                    const int key = t0 + 16 * mb + 4 * q16 + i;
                    if (tail) v = (key < d.hi && (!ALIGN || key >= d.lo)) ? v : -INFINITY;
                    x[4 * mb + i] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = pair32_max(mx);
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
            if constexpr (FP8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] *= v_sc;
            }
            const bf16x8 pop = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
#pragma unroll
            for (int db = 0; db < 8; ++db) oacc[db] = mfma16x16x32(vop[db], pop, oacc[db]);
            ++nc_done;
            // refill the consumed stage once every read of it has returned
            asm volatile("" ::: "memory");
            wait_lgkmcnt0();
            if (more) more = issue_next();
        }
        // the unit's partial result (an empty unit writes O = 0, L = -inf)
        float lt = l_run + shfl_xor(l_run, 16);
        lt = pair32_sum(lt);
        // The unit's partial result (asm stores, counted in vmc; lanes of
        // heads past the group store nothing; the four lanes of a head column
        // store the same log-sum-exp).
        {
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;
            const size_t ws = (((size_t)d.b * p.hq + h) * p.n_split_max + d.c);
            float *wo = p.ws_o + ws * D;
            const float lse2 = lt > 0.f ? m_run + __log2f(lt) : -INFINITY;
            if (head_ok) {
#pragma unroll
                for (int db = 0; db < 8; ++db) store16(wo + 16 * db + 4 * q16, oacc[db] * inv);
                store4(p.ws_lse + ws, lse2);
            }
            vmc += 9;
        }
    }
    wait_vmcnt<0>();
}

// Merge of the split partials: one wave per (sequence, head) row, four rows
// per workgroup.  Each lane owns DV/64 consecutive output values; the
// weights 2^(L_s - M) of the splits are computed once per lane (lane s holds
// split s of a 64-split chunk) and broadcast with readlane, and the partial
// rows of four splits are loaded before they are accumulated.
// An optional sink logit per head (sinks[h], natural-log units like the
// scaled scores) adds one more term to the merged denominator and carries no
// value: Z = sum_s 2^(L_s - M) + 2^(sink log2 e - M).
template <int DV, bool PB16>
__global__ __launch_bounds__(256) void split_combine_kernel(const void *ws_o_, const float *ws_lse,
                                                            const int32_t *seq_lens, __bf16 *o, float *lse,
                                                            int n_rows, int H, int S_max, int split,
                                                            int n_split_max, const float *sinks) {
    constexpr int PER = DV / 64;                  // 2 or 8 values per lane
    typedef __attribute__((ext_vector_type(PER))) float fvec;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int b = row / H;
    int len = ld_uniform(seq_lens, b);
    len = len < 0 ? 0 : (len > S_max ? S_max : len);
    const int ns = (len + split - 1) / split;
    const float *lrow = ws_lse + (size_t)row * n_split_max;
    // partial s of this row: PER values per lane, fp32 or (PB16) bf16
    typedef __attribute__((ext_vector_type(PER))) __bf16 bvec;
    const char *orow = static_cast<const char *>(ws_o_) +
                       ((size_t)row * n_split_max * DV + PER * lane) * (PB16 ? 2 : 4);
    auto part = [&](int sidx) -> fvec {
        const char *ptr = orow + (size_t)sidx * DV * (PB16 ? 2 : 4);
        if constexpr (PB16) return __builtin_convertvector(*reinterpret_cast<const bvec *>(ptr), fvec);
        else return *reinterpret_cast<const fvec *>(ptr);
    };

    float M = -INFINITY;
    for (int c0 = 0; c0 < ns; c0 += 64)
        M = fmaxf(M, c0 + lane < ns ? lrow[c0 + lane] : -INFINITY);
    M = fmaxf(M, shfl_xor(M, 1));
    M = fmaxf(M, shfl_xor(M, 2));
    M = fmaxf(M, shfl_xor(M, 4));
    M = fmaxf(M, shfl_xor(M, 8));
    M = fmaxf(M, shfl_xor(M, 16));
    M = pair32_max(M);
    const float sink2 = sinks ? sinks[row % H] * kLog2e : -INFINITY;
    const float Mall = fmaxf(M, sink2);

    fvec acc;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    float Z = 0.f;
    if (M != -INFINITY) {
        for (int c0 = 0; c0 < ns; c0 += 64) {
            const int cn = min(64, ns - c0);
            const float w = c0 + lane < ns ? fast_exp2(lrow[c0 + lane] - M) : 0.f;
            int s = 0;
            for (; s + 4 <= cn; s += 4) {
                fvec v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = part(c0 + s + u);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float ws = readlane_f32(w, s + u);
                    Z += ws;
                    acc += ws * v[u];
                }
            }
            for (; s < cn; ++s) {
                const fvec v = part(c0 + s);
                const float ws = readlane_f32(w, s);
                Z += ws;
                acc += ws * v;
            }
        }
    }
    if (sinks && Mall != -INFINITY) {             // rescale to the common reference
        const float f = M == -INFINITY ? 0.f : fast_exp2(M - Mall);
        acc *= f;
        Z = Z * f + fast_exp2(sink2 - Mall);
        M = Mall;
    }
    const float inv = Z > 0.f ? 1.0f / Z : 0.f;
    __bf16 *dst = o + (size_t)row * DV + PER * lane;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
        u32x4 w4 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                    pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
        *reinterpret_cast<u32x4 *>(dst) = w4;
    }
    if (lse && lane == 0) lse[row] = Z > 0.f ? (M + __log2f(Z)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_decode_bf16_d128(const DecodeArgs &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.k = static_cast<const char *>(a.k_cache);
    p.v = static_cast<const char *>(a.v_cache);
    p.k_scales = a.k_scales;
    p.v_scales = a.v_scales;
    p.n_stiles = (a.S_max + BN - 1) / BN;
    p.seq_lens = a.seq_lens;
    p.block_table = a.block_table;
    p.max_blocks = a.max_blocks;
    p.page_size = a.page_size;
    p.num_pages = a.num_pages;
    p.plan = a.plan;
    p.ws_o = a.ws_o;
    p.ws_lse = a.ws_lse;
    p.B = a.B;
    p.S_max = a.S_max;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.n_hchunk = (p.G + 15) / 16;
    p.split = a.split;
    p.n_split_max = a.n_split_max;
    p.window = a.window;
    p.scale_log2 = a.scale * kLog2e;
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, a.seq_lens, a.B, a.S_max,
                       a.split, a.hkv * p.n_hchunk, a.plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        const void *fns[4] = {(const void *)decode_bf16_d128_kernel<false, false>,
                              (const void *)decode_bf16_d128_kernel<true, false>,
                              (const void *)decode_bf16_d128_kernel<false, true>,
                              (const void *)decode_bf16_d128_kernel<true, true>};
        const int which = (a.k_scales ? 2 : 0) + (a.block_table ? 1 : 0);
        e = ensure_dynamic_lds(fns[which], a.k_scales ? Layout<true>::lds : Layout<false>::lds);
        if (e != hipSuccess) return e;
    }
    // persistent grid: one workgroup per CU (its LDS takes most of the CU),
    // never more workgroups than the largest possible number of units needs
    const long long max_units = (long long)a.B * a.hkv * p.n_hchunk * a.n_split_max;
    const int nw = a.k_scales ? Layout<true>::nw : Layout<false>::nw;
    long long blocks = (max_units + nw - 1) / nw;
    if (blocks > a.num_cus) blocks = a.num_cus;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(64 * nw);
    if (a.k_scales) {
        if (a.block_table)
            hipLaunchKernelGGL((decode_bf16_d128_kernel<true, true>), grid, block, Layout<true>::lds, stream, p);
        else
            hipLaunchKernelGGL((decode_bf16_d128_kernel<false, true>), grid, block, Layout<true>::lds, stream, p);
    } else {
        if (a.block_table)
            hipLaunchKernelGGL((decode_bf16_d128_kernel<true, false>), grid, block, Layout<false>::lds, stream, p);
        else
            hipLaunchKernelGGL((decode_bf16_d128_kernel<false, false>), grid, block, Layout<false>::lds, stream, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_combine(a.ws_o, a.ws_lse, a.seq_lens, a.o, a.lse, a.B, a.hq, D, a.S_max,
                                a.split, a.n_split_max, a.sinks, stream);
}

hipError_t launch_split_combine(const void *ws_o, const float *ws_lse, const int32_t *seq_lens,
                                void *o, float *lse, int B, int H, int dv, int S_max, int split,
                                int n_split_max, const float *sinks, hipStream_t stream,
                                bool partial_bf16) {
    const long long n_rows = (long long)B * H;
    if (n_rows > 0x7fffffffLL - 4) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((n_rows + 3) / 4));
    __bf16 *ob = static_cast<__bf16 *>(o);
    if (dv == 128 && !partial_bf16)
        hipLaunchKernelGGL((split_combine_kernel<128, false>), grid, dim3(256), 0, stream, ws_o, ws_lse,
                           seq_lens, ob, lse, (int)n_rows, H, S_max, split, n_split_max, sinks);
    else if (dv == 512 && partial_bf16)
        hipLaunchKernelGGL((split_combine_kernel<512, true>), grid, dim3(256), 0, stream, ws_o, ws_lse,
                           seq_lens, ob, lse, (int)n_rows, H, S_max, split, n_split_max, sinks);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mi355
