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
//  * workgroup = 256 query rows of 1, 2, 4 or 8 heads of one K/V group,
//    as 8 waves of 32 rows (two waves per SIMD, one wave's softmax overlaps
//    the other's MFMAs) or 4 waves of 64 rows (every K/V operand read from
//    LDS feeds two MFMAs, halving LDS traffic per FLOP);
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (A = K rows from LDS, B = the wave's Q rows held in registers).  In the
//    D layout each lane owns ONE query row (its column), so a row's max/sum
//    is a per-lane reduction plus one exchange with lane l^32;
//  * the P.V product is computed as O^T = V^T P^T: the S^T accumulator,
//    rounded to bf16, is directly the B operand (no LDS round trip for P);
//    the V^T A operand is read from the row-major V tile with the
//    transposing LDS load ds_read_b64_tr_b16 (two per operand), whose four
//    source rows are exactly the four keys each lane's P values belong to;
//  * K and V tiles (64 keys) are stored row-major in LDS with padded rows so
//    every LDS address stays base + immediate and no read has bank
//    conflicts: K rows are 304 bytes apart (19 16-byte slots, 19 = 3 mod 16:
//    the 16 consecutive rows of one column that a quarter wave reads hit 16
//    distinct slots), V rows 320 bytes apart (20 = 4 mod 16: the 4 rows x 64
//    bytes that a half wave reads through the transposing load fill the 16
//    slots exactly once);
//  * K/V tiles stream HBM -> LDS through a 4-stage ring filled by
//    global_load_lds_dwordx4 (no staging registers): while a wave computes
//    the scores of tile t+1 and the P.V product of tile t, tiles t+2 and t+3
//    are in flight (one barrier per tile);
//  * each wave is software-pipelined: the score MFMAs of tile t+1 are
//    issued around the probabilities of key block 1 of tile t, and the P.V
//    MFMAs of tile t around the probabilities of key block 0 of tile t+1,
//    so each product carries half of the exponentials and the matrix cores
//    and the vector ALUs of one wave work concurrently;
//  * no row max is taken in steady state: a tile's probabilities are taken
//    against the row's current reference max and accepted when every
//    lane's partial sum of them is at most 2^16 (no probability exceeds
//    2^16, far from overflow).  Otherwise (rare) the tile's scores are
//    recomputed from LDS, the reference max of the rows concerned moves to
//    their true running max, and their l and O are rescaled.  Every
//    exponent is taken against the reference that l and O carry, so the
//    quotient O / l is the same.  A row's first reference max is the row
//    max of its first tile with a visible key;
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
constexpr int ROWB = D * 2 + 48;   // LDS row stride of a K row (304 B = 19 slots)
constexpr int VROWB = D * 2 + 64;  // LDS row stride of a V row (320 B = 20 slots)
constexpr int LDS_BUDGET = 160 * 1024;
constexpr int WG_ROWS = 256;    // query rows x heads per workgroup
// A tile is accepted against the current reference max when every lane's
// partial row sum of its probabilities stays at or below THR (so no single
// probability exceeds 2^16); otherwise the tile's true row max is taken.
constexpr float THR = 65536.0f;

#ifndef PREFILL_NB
#define PREFILL_NB 1
#endif
#ifndef PREFILL_KB
#define PREFILL_KB 2
#endif
#ifndef PREFILL_NSTAGE
#define PREFILL_NSTAGE 4
#endif
#ifndef PREFILL_KPF
#define PREFILL_KPF 2       // k-steps of K operands read ahead of their MFMAs
#endif
#ifndef PREFILL_VPF
#define PREFILL_VPF 3       // V operands read ahead of their MFMAs
#endif

struct Params {
    const __bf16 *q, *k, *v;
    __bf16 *o;
    float *lse;
    int T, hq, hkv, G;
    int hpw;              // query heads per workgroup (1, 2, 4 or 8)
    int rows_per_wg;      // WG_ROWS / hpw
    int n_row_blocks;
    int n_head_groups;    // B * hkv * (G / hpw)
    int causal, window;
    float scale_log2;     // scale * log2(e)
    const float *sinks;   // [hq] sink logits (natural units) or nullptr
};

// byte offset of (row, 16-byte chunk) inside a K tile / a V tile
__device__ __forceinline__ int tile_off(int r, int chunk) { return r * ROWB + (chunk << 4); }
__device__ __forceinline__ int vtile_off(int r, int chunk) { return r * VROWB + (chunk << 4); }

// NB = number of 32-row MFMA blocks per wave (1: 8 waves, 2: 4 waves);
// KB = number of 32-key blocks per tile; NSTAGE = depth of the LDS ring.
template <int NB, int KB, int NSTAGE>
__global__ __launch_bounds__(64 * (8 / NB), 1) void prefill_bf16_d128_kernel(Params p) {
    constexpr int NW = 8 / NB;      // waves per workgroup
    constexpr int RW = 32 * NB;     // query rows per wave
    constexpr int BN = 32 * KB;     // keys per tile
    constexpr int KTILE_BYTES = BN * ROWB;
    constexpr int STAGE_BYTES = (BN * (ROWB + VROWB) + 1023) / 1024 * 1024;   // K rows, V rows
    constexpr int AHEAD = NSTAGE - 1;                                  // tiles issued ahead
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int q16 = lane >> 4;      // 16-lane group (for the transposing reads)
    const int j16 = lane & 15;

    const int T = p.T;
    const int subs = p.G / p.hpw;
    const int wph = NW / p.hpw;                       // waves per head (hpw <= NW)

    // Work items: (row block, head group) pairs numbered heaviest row block
    // first with the head group fastest.  The grid is persistent: workgroup
    // w takes items w, w + grid, ... of rounds 0, 1, ...; odd rounds run the
    // round's items in reverse order within each residue class mod 8, so
    // every workgroup's total (causal) work is about the same and all items
    // of a workgroup keep its residue class of head groups (with 8 head
    // groups: one K/V head, on the workgroup's XCD and its L2).
    const int n_items = p.n_row_blocks * p.n_head_groups;
    const int grid = gridDim.x;
    auto item_id = [&](int k) {
        int id = k * grid + blockIdx.x;
        if ((k & 1) && grid % 8 == 0) id = k * grid + grid - 8 - 8 * (blockIdx.x / 8) + blockIdx.x % 8;
        return id < n_items ? id : -1;
    };
    // Key tile range of item id and the offset of its K/V head.
    auto item_tiles = [&](int id, int &tb, int &te, size_t &kvb) {
        const int rb = p.n_row_blocks - 1 - id / p.n_head_groups;
        const int hg = id % p.n_head_groups;
        const int g = (hg / subs) % p.hkv;
        const int b = hg / (subs * p.hkv);
        const int r0 = rb * p.rows_per_wg;
        const int kend = p.causal ? min(T, r0 + p.rows_per_wg) : T;
        const int kbeg = p.window > 0 ? max(0, r0 - p.window + 1) : 0;
        tb = kbeg / BN;
        te = (kend + BN - 1) / BN;
        kvb = ((size_t)b * p.hkv + g) * (size_t)T * D;
    };

    // The current item, as seen by this wave.
    int b = 0, h = 0, rw0 = 0, t_begin = 0, t_end = 0, kend_w = 0, kbeg_w = 0;
    bool wave_active = false;
    size_t q_base = 0;
    int row0 = 0;                                     // this lane's rows: row0 + 32 nb
    auto set_item = [&](int id) {
        const int rb = p.n_row_blocks - 1 - id / p.n_head_groups;
        const int hg = id % p.n_head_groups;
        const int sub = hg % subs;
        const int g = (hg / subs) % p.hkv;
        b = hg / (subs * p.hkv);
        h = g * p.G + sub * p.hpw + wave / wph;
        rw0 = rb * p.rows_per_wg + (wave % wph) * RW;
        size_t kvb;
        item_tiles(id, t_begin, t_end, kvb);
        wave_active = rw0 < T;
        kend_w = p.causal ? min(T, rw0 + RW) : T;
        kbeg_w = p.window > 0 ? max(0, rw0 - p.window + 1) : 0;
        q_base = ((size_t)b * p.hq + h) * (size_t)T * D;
        row0 = rw0 + l32;
    };
    auto tile_active = [&](int t) {
        const int ts = t * BN;
        return wave_active && t < t_end && ts < kend_w && ts + BN > kbeg_w;
    };
    auto tile_needs_mask = [&](int t) {
        const int ts = t * BN;
        return (ts + BN > T) || (p.causal && ts + BN - 1 > rw0) ||
               (p.window > 0 && (rw0 + RW - 1) - ts >= p.window);
    };

    const float c = p.scale_log2;

    // Q^T B operands: row = row0 + 32nb, d = 16ks + 8hi .. +7
    bf16x8 qop[NB][8];
    auto load_q = [&]() {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int row = row0 + 32 * nb;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (row < T) val = ldg16(p.q + q_base + (size_t)row * D + 16 * ks + 8 * hi);
                qop[nb][ks] = __builtin_bit_cast(bf16x8, val);
            }
    };

    f32x16 oacc[NB][4];
    float m_run[NB], l_run[NB];
    auto reset_rows = [&]() {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[nb][db][i] = 0.f;
            m_run[nb] = -INFINITY;                    // reference max (log2 units)
            l_run[nb] = 0.f;                          // lane-partial row sum
        }
    };

    // LDS ring of NSTAGE stages, each holding the K and V rows of one tile.
    // Tiles take the stages in the order they are copied, across items: the
    // current item's first tile is number seq_f, its tile t lives in stage
    // (seq_f + t - t_begin) % NSTAGE; at iteration t the stages hold tile t
    // (V in use), t+1 (K in use) and the next two tiles of the sequence (in
    // flight), which near an item's end are the next item's first tiles.
    int seq_f = 0;
    auto kbuf = [&](int rel) { return smem + ((seq_f + rel) % NSTAGE) * STAGE_BYTES; };
    auto vbuf = [&](int rel) { return smem + ((seq_f + rel) % NSTAGE) * STAGE_BYTES + KTILE_BYTES; };
    // DMA of one tile: one-KB blocks (K rows, then V rows), split over the waves.
    // LDS byte o of a region holds row o / stride, chunk (o % stride) / 16;
    // pad slots receive an arbitrary valid chunk; rows past T re-read row T-1
    // (their scores are masked, their P is 0).
    constexpr int NBLK = STAGE_BYTES / 1024;
    constexpr int PER_WAVE = (NBLK + NW - 1) / NW;
    // Every wave issues exactly PER_WAVE one-KB copies per tile (the last
    // wave repeats its final block where the stage has fewer blocks: the
    // repeat writes the same bytes to the same place), so the wait counts
    // below are compile-time constants.  Per block: the byte offset inside
    // the tile's K (or V) rows, computed once; the tile's base address is
    // wave-uniform and goes in SGPRs.
    uint32_t dma_off[PER_WAVE];
    int dma_row[PER_WAVE];
    bool dma_is_v[PER_WAVE];
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int blk = min(PER_WAVE * wave + i, NBLK - 1);
        const int o = blk * 1024 + lane * 16;
        dma_is_v[i] = blk * 1024 >= KTILE_BYTES;      // wave-uniform (a block never straddles)
        const int ro = dma_is_v[i] ? o - KTILE_BYTES : o;
        const int stride = dma_is_v[i] ? VROWB : ROWB;
        const int r = min(ro / stride, BN - 1);
        const int ch = min((ro - r * stride) >> 4, D / 8 - 1);
        dma_row[i] = r;
        dma_off[i] = (uint32_t)(r * D * 2 + ch * 16);
    }
    const uint32_t smem_lds = lds_offset(smem);
    // The copy stream: the next tile to copy is tile dma_t of item dma_id
    // (-1 once every item's tiles are issued), sequence number dma_seq.
    int dma_k = 0, dma_id = item_id(0), dma_t = 0, dma_te = 0, dma_seq = 0;
    size_t dma_kv = 0;
    if (dma_id >= 0) item_tiles(dma_id, dma_t, dma_te, dma_kv);
    auto issue_next = [&]() {
        if (dma_id < 0) return;
        const uint32_t stage = smem_lds + (dma_seq % NSTAGE) * STAGE_BYTES;
        const int ts = dma_t * BN;
        const __bf16 *kb0 = p.k + dma_kv + (size_t)ts * D;
        const __bf16 *vb0 = p.v + dma_kv + (size_t)ts * D;
        if (ts + BN <= T) {
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i)
                dma16_off_at(dma_is_v[i] ? vb0 : kb0, dma_off[i],
                             stage + min(PER_WAVE * wave + i, NBLK - 1) * 1024);
        } else {                                      // ragged last tile: rows past T re-read row T-1
            const int last = T - 1 - ts;
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) {
                const uint32_t off = dma_row[i] > last
                    ? dma_off[i] - (uint32_t)((dma_row[i] - last) * D * 2) : dma_off[i];
                dma16_off_at(dma_is_v[i] ? vb0 : kb0, off, stage + min(PER_WAVE * wave + i, NBLK - 1) * 1024);
            }
        }
        ++dma_seq;
        if (++dma_t == dma_te) {
            dma_id = item_id(++dma_k);
            if (dma_id >= 0) item_tiles(dma_id, dma_t, dma_te, dma_kv);
        }
    };
    static_assert(AHEAD <= 4, "wait counts below assume at most 4 tiles in flight");
    auto wait_tiles = [&](int newer) {       // all but the `newer` most recent tiles landed
        if (newer >= 3) wait_vmcnt<3 * PER_WAVE>();
        else if (newer == 2) wait_vmcnt<2 * PER_WAVE>();
        else if (newer == 1) wait_vmcnt<PER_WAVE>();
        else wait_vmcnt<0>();
    };

    // S^T = K Q^T for one tile: s[nb][kb] holds keys 32kb + 8(i/4) + 4hi + (i%4)
    // of row row0 + 32nb.
    // With 64 rows per wave the output accumulators fill the AGPRs and the
    // score MFMAs go through asm with VGPR accumulators (see mfma_s_first).
    constexpr bool ASM_S = NB >= 2;
    auto smfma = [&](int ks, int kb, int nb, bf16x8 a, f32x16 &acc) {
        if constexpr (ASM_S) {
            if (ks == 0) acc = mfma_s_first(a, qop[nb][0]);
            else if (ks == 7 && kb == KB - 1 && nb == NB - 1) acc = mfma_s_last(a, qop[nb][7], acc);
            else acc = mfma_s_acc(a, qop[nb][ks], acc);
        } else {
            if (ks == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = 0.f;
            }
            acc = mfma32x32x16(a, qop[nb][ks], acc);
        }
    };
    auto qk = [&](const char *kt, f32x16 (&s)[NB][KB]) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kt + tile_off(32 * kb + l32, 2 * ks + hi));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) smfma(ks, kb, nb, a, s[nb][kb]);
            }
        if constexpr (ASM_S) __builtin_amdgcn_sched_barrier(0);
    };
    // Mask tile t in place (raw scores -> -inf where the key is not visible).
    // Element (kb, i) is key ts + 4hi + e with e = 32kb + 8(i/4) + (i%4).
    // The visible keys of a row form one range of e, [lo, lo + width): below
    // T, at or before the row (causal), within the window; one unsigned
    // compare per element tests it.
    auto apply_mask = [&](int t, f32x16 (&s)[NB][KB]) {
        const int base = t * BN + 4 * hi;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int diff = row0 + 32 * nb - base;
            int e_hi = min(T - base, BN);
            if (p.causal) e_hi = min(e_hi, diff + 1);
            const int lo = p.window > 0 ? min(max(diff - p.window + 1, 0), BN) : 0;
            const uint32_t width = (uint32_t)max(e_hi - lo, 0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * kb + 8 * (i >> 2) + (i & 3);
                    s[nb][kb][i] = (uint32_t)(e - lo) < width ? s[nb][kb][i] : -INFINITY;
                }
        }
    };
    // Row max of a (masked) tile in log2 units; scale > 0 so max(c s) = c max(s).
    auto tile_max = [&](const f32x16 (&s)[KB]) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        return pair32_max(mx) * c;
    };
    // V^T operand for (db, kb, half): two transposing reads of rows
    // 32kb + 16half + 4hi + (j16>>2) (+8), d = 32db + 16(q16&1) + 4(j16&3) .. +3.
    const int v_row_lane = 4 * hi + (j16 >> 2);
    const int v_chunk_lane = 2 * (q16 & 1) + ((j16 & 3) >> 1);
    const int v_byte_lane = 8 * (j16 & 1);
    auto v_operand = [&](const char *vt, int db, int kb, int half) {
        const int rA = 32 * kb + 16 * half + v_row_lane;
        const int ch = 4 * db + v_chunk_lane;
        const bf16x4 lo4 = lds_read_tr16(vt + vtile_off(rA, ch) + v_byte_lane);
        const bf16x4 hi4 = lds_read_tr16(vt + vtile_off(rA + 8, ch) + v_byte_lane);
        return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // Probabilities of scores 8h .. 8h+7 of a key block against the reference
    // max m_use -> one bf16x8 B operand (keys 8(h/2)+4hi.. of the two row
    // groups of that half); adds them to lsum.  The row sum adds the fp32
    // probabilities with plain adds: v_dot2 (which could add the bf16 ones
    // two at a time) waits for the matrix pipe, and with the other wave of
    // the SIMD issuing MFMAs it takes about four times as long.
    auto probs8 = [&](const f32x16 &s, int h, float m_use, float &lsum, bf16x8 &pp) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(__builtin_fmaf(s[8 * h + i], c, -m_use));
        pp = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        lsum += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    };
    // Exponents are taken against 0 while a row has seen no visible key.
    auto m_ref = [](float m) { return m == -INFINITY ? 0.f : m; };
    // Keep a value computed where it is written: the IR optimisers would
    // otherwise sink the probabilities of one product into the next.
    auto pin = [](bf16x8 &x) { asm volatile("" : "+v"(x)); };

    // The probabilities of key block 0 of the next tile (and their lane-partial
    // sum) are computed one product ahead: during the P.V MFMAs of the
    // current tile.  Key block 1 follows during the next score MFMAs.
    static_assert(KB == 2, "the probability schedule splits a tile into two 32-key blocks");
    bf16x8 pc[NB][2];
    float lc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) lc[nb] = 0.f;
    // A row's reference max is first set to the row max of the first tile in
    // which it has a visible key, before any of that tile's probabilities
    // are taken.  rows_started turns true (wave-uniform) once every row of
    // the wave below T has one, and the row max is not taken after that.
    bool rows_started = false;
    auto start_rows = [&](const f32x16 (&s)[NB][KB]) {
        bool done = true;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float mx = tile_max(s[nb]);
            if (m_run[nb] == -INFINITY) m_run[nb] = mx;
            done = done && (m_run[nb] != -INFINITY || row0 + 32 * nb >= T);
        }
        rows_started = __all(done);
    };
    // Probabilities of key block 0 of a tile, one product ahead.
    auto probs_block0 = [&](const f32x16 (&s)[NB][KB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            lc[nb] = 0.f;
            probs8(s[nb][0], 0, m_ref(m_run[nb]), lc[nb], pc[nb][0]);
            probs8(s[nb][0], 1, m_ref(m_run[nb]), lc[nb], pc[nb][1]);
        }
    };

    f32x16 sa[NB][KB], sb[NB][KB];

    // Some row of tile t overflowed the threshold: recompute the tile's scores from the K rows still in its stage
    // (bit for bit the same scores), move those rows' reference max to their
    // true running max, rescale their l and O, and recompute the tile's
    // probabilities.  Rows that did not ask keep their reference max, so
    // their probabilities come out unchanged and every row's result depends
    // on its own scores only.
    auto rescale_tile = [&](int t, const bool (&redo)[NB], float (&m_use)[NB], float (&lsum)[NB],
                            bf16x8 (&pop)[NB][KB][2]) {
        f32x16 sr[NB][KB];
        qk(kbuf(t - t_begin), sr);
        if (tile_needs_mask(t)) apply_mask(t, sr);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const bool row_redo = pair32_max(redo[nb] ? 1.0f : 0.0f) > 0.f;   // either lane of the row
            const float m_new = row_redo ? fmaxf(m_run[nb], tile_max(sr[nb])) : m_run[nb];
            const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run[nb] - m_new);
            l_run[nb] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                if constexpr (ASM_S) scale_acc(oacc[nb][db], alpha);
                else oacc[nb][db] *= alpha;
            }
            m_run[nb] = m_new;
            m_use[nb] = m_ref(m_new);
            lsum[nb] = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                probs8(sr[nb][kb], 0, m_use[nb], lsum[nb], pop[nb][kb][0]);
                probs8(sr[nb][kb], 1, m_use[nb], lsum[nb], pop[nb][kb][1]);
            }
        }
    };

    // One iteration: softmax + P.V of tile t (scores in s_cur), scores of
    // tile t+1 into s_nxt.
    auto iteration = [&](int t, f32x16 (&s_cur)[NB][KB], f32x16 (&s_nxt)[NB][KB]) {
        const int rel = t - t_begin;
        wait_tiles(min(AHEAD - 2, dma_seq - (seq_f + rel) - 2));   // tile t+1 landed
        raw_barrier();                                // iteration t-1 done everywhere
        // the copy of the tile AHEAD places on in the sequence (into the stage
        // of tile t-1) is issued between the first score MFMAs when this wave
        // has a tile to compute

        const bool act_c = tile_active(t);
        const bool act_n = tile_active(t + 1);
        const char *kn = kbuf(rel + 1);
        const char *vc = vbuf(rel);

        if (act_c) {
            // Key block 0 of tile t was done one product ahead; block 1 runs
            // between the score MFMAs of tile t+1 (when t+1 is not this
            // wave's, its scores are computed from whatever its stage holds
            // and dropped: s_nxt and the probabilities made from it are not
            // used).
            float m_use[NB], lsum[NB];
            bf16x8 pop[NB][KB][2];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                m_use[nb] = m_ref(m_run[nb]);
                lsum[nb] = lc[nb];
                pop[nb][0][0] = pc[nb][0];
                pop[nb][0][1] = pc[nb][1];
            }
            // K operands are loaded KPF k-steps ahead of their MFMAs
            constexpr int KPF = PREFILL_KPF;
            bf16x8 ka[KPF + 1][KB];
#pragma unroll
            for (int i = 0; i < KPF; ++i)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    ka[i][kb] = *reinterpret_cast<const bf16x8 *>(kn + tile_off(32 * kb + l32, 2 * i + hi));
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks + KPF < 8) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        ka[(ks + KPF) % (KPF + 1)][kb] =
                            *reinterpret_cast<const bf16x8 *>(kn + tile_off(32 * kb + l32, 2 * (ks + KPF) + hi));
                }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) smfma(ks, kb, nb, ka[ks % (KPF + 1)][kb], s_nxt[nb][kb]);
                if (ks == 1) issue_next();
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (ks == 1) { probs8(s_cur[nb][1], 0, m_use[nb], lsum[nb], pop[nb][1][0]); pin(pop[nb][1][0]); }
                    if (ks == 4) { probs8(s_cur[nb][1], 1, m_use[nb], lsum[nb], pop[nb][1][1]); pin(pop[nb][1][1]); }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // Accept tile t unless a lane's partial sum passed the threshold
            // (or is not a number).
            bool redo[NB], any_redo = false;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                redo[nb] = !(lsum[nb] <= THR);
                any_redo = any_redo || redo[nb];
            }
            if (__any(any_redo)) rescale_tile(t, redo, m_use, lsum, pop);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) l_run[nb] += lsum[nb];
            if (act_n && tile_needs_mask(t + 1)) apply_mask(t + 1, s_nxt);
            if (!rows_started && act_n) {
                start_rows(s_nxt);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) m_use[nb] = m_ref(m_run[nb]);
            }
            // P.V of tile t; key block 0 of tile t+1 is exponentiated under it
            // V operands are loaded VPF MFMA steps ahead
            constexpr int NV = KB * 2 * 4;            // (kb, half, db) steps
            constexpr int VPF = PREFILL_VPF;
            bf16x8 va[VPF + 1];
            auto vop = [&](int j) { return v_operand(vc, j & 3, j >> 3, (j >> 2) & 1); };
#pragma unroll
            for (int i = 0; i < VPF; ++i) va[i] = vop(i);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (j + VPF < NV) va[(j + VPF) % (VPF + 1)] = vop(j + VPF);
                const int db = j & 3, kb = j >> 3, half = (j >> 2) & 1;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if constexpr (ASM_S) mfma_o_acc(va[j % (VPF + 1)], pop[nb][kb][half], oacc[nb][db]);
                    else oacc[nb][db] = mfma32x32x16(va[j % (VPF + 1)], pop[nb][kb][half], oacc[nb][db]);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (j == 2) { lc[nb] = 0.f; probs8(s_nxt[nb][0], 0, m_use[nb], lc[nb], pc[nb][0]); pin(pc[nb][0]); }
                    if (j == 8) { probs8(s_nxt[nb][0], 1, m_use[nb], lc[nb], pc[nb][1]); pin(pc[nb][1]); }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            issue_next();
            if (act_n) {                              // first tile of this wave
                qk(kn, s_nxt);
                if (tile_needs_mask(t + 1)) apply_mask(t + 1, s_nxt);
                start_rows(s_nxt);
                probs_block0(s_nxt);
            }
        }
    };

    char *epi_buf = smem;
    static_assert(NB != 1 || 8 * 32 * 144 <= STAGE_BYTES, "epilogue staging exceeds a stage");
    auto epilogue = [&]() {
    if constexpr (ASM_S) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int db = 0; db < 4; ++db) settle_acc(oacc[nb][db]);
    }
    // Epilogue: O = O~ / l, L = m ln2 + ln l.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int row = row0 + 32 * nb;
        const float lt = pair32_sum(l_run[nb]);
        if (NB != 1 && row >= T) continue;
        float inv = lt > 0.f ? 1.0f / lt : 0.f;
        float lse_sink = 0.f;
        if (p.sinks) inv = finish_row_with_sink(m_run[nb], lt, p.sinks[h] * kLog2e, lse_sink);
        if constexpr (NB == 1) {
            // Through LDS, so that the stores are whole 128-byte row halves:
            // each lane holds four-value pieces of its row, which scattered
            // 8-byte stores write one 16-byte piece per row at a time.  The
            // wave's 32 rows x 64 values of one half go to its own region of
            // the item's last stage (rows 144 bytes apart: the 8-byte writes of
            // a quarter wave hit distinct banks), then come back as 16 bytes
            // of 8 consecutive values per lane, 8 lanes per row half.
            char *reg = epi_buf + wave * (32 * 144);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
                for (int db = 2 * half; db < 2 * half + 2; ++db)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int d = 32 * db + 8 * q4 + 4 * hi - 64 * half;
                        u32x2 w = {pack_bf16x2(oacc[nb][db][4 * q4 + 0] * inv, oacc[nb][db][4 * q4 + 1] * inv),
                                   pack_bf16x2(oacc[nb][db][4 * q4 + 2] * inv, oacc[nb][db][4 * q4 + 3] * inv)};
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
        } else {
            __bf16 *orow = p.o + q_base + (size_t)row * D;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d = 32 * db + 8 * q4 + 4 * hi;
                    u32x2 w = {pack_bf16x2(oacc[nb][db][4 * q4 + 0] * inv, oacc[nb][db][4 * q4 + 1] * inv),
                               pack_bf16x2(oacc[nb][db][4 * q4 + 2] * inv, oacc[nb][db][4 * q4 + 3] * inv)};
                    *reinterpret_cast<u32x2 *>(orow + d) = w;
                }
        }
        if (p.lse && hi == 0 && row < T) {
            const size_t li = ((size_t)b * p.hq + h) * (size_t)T + row;
            p.lse[li] = p.sinks ? lse_sink : (lt > 0.f ? m_run[nb] * kLn2 + __logf(lt) : -INFINITY);
        }
    }
    };

    // ---- the workgroup's items ----
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) issue_next();
    for (int k = 0;; ++k) {
        const int id = item_id(k);
        if (id < 0) break;
        set_item(id);
        load_q();
        reset_rows();
        rows_started = false;
        // Wait for every load, Q and the copies in flight alike: the compiler
        // then knows the Q registers are complete and puts no wait for them
        // inside the loop, where the only outstanding loads are the ring's
        // copies, which it does not track.  (An item's first tiles were
        // copied during the previous item's last tiles.)
        wait_vmcnt<0>();
        raw_barrier();
        if (tile_active(t_begin)) {
            qk(kbuf(0), sa);
            if (tile_needs_mask(t_begin)) apply_mask(t_begin, sa);
            start_rows(sa);
            probs_block0(sa);
        }
        int t = t_begin;
        for (; t + 1 < t_end; t += 2) {
            iteration(t, sa, sb);
            iteration(t + 1, sb, sa);
        }
        if (t < t_end) iteration(t, sa, sb);
        // every wave is done with the item's last stage, which no copy in
        // flight targets: the epilogue stages its output there
        raw_barrier();
        epi_buf = smem + ((seq_f + t_end - t_begin - 1) % NSTAGE) * STAGE_BYTES;
        if (wave_active) epilogue();
        seq_f += t_end - t_begin;
    }
}


}  // namespace

hipError_t launch_prefill_bf16_d128(const PrefillArgs &a, hipStream_t stream) {
    constexpr int NB = PREFILL_NB, KB = PREFILL_KB, NST = PREFILL_NSTAGE;
    constexpr int NW = 8 / NB;
    constexpr int LDS_BYTES = NST * ((32 * KB * (ROWB + VROWB) + 1023) / 1024 * 1024);
    static_assert(LDS_BYTES <= LDS_BUDGET, "LDS ring too large");
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
    const int hmax = NW;                      // at most one head per wave
    p.hpw = (p.G % 8 == 0 && hmax >= 8) ? 8 : (p.G % 4 == 0) ? 4 : (p.G % 2 == 0 ? 2 : 1);
    p.rows_per_wg = WG_ROWS / p.hpw;
    p.n_row_blocks = (a.T + p.rows_per_wg - 1) / p.rows_per_wg;
    p.n_head_groups = a.B * a.hkv * (p.G / p.hpw);
    p.causal = a.causal;
    p.window = a.window;
    p.scale_log2 = a.scale * kLog2e;
    p.sinks = a.sinks;
    hipError_t e = ensure_dynamic_lds((const void *)prefill_bf16_d128_kernel<NB, KB, NST>, LDS_BYTES);
    if (e != hipSuccess) return e;
    const long long n_items = (long long)p.n_row_blocks * p.n_head_groups;
    if (n_items <= 0) return hipSuccess;
    // One persistent workgroup per compute unit (the LDS ring admits one).
    int dev = 0, n_cu = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const long long grid = n_items < n_cu ? n_items : (long long)n_cu;
    hipLaunchKernelGGL((prefill_bf16_d128_kernel<NB, KB, NST>), dim3((unsigned)grid), dim3(64 * NW),
                       LDS_BYTES, stream, p);
    return hipGetLastError();
}

}  // namespace mi355
