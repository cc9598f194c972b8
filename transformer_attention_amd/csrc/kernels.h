// kernels.h -- host-side launchers of the gfx950 attention kernels (internal
// to libmi355attn.so; the public ABI is include/mi355attn.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mi355 {

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (device, kernel) in the process; safe to call from several threads.
// The limit belongs to the function on each device, so a process that
// launches on several GPUs sets it on every one of them.
hipError_t ensure_dynamic_lds(const void *kernel, int bytes);

struct PrefillArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, T, hq, hkv, d;
    int causal, window;
    float scale;
    const float *sinks;   // [hq] sink logits or nullptr
};

// bf16, d = 128, bf16 MFMA.  Returns hipSuccess or the launch error.
hipError_t launch_prefill_bf16_d128(const PrefillArgs &a, hipStream_t stream);
// fp32, d in {16, 32, 64, 128}, fp32 FMA.
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t stream);

// Prefill with FP8 attention, d = 128: q, k, v as E4M3 codes ([B, hq, T, d]
// and [B, hkv, T, d]) with one fp32 scale per 32 positions of a head
// ([B, h, ceil(T / 32)]); o bf16, lse fp32 (may be null).
struct PrefillFp8Args {
    const void *q, *k, *v;
    const float *q_scales, *k_scales, *v_scales;
    void *o;
    float *lse;
    int B, T, hq, hkv;
    int causal, window;
    float scale;
    const float *sinks;
};
hipError_t launch_prefill_fp8_d128(const PrefillFp8Args &a, hipStream_t stream);

struct PrefillBwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    int B, T, hq, hkv, d;
    int causal, window;
    float scale;
    float *ws_stats;      // [B * hq, Tpad, 2]: lse * log2(e) (+inf on pad rows), dout . o
    int Tpad;             // T rounded up to a multiple of 64
    const float *sinks;   // [hq] sink logits or nullptr
    float *dsinks;        // [hq] their gradient (written when non-null; needs sinks)
};
// bf16, d = 128: a row-statistics pass, then dK/dV (key-block parallel)
// and dQ (query-block parallel).
hipError_t launch_prefill_bwd_bf16_d128(const PrefillBwdArgs &a, hipStream_t stream);

struct DecodeArgs {
    const void *q, *k_cache, *v_cache;
    void *o;
    float *lse;
    const int32_t *seq_lens;
    int B, S_max, hq, hkv, d;
    int window;
    float scale;
    int split;            // keys per work item (multiple of 64)
    int n_split_max;      // ceil(S_max / split)
    float *ws_o;          // [B, hq, n_split_max, d]
    float *ws_lse;        // [B, hq, n_split_max]  (log2 units)
    int32_t *plan;        // [B + 1] unit prefix sums (workspace)
    int num_cus;          // compute units of the device (persistent grid size)
    // paged cache (block_table == nullptr: contiguous [B, hkv, S_max, d]):
    // k_cache / v_cache are [num_pages, hkv, page_size, d], S_max =
    // max_blocks * page_size
    const int32_t *block_table;
    int max_blocks, page_size, num_pages;
    const float *sinks;   // [hq] sink logits or nullptr
    // FP8 (E4M3) cache when non-null: k_cache / v_cache hold one-byte codes
    // and these one scale per 32 positions of a K/V head ([B, hkv,
    // ceil(S_max / 32)] contiguous, [num_pages, hkv, page_size / 32] paged)
    const float *k_scales, *v_scales;
};
hipError_t launch_decode_bf16_d128(const DecodeArgs &a, hipStream_t stream);

struct MlaArgs {
    const void *q, *cache;
    void *o;
    float *lse;
    const int32_t *seq_lens;
    int B, S_max, H, d_c, d_r;
    float scale;
    int split;
    int n_split_max;
    __bf16 *ws_o;         // [B, H, n_split_max, d_c] bf16 (normalised partial outputs)
    float *ws_lse;        // [B, H, n_split_max]  (log2 units)
    // paged cache (block_table == nullptr: contiguous [B, S_max, d_c + d_r]):
    // cache is [num_pages, page_size, d_c + d_r], S_max = max_blocks * page_size
    const int32_t *block_table;
    int max_blocks, page_size, num_pages;
    const float *sinks;   // [H] sink logits or nullptr
};
hipError_t launch_mla_decode_bf16(const MlaArgs &a, hipStream_t stream);

// MLA decode with FP8 attention: the cache as E4M3 codes [B, S_max, d_c + d_r]
// with one fp32 scale per 32 tokens [B, ceil(S_max / 32)]; the bf16 query is
// quantised per head into ws_q8 / ws_qs first.
struct MlaFp8Args {
    const void *q;              // [B, H, d_c + d_r] bf16
    const void *cache;          // codes
    const float *cache_scales;
    void *o;
    float *lse;
    const int32_t *seq_lens;
    int B, S_max, H;
    float scale;
    int split, n_split_max;     // split: a multiple of 64
    __bf16 *ws_o;               // as MlaArgs
    float *ws_lse;
    void *ws_q8;                // [B, H, d_c + d_r] query codes
    float *ws_qs;               // [B, H] query scales
    const float *sinks;
};
hipError_t launch_mla_decode_fp8(const MlaFp8Args &a, hipStream_t stream);

// Rotary position embedding of q [B, hq, T, row_q] and k [B, hk, T, row_k]
// (k may be null with hk = 0), dimensions [rope_offset, rope_offset +
// rope_dim) of each row, in place.
struct RopeArgs {
    void *q, *k;
    const int32_t *positions;   // [B, T] or nullptr (position t)
    int B, T, hq, hk, row_q, row_k, rope_offset, rope_dim;
    float base;
    bool bf16;
};
hipError_t launch_rope_qk(const RopeArgs &a, hipStream_t stream);

// Per-tile FP8 (E4M3) quantisation of a bf16 cache x [B*hkv, S, d]: one
// scale per 32 positions of a head (amax / 448), codes [B*hkv, S, d].
hipError_t launch_quantize_kv_fp8(const void *x, void *codes, float *scales, long long n_heads,
                                  int S, int d, hipStream_t stream);
// Merge of split partials: o[b,h,:] (bf16) and lse[b,h] (natural log, may be
// null) from ws_o/ws_lse over the ceil(len_b / split) splits of sequence b;
// sinks (per head, may be null) adds a sink logit to each merged denominator.
// ws_o holds fp32 partials (GQA decode) or, with partial_bf16, bf16 ones (MLA).
hipError_t launch_split_combine(const void *ws_o, const float *ws_lse,
                                const int32_t *seq_lens, void *o, float *lse,
                                int B, int H, int dv, int S_max, int split,
                                int n_split_max, const float *sinks, hipStream_t stream,
                                bool partial_bf16 = false);

}  // namespace mi355
