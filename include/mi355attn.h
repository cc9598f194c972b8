/*
 * mi355attn.h -- C ABI of libmi355attn.so: exact scaled-dot-product attention
 * with grouped K/V heads on AMD Instinct MI355X (gfx950).
 *
 * What is computed (for every query head h of a batch entry b):
 *
 *     O[h] = softmax( scale * Q[h] K[g]^T  (+ mask) ) V[g],   g = h / (h_q / h_kv)
 *
 * the grouped-query form in "Attention Engineering: From MHA to GQA, MLA &
 * FlashAttention", section 2 (equation "Grouped-Query Attention
 * Formulation"), with consecutive query heads sharing one K/V head ("2.4
 * Multi-Head Attention, MQA, GQA & MLA", "Implementing the MHA -> GQA
 * conversion").  h_kv == h_q is MHA, h_kv == 1 is MQA.  The S x S score
 * matrix is never written to memory: the kernels stream K/V tiles and keep
 * the online-softmax state (running max m, running sum l, unnormalised
 * output) in registers, dividing by l once at the end ("Attention
 * Engineering ...", section 4, the FlashAttention-2 recurrence).
 *
 * Conventions shared by every entry point
 *  - All tensors are dense, row-major ("contiguous"), in device memory of the
 *    current HIP device, and owned by the caller.  The library allocates,
 *    frees and synchronises nothing; every call only enqueues work on
 *    `stream` and returns.  A workspace, where one is needed, is caller
 *    memory of at least the size the matching *_workspace_size() returns.
 *  - `scale` multiplies Q.K before masking and softmax (1/sqrt(d_h) for plain
 *    attention; 1/sqrt(d_h + d_R) for MLA); it must be finite and > 0.
 *    Masked keys get weight exactly 0.  Cache positions outside a sequence's
 *    visible range are never read.  Inside a prefill tile, a masked key's
 *    values must be finite (they are multiplied by the weight 0).
 *  - Accumulation (m, l, output, log-sum-exp) is fp32.  For bf16 inputs the
 *    softmax weights are rounded to bf16 as the operand of the P.V product;
 *    outputs are rounded to bf16 (round-to-nearest-even).
 *  - `lse`, where offered, receives the natural-log log-sum-exp of the
 *    scaled, masked score row, L = m + ln(l); it may be NULL.  A row with no
 *    visible key gets O = 0 and L = -inf (the sink logit, where one is
 *    given: see attn_prefill).
 *  - Inputs are checked on the host before anything is launched.  Failures
 *    return a status and enqueue nothing.  ATTN_ERR_HIP reports a launch
 *    error from the HIP runtime (hipGetLastError after the launch).
 *  - Calls on different streams may run concurrently; calls that share a
 *    workspace must be ordered by the caller.
 */
#ifndef MI355ATTN_H
#define MI355ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,   /* null pointer, bad size, h_q % h_kv != 0, window without causal, scale not finite and > 0 */
    ATTN_ERR_UNSUPPORTED = 2,   /* a head size / dtype / head count with no kernel instantiated */
    ATTN_ERR_WORKSPACE = 3,     /* workspace missing or smaller than *_workspace_size() */
    ATTN_ERR_HIP = 4            /* the HIP runtime rejected a launch */
} attn_status_t;

typedef enum {
    ATTN_F32 = 0,               /* IEEE float32 */
    ATTN_BF16 = 1               /* bfloat16 (1-8-7) */
} attn_dtype_t;

/*
 * attn_prefill -- prefill / training forward over a whole sequence.
 *
 *   q   : [B, h_q,  T, d_h]   dtype            (read)
 *   k, v: [B, h_kv, T, d_h]   dtype            (read)
 *   o   : [B, h_q,  T, d_h]   dtype            (written)
 *   lse : [B, h_q,  T]        float32 or NULL  (written)
 *
 * Visibility of key j to query i (queries and keys share positions 0..T-1):
 *   causal != 0 : j <= i                              ("Attention Engineering ...", section 2 listing: upper-triangular -inf mask)
 *   window  > 0 : additionally i - j < window         ("Attention deep dive (MHA -> MQA -> GQA -> FlashAttention)", section 6)
 * window > 0 requires causal != 0.  causal == 0 with window == 0 is full
 * (bidirectional) attention.
 *
 * sinks: NULL, or [h_q] float32 in device memory, one sink logit per query
 * head: an extra term exp(sinks[h]) in every row's softmax denominator that
 * carries no value row, so a row may put weight on "nothing" ("Attention
 * Engineering ...", section 5, failure mode 2: a learnable scalar logit in
 * the denominator).  It is in the units of the scaled scores (natural log):
 *   o_i = sum_j exp(s_ij) v_j / (exp(sinks[h]) + sum_j exp(s_ij)),
 *   lse_i = log(exp(sinks[h]) + sum_j exp(s_ij)).
 * A row with no visible key gets o = 0 and lse = sinks[h] (-inf without a
 * sink).  Every entry point below that takes `sinks` reads it the same way.
 *
 * Supported: dtype ATTN_BF16 with d_h = 128 (MFMA kernel); dtype ATTN_F32
 * with d_h in {16, 32, 64, 128}.  Any B >= 1, T >= 1, h_q a multiple of h_kv.
 */
attn_status_t attn_prefill(const void *q, const void *k, const void *v, void *o,
                           float *lse, int B, int T, int h_q, int h_kv, int d_h,
                           attn_dtype_t dtype, int causal, int window, float scale,
                           const float *sinks, hipStream_t stream);

/*
 * attn_prefill_fp8 -- attn_prefill with FP8 attention: the pages' FP8 recipe
 * ("Flash Attention 3 and Multi-Headed Latent Attention", the FP8 attention
 * section: q, k and v quantised to E4M3 per tile with scale amax / 448,
 * both matrix products on FP8 operands, p quantised before the second,
 * results dequantised by the scales), both products on E4M3 matrix
 * instructions with fp32 accumulation.
 *
 *   q        : [B, h_q,  T, d_h] uint8 E4M3 codes   (read)
 *   k, v     : [B, h_kv, T, d_h] uint8 E4M3 codes   (read)
 *   q_scales : [B, h_q,  ceil(T / 32)] float32      (read)
 *   k_scales, v_scales : [B, h_kv, ceil(T / 32)] float32 (read)
 *              one scale per 32 positions of a head: the layout
 *              attn_quantize_kv_fp8 writes for each of q, k and v
 *   o        : [B, h_q, T, d_h] bf16 (written);  lse : [B, h_q, T] or NULL
 * s_ij = scale * sq_i * sk_j * (q8_i . k8_j).  Each row's probabilities are
 * quantised to E4M3 in 64-key tiles against the row's reference R, with the
 * value scale of their key folded in: e = 448 * 2^(y - R), y = s log2(e) +
 * log2(sv_j); when a tile's max of y exceeds R, R moves to that max plus 5
 * (log2 units), so no weight passes 448.  o = sum_j e_j v8_j / (448 l), l =
 * sum_j 2^(s_ij log2(e) - R) unquantised; lse = (R + log2 l) ln 2.  causal,
 * window, scale and sinks as for attn_prefill; masked keys inside a visited
 * tile must have finite codes (not 0x7f / 0xff).  Supported: d_h = 128.
 */
attn_status_t attn_prefill_fp8(const void *q, const void *k, const void *v,
                               const float *q_scales, const float *k_scales,
                               const float *v_scales, void *o, float *lse,
                               int B, int T, int h_q, int h_kv, int d_h, int causal,
                               int window, float scale, const float *sinks,
                               hipStream_t stream);

/*
 * attn_prefill_backward -- gradients of attn_prefill with respect to q, k, v.
 *
 *   q, o, dout : [B, h_q,  T, d_h]  dtype    (read; o and lse are what
 *   lse        : [B, h_q,  T]       float32   attn_prefill returned for q, k, v)
 *   k, v       : [B, h_kv, T, d_h]  dtype    (read)
 *   dq         : [B, h_q,  T, d_h]  dtype    (written)
 *   dk, dv     : [B, h_kv, T, d_h]  dtype    (written; each K/V head's
 *                gradient sums over the h_q / h_kv query heads that share it)
 *
 * The forward keeps only the per-row log-sum-exp for this pass, and the
 * scores are recomputed from q and k ("Attention Engineering ...", section
 * 4, the text after the FlashAttention-2 recurrence; "Attention, Worked Out
 * by Hand (Part 2)", section 2): on visible keys P_ij = exp(scale q_i.k_j -
 * lse_i).  With dP_ij = dout_i.v_j and D_i = dout_i.o_i:
 *   dS_ij = P_ij (dP_ij - D_i),   dq_i = scale sum_j dS_ij k_j,
 *   dk_j = scale sum_i dS_ij q_i, dv_j = sum_i P_ij dout_i,
 * the derivative of the forward.  causal, window and scale must be the ones
 * the forward used.  Accumulation is fp32; P and dS are rounded to bf16 as
 * MFMA operands and the outputs to bf16 (round-to-nearest-even).  No atomics:
 * the result is bitwise reproducible.
 *
 * sinks, dsinks: for a forward run with sink logits, o and lse already
 * include the sink's denominator term, so the formulas above hold as they
 * stand (the sink has no value row).  When dsinks ([h_q] float32, device) is
 * not NULL, the sinks' gradient is written there:
 *   dsinks[h] = -sum over b, i of exp(sinks[h] - lse_i) D_i,
 * summed in a fixed order.  dsinks without sinks is ATTN_ERR_INVALID_ARG;
 * sinks alone is read for nothing.
 *
 * workspace: caller device memory of at least
 * attn_prefill_backward_workspace_size(B, T, h_q) bytes (per-row lse in log2
 * units and D, rows padded to a multiple of 64); it is overwritten.
 * Supported: dtype ATTN_BF16 with d_h = 128 (ATTN_ERR_UNSUPPORTED otherwise).
 * Returns 0 from the size function for invalid sizes.
 */
size_t attn_prefill_backward_workspace_size(int B, int T, int h_q);
attn_status_t attn_prefill_backward(const void *q, const void *k, const void *v,
                                    const void *o, const void *dout, const float *lse,
                                    void *dq, void *dk, void *dv,
                                    int B, int T, int h_q, int h_kv, int d_h,
                                    attn_dtype_t dtype, int causal, int window, float scale,
                                    const float *sinks, float *dsinks,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * attn_decode -- one new query token per sequence against a bf16 KV cache
 * ("Attention deep dive ...", section 5 "The KV cache": the new query
 * attends to every cached key, cached + new, so no causal mask applies
 * inside the cache).
 *
 *   q        : [B, h_q, d_h]          bf16   (read; a [B,h_q,1,d_h] tensor has this layout)
 *   k_cache  : [B, h_kv, S_max, d_h]  bf16   (read; only positions < seq_lens[b])
 *   v_cache  : [B, h_kv, S_max, d_h]  bf16   (read; only positions < seq_lens[b])
 *   o        : [B, h_q, d_h]          bf16   (written)
 *   lse      : [B, h_q]               float32 or NULL (written)
 *   seq_lens : [B]                    int32, device memory; the valid cache
 *              length of sequence b, including the current token.  Values are
 *              clamped to [0, S_max]; a zero length gives o = 0, lse = -inf.
 *
 * window > 0 restricts the query (position seq_lens[b]-1) to the last
 * `window` cached keys.  The cache is split into chunks of `split_tokens`
 * positions (0 = the library's choice; otherwise a positive multiple of
 * 64), each chunk is attended to independently and the partial results are
 * merged with their log-sum-exp weights; the split changes only rounding.
 * sinks: NULL or [h_q] sink logits, as for attn_prefill (a sequence with
 * seq_lens[b] = 0 gets o = 0 and lse = sinks[h]).
 * Supported: d_h = 128, any h_q that is a multiple of h_kv.
 */
size_t attn_decode_workspace_size(int B, int S_max, int h_q, int h_kv, int d_h,
                                  int split_tokens);
attn_status_t attn_decode(const void *q, const void *k_cache, const void *v_cache,
                          void *o, float *lse, const int32_t *seq_lens,
                          int B, int S_max, int h_q, int h_kv, int d_h,
                          int window, float scale, const float *sinks, int split_tokens,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * mla_decode -- Multi-head Latent Attention decode with the up-projections
 * absorbed ("Attention Engineering ...", section 3, equations "Associative
 * Weight Absorption Identity" and "Complete MLA Attention Score").
 *
 *   q        : [B, h_q, d_c + d_r]     bf16  (read) per head the absorbed content
 *              query W_UK^T q_C (first d_c) then the rotated RoPE query (last d_r)
 *   kv_cache : [B, S_max, d_c + d_r]   bf16  (read) per token the latent c_KV
 *              (first d_c) then the shared rotated RoPE key k_R (last d_r)
 *   o        : [B, h_q, d_c]           bf16  (written) sum_j softmax_j c_j, the
 *              latent context before the caller applies W_UV
 *   lse      : [B, h_q]                float32 or NULL (written)
 *   seq_lens : [B] int32, device memory, clamped to [0, S_max].
 *
 * score_j = scale * (q[:d_c] . c_j + q[d_c:] . kR_j); the value of token j
 * is the first d_c entries of the same cache row.  split_tokens and sinks
 * as for attn_decode; each chunk's normalised partial output is kept in
 * bf16 in the workspace (mla_decode_workspace_size bytes) before the merge.
 * Supported: d_c = 512, d_r = 64, h_q a multiple of 16.
 */
size_t mla_decode_workspace_size(int B, int S_max, int h_q, int d_c, int d_r,
                                 int split_tokens);
attn_status_t mla_decode(const void *q, const void *kv_cache, void *o, float *lse,
                         const int32_t *seq_lens, int B, int S_max, int h_q,
                         int d_c, int d_r, float scale, const float *sinks,
                         int split_tokens, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Paged KV caches -- the same two decode steps with the cache held in
 * fixed-size pages that a per-sequence block table maps to, the layout of
 * production serving engines ("Attention deep dive ...", section 5 "The KV
 * cache", the production-engine notes: pages remove fragmentation and let
 * sequences of different lengths share memory; "2.4 Multi-Head Attention,
 * MQA, GQA & MLA", GQA in the real libraries: paged blocks sized from the
 * K/V head count).  Only the addressing changes: the result is the
 * contiguous decode's on the gathered cache.
 *
 *   k_pages, v_pages : [num_pages, h_kv, page_size, d_h]  bf16 (read)
 *   kv_pages (MLA)   : [num_pages, page_size, d_c + d_r]   bf16 (read)
 *   block_table      : [B, max_blocks] int32, device memory: position t of
 *                      sequence b is row t % page_size of page
 *                      block_table[b * max_blocks + t / page_size].  Only the
 *                      entries of positions < seq_lens[b] are read; an entry
 *                      outside [0, num_pages) is clamped into it (no fault,
 *                      wrong data).
 *   seq_lens         : as for the contiguous calls, clamped to
 *                      [0, max_blocks * page_size].
 * Everything else (q, o, lse, window, scale, sinks, split_tokens, workspace,
 * errors) is as in attn_decode / mla_decode with S_max = max_blocks *
 * page_size; the *_paged_workspace_size functions return exactly that.
 * page_size must be a positive multiple of 32 (ATTN_ERR_UNSUPPORTED
 * otherwise); a null block_table or non-positive max_blocks, page_size or
 * num_pages is ATTN_ERR_INVALID_ARG.
 */
size_t attn_decode_paged_workspace_size(int B, int max_blocks, int page_size, int h_q,
                                        int h_kv, int d_h, int split_tokens);
attn_status_t attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                                void *o, float *lse, const int32_t *seq_lens,
                                const int32_t *block_table, int B, int max_blocks,
                                int page_size, int num_pages, int h_q, int h_kv, int d_h,
                                int window, float scale, const float *sinks,
                                int split_tokens, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);
size_t mla_decode_paged_workspace_size(int B, int max_blocks, int page_size, int h_q,
                                       int d_c, int d_r, int split_tokens);
attn_status_t mla_decode_paged(const void *q, const void *kv_pages, void *o, float *lse,
                               const int32_t *seq_lens, const int32_t *block_table,
                               int B, int max_blocks, int page_size, int num_pages,
                               int h_q, int d_c, int d_r, float scale, const float *sinks,
                               int split_tokens, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * FP8 KV cache -- the decode steps against a cache quantised to OCP FP8 E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest value 448,
 * no infinities), half the bytes of bf16.  The pages quantise per tile with
 * scale = amax / 448 and cast x / scale to E4M3 ("Flash Attention 3 and
 * Multi-Headed Latent Attention", the FP8 attention section), and name the
 * quantised cache as what production engines keep ("Attention deep dive
 * ...", section 5, production-engine notes; "2.4 Multi-Head Attention, MQA,
 * GQA & MLA": an fp8 cache stacks with GQA).
 *
 * Tile: 32 consecutive positions of one K/V head of one sequence (or page),
 * all d_h values; one fp32 scale per tile, separately for K and for V.  The
 * cached value is code * scale.
 *
 * attn_quantize_kv_fp8 -- writes such a cache from a bf16 one:
 *   x      : [B, h_kv, S, d_h] bf16 (read)
 *   codes  : [B, h_kv, S, d_h] uint8 E4M3 codes (written)
 *   scales : [B, h_kv, ceil(S / 32)] float32 (written)
 * scale = amax / 448 over the tile (1 for an all-zero tile, fp32 division);
 * code = E4M3 nearest to x / scale (fp32 division, ties to even, magnitudes
 * clamped to 448).  Non-finite input: E4M3 has no infinities, so a NaN or
 * +-inf is stored as the NaN code 0x7f (0xff when its sign bit is set) and
 * reads back as NaN; amax runs over the tile's finite values only, so such
 * an entry changes no other code or scale (a tile with no finite nonzero
 * value gets scale 1).  The last tile may hold fewer than 32 positions.  A paged
 * cache [num_pages, h_kv, page_size, d_h] is quantised by passing B =
 * num_pages, S = page_size.  d_h must be a multiple of 8.
 *
 * attn_decode_fp8 / attn_decode_paged_fp8 -- attn_decode / attn_decode_paged
 * with k_cache / v_cache (or the pages) holding codes and k_scales / v_scales
 * their tile scales:
 *   contiguous : [B, h_kv, ceil(S_max / 32)]
 *   paged      : [num_pages, h_kv, page_size / 32]
 * (the layouts attn_quantize_kv_fp8 writes).  The result is attention over
 * the dequantised cache: the codes are widened to bf16 exactly, the K scale
 * multiplies the scores of its tile and the V scale the weights of its
 * tile's values, accumulation as in attn_decode.  Everything else
 * (arguments, workspace, errors) is as in attn_decode / attn_decode_paged;
 * null k_scales or v_scales is ATTN_ERR_INVALID_ARG.  With split_tokens = 0
 * the FP8 calls choose longer chunks than the bf16 ones (never shorter), so
 * attn_decode_workspace_size / attn_decode_paged_workspace_size still cover
 * them.
 */
attn_status_t attn_quantize_kv_fp8(const void *x, void *codes, float *scales,
                                   int B, int h_kv, int S, int d_h, hipStream_t stream);
attn_status_t attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                              const float *k_scales, const float *v_scales,
                              void *o, float *lse, const int32_t *seq_lens,
                              int B, int S_max, int h_q, int h_kv, int d_h,
                              int window, float scale, const float *sinks, int split_tokens,
                              void *workspace, size_t workspace_bytes,
                              hipStream_t stream);
attn_status_t attn_decode_paged_fp8(const void *q, const void *k_pages, const void *v_pages,
                                    const float *k_scales, const float *v_scales,
                                    void *o, float *lse, const int32_t *seq_lens,
                                    const int32_t *block_table, int B, int max_blocks,
                                    int page_size, int num_pages, int h_q, int h_kv, int d_h,
                                    int window, float scale, const float *sinks,
                                    int split_tokens, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * mla_decode_fp8 -- mla_decode with FP8 attention: the pages' FP8 recipe
 * ("Flash Attention 3 and Multi-Headed Latent Attention", the FP8 attention
 * section and its per-tile block processor: q, k, v and p quantised to E4M3
 * with scale amax / 448, both products on FP8 operands, dequantised by the
 * scales) on the absorbed MLA decode.  Both products run on E4M3 matrix
 * instructions with fp32 accumulation.
 *
 *   q         : [B, h_q, d_c + d_r] bf16 (read); quantised inside the call,
 *               one scale per head row (amax / 448, as attn_quantize_kv_fp8
 *               does for a one-row tile)
 *   kv_codes  : [B, S_max, d_c + d_r] uint8 E4M3 codes (read; only tokens
 *               < seq_lens[b])
 *   kv_scales : [B, ceil(S_max / 32)] float32: one scale per 32 tokens, the
 *               layout attn_quantize_kv_fp8 writes for a [B, 1, S_max, d_c +
 *               d_r] cache (h_kv = 1)
 *   o, lse, seq_lens, scale, sinks, split_tokens : as mla_decode
 * s_j = scale * sq * sc_j * (q8 . c8_j).  The probabilities are quantised to
 * E4M3 in 64-token tiles against each chunk's reference R, with the value
 * scale of their token folded in: e_j = 448 * 2^(y_j - R), y_j = s_j log2(e)
 * + log2(sc_j); when a tile's max of y exceeds R, R moves to that max plus 5
 * (log2 units), so no weight passes 448.  The output is sum_j e_j c8_j /
 * (448 l) with the unquantised denominator l = sum_j 2^(s_j log2(e) - R).
 * Chunks (and the sink) merge by their log-sum-exp.  The result differs from
 * mla_decode on the same values by the E4M3 rounding of q, the cache and p.
 * workspace: at least mla_decode_fp8_workspace_size(...) bytes (the split
 * partials plus the query codes and scales).  Supported: d_c = 512, d_r = 64.
 */
size_t mla_decode_fp8_workspace_size(int B, int S_max, int h_q, int d_c, int d_r,
                                     int split_tokens);
attn_status_t mla_decode_fp8(const void *q, const void *kv_codes, const float *kv_scales,
                             void *o, float *lse, const int32_t *seq_lens, int B, int S_max,
                             int h_q, int d_c, int d_r, float scale, const float *sinks,
                             int split_tokens, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * attn_rope_qk -- rotary position embedding of the queries and keys, in
 * place, in one launch ("Attention Engineering ...", section 1: pair j of
 * the rotated dimensions, (x_{2j}, x_{2j+1}), is rotated as a complex number
 * by the angle m theta_j at position m, theta_j = base^(-2j / rope_dim), so
 * that rotated queries and keys interact through their distance only;
 * section 3: MLA rotates only the decoupled RoPE part).
 *
 *   q : [B, h_q, T, row_q]  dtype  (read and written)
 *   k : [B, h_k, T, row_k]  dtype  (read and written; NULL with h_k = 0)
 *   positions : [B, T] int32 device memory, or NULL for positions 0..T-1
 *               (decode: T = 1 and the new token's position per sequence)
 * The rotated dimensions of every row are [rope_offset, rope_offset +
 * rope_dim): rope_offset = 0, rope_dim = d_h for a plain head; 512 and 64
 * for the MLA query row and the cache row's k_R.  The others are left as
 * they are.  The angle and its cosine and sine are computed in double
 * precision, the rotation in fp32, rounded to dtype (bf16: nearest even).
 * rope_dim and rope_offset must be even, base finite and > 0; dtype
 * ATTN_BF16 or ATTN_F32.
 */
attn_status_t attn_rope_qk(void *q, void *k, const int32_t *positions, int B, int T,
                           int h_q, int h_k, int row_q, int row_k, int rope_offset,
                           int rope_dim, float base, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, semantics and results as attn_decode
 * without the workspace: the split partials and the work plan live in a
 * static device array of MI355ATTN_DECODE_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds on every GPU it runs on until the process ends.  The
 * call allocates nothing.
 *
 * Limit: the problem's workspace, attn_decode_workspace_size(B, S_max, h_q,
 * h_kv, d_h, split_tokens), must fit in the array; otherwise the call
 * returns ATTN_ERR_WORKSPACE and launches nothing.  The 70B-shaped decode
 * (B = 64, h_q / h_kv = 64 / 8, d_h = 128, S_max = 32768) needs about 34 MB
 * at the default split; a larger split_tokens shrinks the need.  All calls
 * on one GPU share the array: calls that overlap in time on
 * one GPU (different streams, or different threads without ordering) race
 * and must be ordered by the caller.  Nothing in the array needs to start at
 * zero; each call writes what it reads.
 */
#define MI355ATTN_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
attn_status_t attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  void *o, float *lse, const int32_t *seq_lens,
                                  int B, int S_max, int h_q, int h_kv, int d_h,
                                  int window, float scale, const float *sinks, int split_tokens,
                                  hipStream_t stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char *attn_status_string(attn_status_t status);

/* ABI version of this header (bumped on incompatible change). */
#define MI355ATTN_ABI_VERSION 2
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355ATTN_H */
