// api.hip -- the C ABI of libmi355attn.so (declared in include/mi355attn.h):
// argument validation, workspace sizing and kernel dispatch.  No allocation,
// no synchronisation: every entry point validates on the host, then enqueues
// on the caller's stream and returns.
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <utility>

#include "mi355attn.h"
#include "kernels.h"

namespace mi355 {

hipError_t ensure_dynamic_lds(const void *kernel, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::set<std::pair<int, const void *>> done;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({dev, kernel})) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.insert({dev, kernel});
    return e;
}

}  // namespace mi355

namespace {

// Default split of the cache for decode, in keys (a multiple of the 32-key
// tile).  A split is one unit of work of the persistent decode kernel; the
// bf16 choice aims at about 8 units per wave (4 waves per CU) for full-length
// sequences, which balances the waves while keeping units long.  The FP8
// kernel (6 waves per CU, half the bytes per tile) measured fastest with
// about one unit per wave (70B workload: 0.408 ms at a split of 8192 against
// 0.422 ms at 2048); its split is never smaller than the bf16 one, so the
// bf16 workspace size covers it.
int device_cu_count();
int default_decode_split(int B, int S_max, int hkv, int G, int num_cus, bool fp8 = false) {
    const long long groups = (long long)B * hkv * ((G + 15) / 16);
    const long long target_units = fp8 ? 6LL * num_cus : 8LL * 4 * num_cus;
    long long split = groups * (long long)S_max / target_units;
    int p2 = 256;
    while (p2 < 8192 && p2 < split) p2 *= 2;
    return p2;
}

// MLA: one workgroup per (sequence, 128-head chunk, split); aim at one
// workgroup per CU (256 CUs) for full-length sequences.
int default_mla_split(int B, int S_max, int H) {
    const long long chunks = (long long)B * ((H + 127) / 128);
    long long split = (S_max * chunks + 255) / 256;
    split = (split + 63) / 64 * 64;
    if (split < 64) split = 64;
    if (split > S_max) split = (S_max + 63) / 64 * 64;
    return (int)split;
}

bool bad_ptr(const void *p) { return p == nullptr; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t split_ws_bytes(long long rows, long long n_split, long long dv) {
    return align_up((size_t)(rows * n_split * dv) * sizeof(float), 256) +
           align_up((size_t)(rows * n_split) * sizeof(float), 256);
}
// The MLA decodes keep their normalised partial outputs in bf16.
size_t mla_ws_bytes(long long rows, long long n_split, long long dv) {
    return align_up((size_t)(rows * n_split * dv) * sizeof(uint16_t), 256) +
           align_up((size_t)(rows * n_split) * sizeof(float), 256);
}

// Compute units of the current device (cached per device id).
int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cached[dev] = n;
    return n;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return MI355ATTN_ABI_VERSION; }

const char *attn_status_string(attn_status_t s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID_ARG: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case ATTN_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

attn_status_t attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int T, int h_q, int h_kv, int d_h, attn_dtype_t dtype,
                           int causal, int window, float scale, const float *sinks,
                           hipStream_t stream) {
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(o)) return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0 || h_q <= 0 || h_kv <= 0 || d_h <= 0) return ATTN_ERR_INVALID_ARG;
    if (h_q % h_kv != 0) return ATTN_ERR_INVALID_ARG;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * h_q * T * d_h >= (1LL << 40)) return ATTN_ERR_UNSUPPORTED;
    mi355::PrefillArgs a{q, k, v, o, lse, B, T, h_q, h_kv, d_h, causal ? 1 : 0, window, scale, sinks};
    hipError_t e;
    if (dtype == ATTN_BF16) {
        if (d_h != 128) return ATTN_ERR_UNSUPPORTED;
        e = mi355::launch_prefill_bf16_d128(a, stream);
    } else if (dtype == ATTN_F32) {
        if (d_h != 16 && d_h != 32 && d_h != 64 && d_h != 128) return ATTN_ERR_UNSUPPORTED;
        if (h_q > 65535 || B > 65535) return ATTN_ERR_UNSUPPORTED;
        e = mi355::launch_prefill_f32(a, stream);
    } else {
        return ATTN_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_prefill_fp8(const void *q, const void *k, const void *v, const float *q_scales,
                               const float *k_scales, const float *v_scales, void *o, float *lse,
                               int B, int T, int h_q, int h_kv, int d_h, int causal, int window,
                               float scale, const float *sinks, hipStream_t stream) {
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(o) || bad_ptr(q_scales) ||
        bad_ptr(k_scales) || bad_ptr(v_scales))
        return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0 || h_q <= 0 || h_kv <= 0 || d_h <= 0) return ATTN_ERR_INVALID_ARG;
    if (h_q % h_kv != 0) return ATTN_ERR_INVALID_ARG;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_INVALID_ARG;
    if (d_h != 128) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * h_q * T * d_h >= (1LL << 40)) return ATTN_ERR_UNSUPPORTED;
    mi355::PrefillFp8Args a{q, k, v, q_scales, k_scales, v_scales, o, lse, B, T, h_q, h_kv,
                            causal ? 1 : 0, window, scale, sinks};
    return mi355::launch_prefill_fp8_d128(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_prefill_backward_workspace_size(int B, int T, int h_q) {
    if (B <= 0 || T <= 0 || h_q <= 0) return 0;
    const long long tpad = ((long long)T + 63) / 64 * 64;
    return align_up((size_t)((long long)B * h_q * tpad) * 2 * sizeof(float), 256);
}

attn_status_t attn_prefill_backward(const void *q, const void *k, const void *v, const void *o,
                                    const void *dout, const float *lse, void *dq, void *dk,
                                    void *dv, int B, int T, int h_q, int h_kv, int d_h,
                                    attn_dtype_t dtype, int causal, int window, float scale,
                                    const float *sinks, float *dsinks, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(o) || bad_ptr(dout) || bad_ptr(lse) ||
        bad_ptr(dq) || bad_ptr(dk) || bad_ptr(dv))
        return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0 || h_q <= 0 || h_kv <= 0 || d_h <= 0) return ATTN_ERR_INVALID_ARG;
    if (h_q % h_kv != 0) return ATTN_ERR_INVALID_ARG;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_INVALID_ARG;
    if (dsinks && !sinks) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_BF16 || d_h != 128) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * h_q * (T + 63) * d_h >= (1LL << 40)) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * h_q > 65535) return ATTN_ERR_UNSUPPORTED;
    const size_t need = attn_prefill_backward_workspace_size(B, T, h_q);
    if (bad_ptr(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const int tpad = (T + 63) / 64 * 64;
    mi355::PrefillBwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, T, h_q, h_kv, d_h,
                            causal ? 1 : 0, window, scale, static_cast<float *>(workspace), tpad,
                            sinks, dsinks};
    return mi355::launch_prefill_bwd_bf16_d128(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

static int resolve_decode_split(int split_tokens, int B, int S_max, int h_q, int h_kv,
                                bool fp8 = false) {
    if (split_tokens == 0) return default_decode_split(B, S_max, h_kv, h_q / h_kv, device_cu_count(), fp8);
    return split_tokens;
}

size_t attn_decode_workspace_size(int B, int S_max, int h_q, int h_kv, int d_h, int split_tokens) {
    if (B <= 0 || S_max <= 0 || h_q <= 0 || h_kv <= 0 || d_h <= 0 || h_q % h_kv) return 0;
    if (split_tokens < 0 || split_tokens % 64) return 0;
    const int split = resolve_decode_split(split_tokens, B, S_max, h_q, h_kv);
    const long long ns = (S_max + split - 1) / split;
    return split_ws_bytes((long long)B * h_q, ns, d_h) + align_up((size_t)(B + 1) * sizeof(int32_t), 256);
}

// The argument checks every GQA decode entry point shares (host only: no
// HIP call is made before they pass).
static attn_status_t decode_check(const void *q, const void *k, const void *v, const void *o,
                                  const int32_t *seq_lens, int B, int S_max, int h_q, int h_kv,
                                  int d_h, int window, float scale, int split_tokens) {
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(o) || bad_ptr(seq_lens))
        return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || S_max <= 0 || h_q <= 0 || h_kv <= 0 || d_h <= 0) return ATTN_ERR_INVALID_ARG;
    if (h_q % h_kv != 0 || window < 0 || !isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_INVALID_ARG;
    if (split_tokens < 0 || split_tokens % 64) return ATTN_ERR_INVALID_ARG;
    if (d_h != 128) return ATTN_ERR_UNSUPPORTED;
    if (B > 65535 || h_kv * ((h_q / h_kv + 15) / 16) > 65535) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

// Shared by the GQA decode entry points (contiguous / paged, bf16 / FP8,
// caller workspace or static scratch): everything after the layout-specific
// checks.
static attn_status_t decode_launch(const void *q, const void *k, const void *v, const float *k_scales,
                                   const float *v_scales, void *o, float *lse,
                                   const int32_t *seq_lens, const int32_t *block_table, int B,
                                   int S_max, int max_blocks, int page_size, int num_pages, int h_q,
                                   int h_kv, int d_h, int window, float scale, const float *sinks,
                                   int split_tokens, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    const attn_status_t checked = decode_check(q, k, v, o, seq_lens, B, S_max, h_q, h_kv, d_h,
                                               window, scale, split_tokens);
    if (checked != ATTN_OK) return checked;
    const int split = resolve_decode_split(split_tokens, B, S_max, h_q, h_kv, k_scales != nullptr);
    const int ns = (S_max + split - 1) / split;
    const size_t need = attn_decode_workspace_size(B, S_max, h_q, h_kv, d_h, split_tokens);
    if (bad_ptr(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    float *ws_o = static_cast<float *>(workspace);
    char *ws_end = static_cast<char *>(workspace) + align_up((size_t)B * h_q * ns * d_h * sizeof(float), 256);
    float *ws_lse = reinterpret_cast<float *>(ws_end);
    int32_t *plan = reinterpret_cast<int32_t *>(ws_end + align_up((size_t)B * h_q * ns * sizeof(float), 256));
    mi355::DecodeArgs a{q, k, v, o, lse, seq_lens, B, S_max, h_q, h_kv, d_h,
                        window, scale, split, ns, ws_o, ws_lse, plan, device_cu_count(),
                        block_table, max_blocks, page_size, num_pages, sinks, k_scales, v_scales};
    return mi355::launch_decode_bf16_d128(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_decode(const void *q, const void *k_cache, const void *v_cache, void *o,
                          float *lse, const int32_t *seq_lens, int B, int S_max, int h_q,
                          int h_kv, int d_h, int window, float scale, const float *sinks,
                          int split_tokens, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return decode_launch(q, k_cache, v_cache, nullptr, nullptr, o, lse, seq_lens, nullptr, B, S_max,
                         0, 0, 0, h_q, h_kv, d_h, window, scale, sinks, split_tokens, workspace,
                         workspace_bytes, stream);
}

attn_status_t attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                              const float *k_scales, const float *v_scales, void *o, float *lse,
                              const int32_t *seq_lens, int B, int S_max, int h_q, int h_kv,
                              int d_h, int window, float scale, const float *sinks,
                              int split_tokens, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    if (bad_ptr(k_scales) || bad_ptr(v_scales)) return ATTN_ERR_INVALID_ARG;
    return decode_launch(q, k_cache, v_cache, k_scales, v_scales, o, lse, seq_lens, nullptr, B,
                         S_max, 0, 0, 0, h_q, h_kv, d_h, window, scale, sinks, split_tokens,
                         workspace, workspace_bytes, stream);
}

size_t attn_decode_paged_workspace_size(int B, int max_blocks, int page_size, int h_q, int h_kv,
                                        int d_h, int split_tokens) {
    if (max_blocks <= 0 || page_size <= 0 || (long long)max_blocks * page_size > 0x7fffffffLL) return 0;
    return attn_decode_workspace_size(B, max_blocks * page_size, h_q, h_kv, d_h, split_tokens);
}

static bool bad_pages(const int32_t *block_table, int max_blocks, int page_size, int num_pages) {
    return bad_ptr(block_table) || max_blocks <= 0 || page_size <= 0 || num_pages <= 0 ||
           (long long)max_blocks * page_size > 0x7fffffffLL;
}

static attn_status_t decode_paged_launch(const void *q, const void *k_pages, const void *v_pages,
                                         const float *k_scales, const float *v_scales, void *o,
                                         float *lse, const int32_t *seq_lens,
                                         const int32_t *block_table, int B, int max_blocks,
                                         int page_size, int num_pages, int h_q, int h_kv, int d_h,
                                         int window, float scale, const float *sinks,
                                         int split_tokens, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    if (bad_pages(block_table, max_blocks, page_size, num_pages)) return ATTN_ERR_INVALID_ARG;
    if (B <= 0) return ATTN_ERR_INVALID_ARG;
    if (page_size % 32) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * max_blocks > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
    return decode_launch(q, k_pages, v_pages, k_scales, v_scales, o, lse, seq_lens, block_table, B,
                         max_blocks * page_size, max_blocks, page_size, num_pages, h_q, h_kv, d_h,
                         window, scale, sinks, split_tokens, workspace, workspace_bytes, stream);
}

attn_status_t attn_decode_paged(const void *q, const void *k_pages, const void *v_pages, void *o,
                                float *lse, const int32_t *seq_lens, const int32_t *block_table,
                                int B, int max_blocks, int page_size, int num_pages, int h_q,
                                int h_kv, int d_h, int window, float scale, const float *sinks,
                                int split_tokens, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    return decode_paged_launch(q, k_pages, v_pages, nullptr, nullptr, o, lse, seq_lens, block_table,
                               B, max_blocks, page_size, num_pages, h_q, h_kv, d_h, window, scale,
                               sinks, split_tokens, workspace, workspace_bytes, stream);
}

attn_status_t attn_decode_paged_fp8(const void *q, const void *k_pages, const void *v_pages,
                                    const float *k_scales, const float *v_scales, void *o,
                                    float *lse, const int32_t *seq_lens,
                                    const int32_t *block_table, int B, int max_blocks,
                                    int page_size, int num_pages, int h_q, int h_kv, int d_h,
                                    int window, float scale, const float *sinks, int split_tokens,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (bad_ptr(k_scales) || bad_ptr(v_scales)) return ATTN_ERR_INVALID_ARG;
    return decode_paged_launch(q, k_pages, v_pages, k_scales, v_scales, o, lse, seq_lens,
                               block_table, B, max_blocks, page_size, num_pages, h_q, h_kv, d_h,
                               window, scale, sinks, split_tokens, workspace, workspace_bytes,
                               stream);
}

attn_status_t attn_rope_qk(void *q, void *k, const int32_t *positions, int B, int T, int h_q,
                           int h_k, int row_q, int row_k, int rope_offset, int rope_dim,
                           float base, attn_dtype_t dtype, hipStream_t stream) {
    if (bad_ptr(q) || (h_k > 0 && bad_ptr(k))) return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0 || h_q <= 0 || h_k < 0 || row_q <= 0 || (h_k > 0 && row_k <= 0))
        return ATTN_ERR_INVALID_ARG;
    if (rope_dim <= 0 || rope_dim % 2 || rope_offset < 0 || rope_offset % 2 ||
        rope_offset + rope_dim > row_q || (h_k > 0 && rope_offset + rope_dim > row_k))
        return ATTN_ERR_INVALID_ARG;
    if (row_q % 2 || (h_k > 0 && row_k % 2)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(base) || !(base > 0.f)) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * h_q * T * row_q >= (1LL << 40) || (long long)B * h_k * T * row_k >= (1LL << 40))
        return ATTN_ERR_UNSUPPORTED;
    mi355::RopeArgs a{q, h_k > 0 ? k : nullptr, positions, B, T, h_q, h_k, row_q, row_k,
                      rope_offset, rope_dim, base, dtype == ATTN_BF16};
    return mi355::launch_rope_qk(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_quantize_kv_fp8(const void *x, void *codes, float *scales, int B, int h_kv,
                                   int S, int d_h, hipStream_t stream) {
    if (bad_ptr(x) || bad_ptr(codes) || bad_ptr(scales)) return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || h_kv <= 0 || S <= 0 || d_h <= 0) return ATTN_ERR_INVALID_ARG;
    if (d_h % 8) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * h_kv * S * d_h >= (1LL << 40)) return ATTN_ERR_UNSUPPORTED;
    return mi355::launch_quantize_kv_fp8(x, codes, scales, (long long)B * h_kv, S, d_h, stream) ==
                   hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t mla_decode_workspace_size(int B, int S_max, int h_q, int d_c, int d_r, int split_tokens) {
    if (B <= 0 || S_max <= 0 || h_q <= 0 || d_c <= 0 || d_r < 0) return 0;
    if (split_tokens < 0 || split_tokens % 64) return 0;
    const int split = split_tokens ? split_tokens : default_mla_split(B, S_max, h_q);
    const long long ns = (S_max + split - 1) / split;
    return mla_ws_bytes((long long)B * h_q, ns, d_c);
}

attn_status_t mla_decode(const void *q, const void *kv_cache, void *o, float *lse,
                         const int32_t *seq_lens, int B, int S_max, int h_q, int d_c, int d_r,
                         float scale, const float *sinks, int split_tokens, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    if (bad_ptr(q) || bad_ptr(kv_cache) || bad_ptr(o) || bad_ptr(seq_lens)) return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || S_max <= 0 || h_q <= 0 || d_c <= 0 || d_r < 0) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f) || split_tokens < 0 || split_tokens % 64)
        return ATTN_ERR_INVALID_ARG;
    if (d_c != 512 || d_r != 64 || h_q % 16 != 0) return ATTN_ERR_UNSUPPORTED;
    if (B > 65535) return ATTN_ERR_UNSUPPORTED;
    const int split = split_tokens ? split_tokens : default_mla_split(B, S_max, h_q);
    const int ns = (S_max + split - 1) / split;
    const size_t need = mla_decode_workspace_size(B, S_max, h_q, d_c, d_r, split_tokens);
    if (bad_ptr(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    __bf16 *ws_o = static_cast<__bf16 *>(workspace);
    float *ws_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                              align_up((size_t)B * h_q * ns * d_c * sizeof(uint16_t), 256));
    mi355::MlaArgs a{q, kv_cache, o, lse, seq_lens, B, S_max, h_q, d_c, d_r, scale, split, ns,
                     ws_o, ws_lse, nullptr, 0, 0, 0, sinks};
    return mi355::launch_mla_decode_bf16(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t mla_decode_fp8_workspace_size(int B, int S_max, int h_q, int d_c, int d_r, int split_tokens) {
    const size_t base = mla_decode_workspace_size(B, S_max, h_q, d_c, d_r, split_tokens);
    if (base == 0) return 0;
    const size_t rows = (size_t)B * h_q;
    return base + align_up(rows * (size_t)(d_c + d_r), 256) + align_up(rows * sizeof(float), 256);
}

attn_status_t mla_decode_fp8(const void *q, const void *kv_codes, const float *kv_scales, void *o,
                             float *lse, const int32_t *seq_lens, int B, int S_max, int h_q,
                             int d_c, int d_r, float scale, const float *sinks, int split_tokens,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (bad_ptr(q) || bad_ptr(kv_codes) || bad_ptr(kv_scales) || bad_ptr(o) || bad_ptr(seq_lens))
        return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || S_max <= 0 || h_q <= 0 || d_c <= 0 || d_r < 0) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f) || split_tokens < 0 || split_tokens % 64)
        return ATTN_ERR_INVALID_ARG;
    if (d_c != 512 || d_r != 64) return ATTN_ERR_UNSUPPORTED;
    if (B > 65535 || (long long)B * h_q * (d_c + d_r) >= (1LL << 40)) return ATTN_ERR_UNSUPPORTED;
    const int split = split_tokens ? split_tokens : default_mla_split(B, S_max, h_q);
    const int ns = (S_max + split - 1) / split;
    const size_t need = mla_decode_fp8_workspace_size(B, S_max, h_q, d_c, d_r, split_tokens);
    if (bad_ptr(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    char *w = static_cast<char *>(workspace);
    const size_t rows = (size_t)B * h_q;
    __bf16 *ws_o = reinterpret_cast<__bf16 *>(w);
    w += align_up(rows * ns * d_c * sizeof(uint16_t), 256);
    float *ws_lse = reinterpret_cast<float *>(w);
    w += align_up(rows * ns * sizeof(float), 256);
    void *ws_q8 = w;
    w += align_up(rows * (size_t)(d_c + d_r), 256);
    float *ws_qs = reinterpret_cast<float *>(w);
    mi355::MlaFp8Args a{q, kv_codes, kv_scales, o, lse, seq_lens, B, S_max, h_q, scale, split, ns,
                        ws_o, ws_lse, ws_q8, ws_qs, sinks};
    return mi355::launch_mla_decode_fp8(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t mla_decode_paged_workspace_size(int B, int max_blocks, int page_size, int h_q, int d_c,
                                       int d_r, int split_tokens) {
    if (max_blocks <= 0 || page_size <= 0 || (long long)max_blocks * page_size > 0x7fffffffLL) return 0;
    return mla_decode_workspace_size(B, max_blocks * page_size, h_q, d_c, d_r, split_tokens);
}

attn_status_t mla_decode_paged(const void *q, const void *kv_pages, void *o, float *lse,
                               const int32_t *seq_lens, const int32_t *block_table, int B,
                               int max_blocks, int page_size, int num_pages, int h_q, int d_c,
                               int d_r, float scale, const float *sinks, int split_tokens,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (bad_ptr(q) || bad_ptr(kv_pages) || bad_ptr(o) || bad_ptr(seq_lens)) return ATTN_ERR_INVALID_ARG;
    if (bad_pages(block_table, max_blocks, page_size, num_pages)) return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || h_q <= 0 || d_c <= 0 || d_r < 0) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f) || split_tokens < 0 || split_tokens % 64)
        return ATTN_ERR_INVALID_ARG;
    if (page_size % 32) return ATTN_ERR_UNSUPPORTED;
    if (d_c != 512 || d_r != 64 || h_q % 16 != 0) return ATTN_ERR_UNSUPPORTED;
    if (B > 65535 || (long long)B * max_blocks > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
    const int S_max = max_blocks * page_size;
    const int split = split_tokens ? split_tokens : default_mla_split(B, S_max, h_q);
    const int ns = (S_max + split - 1) / split;
    const size_t need = mla_decode_workspace_size(B, S_max, h_q, d_c, d_r, split_tokens);
    if (bad_ptr(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    __bf16 *ws_o = static_cast<__bf16 *>(workspace);
    float *ws_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                              align_up((size_t)B * h_q * ns * d_c * sizeof(uint16_t), 256));
    mi355::MlaArgs a{q, kv_pages, o, lse, seq_lens, B, S_max, h_q, d_c, d_r, scale, split, ns,
                     ws_o, ws_lse, block_table, max_blocks, page_size, num_pages, sinks};
    return mi355::launch_mla_decode_bf16(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// attn_decode_noalloc: attn_decode with its workspace in a static device
// array instead of caller memory, for callers that cannot allocate.
//
// `scratch` is a file-scope device array; every GPU the library runs on
// holds its own copy from module load until the process ends.  In host code
// its name is only a host-side stand-in, so the device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever handed to kernels.  The decode writes the whole plan
// and every partial it later reads within the same call (stream-ordered), so
// nothing in the array has to start at zero and the contents left by a
// previous call are never read.  Calls that overlap on one GPU share the
// array and race; the caller orders them.
namespace {

__device__ __align__(256) unsigned char scratch[MI355ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices] = {};

attn_status_t device_scratch(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return ATTN_ERR_HIP;
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" attn_status_t attn_decode_noalloc(const void *q, const void *k_cache,
                                             const void *v_cache, void *o, float *lse,
                                             const int32_t *seq_lens, int B, int S_max, int h_q,
                                             int h_kv, int d_h, int window, float scale,
                                             const float *sinks, int split_tokens,
                                             hipStream_t stream) {
    const attn_status_t checked = decode_check(q, k_cache, v_cache, o, seq_lens, B, S_max, h_q,
                                               h_kv, d_h, window, scale, split_tokens);
    if (checked != ATTN_OK) return checked;
    const size_t need = attn_decode_workspace_size(B, S_max, h_q, h_kv, d_h, split_tokens);
    if (need == 0 || need > (size_t)MI355ATTN_DECODE_NOALLOC_SCRATCH_BYTES)
        return ATTN_ERR_WORKSPACE;                  // does not fit: nothing is launched
    void *ws = nullptr;
    const attn_status_t st = device_scratch(&ws);
    if (st != ATTN_OK) return st;
    return decode_launch(q, k_cache, v_cache, nullptr, nullptr, o, lse, seq_lens, nullptr, B, S_max,
                         0, 0, 0, h_q, h_kv, d_h, window, scale, sinks, split_tokens, ws,
                         (size_t)MI355ATTN_DECODE_NOALLOC_SCRATCH_BYTES, stream);
}
